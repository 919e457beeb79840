"""Seeded synthetic inputs for the FP8 block-scaled GEMM workloads.

This module only draws random numbers and lays out group structure; it does
no quantization and no GEMM arithmetic, so the GPU path and the CPU oracle
can both start from it without sharing any of the method's arithmetic.

Recipe (one CPU ``torch.Generator`` per case, seeded with the case's seed):
group sizes or masks are drawn first (``torch.randint``), then the fp32
activation matrix ``x_a`` (``torch.randn``), then the fp32 weight matrix
``x_b`` (``torch.randn``).  The fp32 matrices are quantized afterwards by the
caller: per token (1x128) for A and per 128x128 block for B, with fp32
scales or, for the cases marked ``scales="e8m0"``, power-of-two scales.

The workloads follow DeepSeek-style projection and MoE expert shapes; no
dataset is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass
class Case:
    """One synthetic workload.

    form: "dense", "dense_acc", "contiguous" or "masked".
    x_a:  fp32 activations, [M][K] (dense), [M_sum][K] (contiguous) or
          [G][M_max][K] (masked).
    x_b:  fp32 weights, [N][K] (dense) or [G][N][K] (grouped).
    layout: int32 [M_sum] group id per row, -1 on padding (contiguous).
    masked_m: int32 [G] valid rows per group (masked).
    x_c:  fp32 addend [M][N] (dense_acc).
    scales: "fp32" (amax/448) or "e8m0" (power-of-two exponent bytes).
    """
    name: str
    form: str
    M: int
    N: int
    K: int
    G: int
    x_a: torch.Tensor
    x_b: torch.Tensor
    layout: torch.Tensor | None = None
    masked_m: torch.Tensor | None = None
    group_rows: list = field(default_factory=list)
    x_c: torch.Tensor | None = None
    scales: str = "fp32"

    @property
    def valid_rows(self) -> int:
        if self.form in ("dense", "dense_acc"):
            return self.M
        if self.form == "contiguous":
            return int((self.layout >= 0).sum())
        return int(self.masked_m.clamp(0, self.M).sum())

    @property
    def active_groups(self) -> int:
        if self.form in ("dense", "dense_acc"):
            return 1
        if self.form == "contiguous":
            return int(torch.unique(self.layout[self.layout >= 0]).numel())
        return int((self.masked_m.clamp(0, self.M) > 0).sum())


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def dense_case(M: int, N: int, K: int, seed: int, name: str = "dense") -> Case:
    g = _gen(seed)
    x_a = torch.randn(M, K, generator=g, dtype=torch.float32)
    x_b = torch.randn(N, K, generator=g, dtype=torch.float32)
    return Case(name, "dense", M, N, K, 1, x_a, x_b)


def dense_acc_case(M: int, N: int, K: int, seed: int, name: str = "dense_acc") -> Case:
    """Dense operands plus an fp32 addend C of the product's magnitude
    (standard normal times sqrt(K))."""
    g = _gen(seed)
    x_a = torch.randn(M, K, generator=g, dtype=torch.float32)
    x_b = torch.randn(N, K, generator=g, dtype=torch.float32)
    x_c = torch.randn(M, N, generator=g, dtype=torch.float32) * float(K) ** 0.5
    return Case(name, "dense_acc", M, N, K, 1, x_a, x_b, x_c=x_c)


def contiguous_case(G: int, N: int, K: int, seed: int, m_lo: int = 3072, m_hi: int = 5120,
                    align: int = 128, name: str = "contiguous", sizes=None) -> Case:
    """Group g gets m_g rows (uniform in [m_lo, m_hi] unless ``sizes`` is
    given), padded up to a multiple of ``align``; padding rows carry id -1
    and random activations like every other row."""
    g = _gen(seed)
    if sizes is None:
        sizes = torch.randint(m_lo, m_hi + 1, (G,), generator=g, dtype=torch.int64).tolist()
    sizes = [int(s) for s in sizes]
    padded = [((s + align - 1) // align) * align for s in sizes]
    M_sum = sum(padded)
    layout = torch.full((M_sum,), -1, dtype=torch.int32)
    off = 0
    for gi, (s, p) in enumerate(zip(sizes, padded)):
        layout[off:off + s] = gi
        off += p
    x_a = torch.randn(M_sum, K, generator=g, dtype=torch.float32)
    x_b = torch.randn(G, N, K, generator=g, dtype=torch.float32)
    return Case(name, "contiguous", M_sum, N, K, G, x_a, x_b, layout=layout, group_rows=sizes)


def masked_case(G: int, M_max: int, N: int, K: int, seed: int, name: str = "masked",
                masked=None) -> Case:
    """Group g has masked_m[g] valid rows, uniform in [0, M_max] unless
    ``masked`` is given."""
    g = _gen(seed)
    if masked is None:
        mm = torch.randint(0, M_max + 1, (G,), generator=g, dtype=torch.int64).to(torch.int32)
    else:
        mm = torch.tensor(list(masked), dtype=torch.int32)
    x_a = torch.randn(G, M_max, K, generator=g, dtype=torch.float32)
    x_b = torch.randn(G, N, K, generator=g, dtype=torch.float32)
    return Case(name, "masked", M_max, N, K, G, x_a, x_b, masked_m=mm, group_rows=mm.tolist())


# The named workloads: projection and MoE expert shapes of a DeepSeek-style
# model, each with its fixed seed.
WORKLOADS = {
    "dense_128x512x512": lambda: dense_case(128, 512, 512, 1, "dense_128x512x512"),
    "dense_4096x7168x2048": lambda: dense_case(4096, 7168, 2048, 2, "dense_4096x7168x2048"),
    "dense_64x7168x2048": lambda: dense_case(64, 7168, 2048, 21, "dense_64x7168x2048"),
    "dense_128x7168x2048": lambda: dense_case(128, 7168, 2048, 22, "dense_128x7168x2048"),
    "dense_4096x24576x1536": lambda: dense_case(4096, 24576, 1536, 3, "dense_4096x24576x1536"),
    "dense_4096x2112x7168": lambda: dense_case(4096, 2112, 7168, 31, "dense_4096x2112x7168"),
    "dense_acc_4096x7168x2048": lambda: dense_acc_case(4096, 7168, 2048, 23,
                                                       "dense_acc_4096x7168x2048"),
    "contiguous_8x4096x7168": lambda: contiguous_case(8, 4096, 7168, 4, name="contiguous_8x4096x7168"),
    "masked_16x256x4096x7168": lambda: masked_case(16, 256, 4096, 7168, 5, name="masked_16x256x4096x7168"),
    "masked_16x256x7168x2048": lambda: masked_case(16, 256, 7168, 2048, 51, name="masked_16x256x7168x2048"),
}


def _e8m0(case: Case) -> Case:
    case.scales = "e8m0"
    return case


WORKLOADS.update({
    "dense_e8m0_4096x7168x2048": lambda: _e8m0(dense_case(4096, 7168, 2048, 2,
                                                          "dense_e8m0_4096x7168x2048")),
    "dense_e8m0_4096x24576x1536": lambda: _e8m0(dense_case(4096, 24576, 1536, 3,
                                                           "dense_e8m0_4096x24576x1536")),
    "contiguous_e8m0_8x4096x7168": lambda: _e8m0(contiguous_case(
        8, 4096, 7168, 4, name="contiguous_e8m0_8x4096x7168")),
    "masked_e8m0_16x256x4096x7168": lambda: _e8m0(masked_case(
        16, 256, 4096, 7168, 5, name="masked_e8m0_16x256x4096x7168")),
})


def workload(name: str) -> Case:
    return WORKLOADS[name]()


def e4m3_pattern_matrix(rows: int, K: int, seed: int) -> np.ndarray:
    """Random e4m3 byte codes (never the NaN codes 0x7F/0xFF), for tests that
    feed codes straight to a GEMM without quantizing."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] ^= 0x01
    return q
