"""Helpers for the GPU parity tests: move arrays to the device, run the C-ABI
entry points through the binding, and compare with the oracle to the
tolerance the workload fixes:

    |gpu - oracle| <= 2 * ulp_bf16(|oracle|) + 1e-3 * RMS(oracle)   per element

with RMS over every routed element of the call, and bit-exact equality of
every element the call must not write (they keep the 0xFFFF pre-fill)."""
from __future__ import annotations

import numpy as np
import torch

SENTINEL = -1  # int16 view of 0xFFFF (a NaN pattern no result produces)


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, np.exp2(e - 7), 2.0 ** -133)


def assert_close_bf16(got_bits: np.ndarray, ref_bits: np.ndarray, what: str = "",
                      rms: float | None = None):
    """Elementwise tolerance check on routed elements (same shapes)."""
    g = bf16_to_f64(got_bits)
    r = bf16_to_f64(ref_bits)
    assert np.isfinite(r).all(), f"{what}: oracle produced non-finite values"
    if rms is None:
        rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    tol = 2 * ulp_bf16(r) + 1e-3 * rms
    err = np.abs(g - r)
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        details = ", ".join(f"{tuple(i)}: gpu {g[tuple(i)]!r} oracle {r[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance "
                             f"(rms {rms:.4g}); first: {details}")
    return float(err.max()) if err.size else 0.0


def same_codes(a: np.ndarray, b: np.ndarray) -> bool:
    """e4m3 codes equal, with +0 (0x00) and -0 (0x80) counted as one."""
    za = (a & 0x7F) == 0
    zb = (b & 0x7F) == 0
    return bool(np.array_equal(za, zb) and np.array_equal(a[~za], b[~zb]))


def check_call(got_bits: np.ndarray, ref_bits: np.ndarray, routed: np.ndarray, what: str,
               chunk_rows: int = 2048) -> float:
    """Whole-call comparison of D viewed as [rows][N]: every row in ``routed``
    against the oracle (RMS over all routed elements of the call, then the
    per-element bound), every other row bit-exact at the 0xFFFF pre-fill.
    Works in row chunks so full-size workloads stay within a few GB of host
    memory."""
    assert got_bits.shape == ref_bits.shape, (got_bits.shape, ref_bits.shape)
    routed = np.asarray(routed, dtype=np.int64)
    unrouted = np.ones(got_bits.shape[0], bool)
    unrouted[routed] = False
    assert (got_bits[unrouted] == 0xFFFF).all(), f"{what}: an unrouted row of D was written"
    if routed.size == 0:
        return 0.0
    ss = 0.0
    for c in range(0, routed.size, chunk_rows):
        r = bf16_to_f64(ref_bits[routed[c:c + chunk_rows]])
        assert np.isfinite(r).all(), f"{what}: oracle produced non-finite values"
        ss += float(np.sum(r * r))
    rms = float(np.sqrt(ss / (routed.size * got_bits.shape[1])))
    worst = 0.0
    for c in range(0, routed.size, chunk_rows):
        rows = routed[c:c + chunk_rows]
        worst = max(worst, assert_close_bf16(got_bits[rows], ref_bits[rows], what, rms=rms))
    return worst
