"""Pins for the oracle's power-of-two (E8M0) scale recipe and its GEMM.

The exponent rule is checked against values worked out by hand from its
statement (smallest e >= -127 with amax <= 448 * 2^e); codes against torch's
float8_e4m3fn cast of x * 2^-e; the GEMM against an fp64 torch reference,
which is exact when every scale is a power of two, and against a
brute-force sum in exact rationals."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests.bf16_ref import bf16_bits_of_fraction
from tests.test_oracle_gemm import _per_kb_reference, dec
from tests.test_oracle_quantize import _same_codes

F32_MAX = float(np.finfo(np.float32).max)


def _up(v):
    return float(np.nextafter(np.float32(v), np.float32(np.inf)))


# (amax, byte) pairs, each worked out from the rule by hand
HAND = [
    (448.0, 127),           # 448 <= 448 * 2^0, 448 > 448 * 2^-1 = 224: e = 0
    (_up(448.0), 128),      # just above 448: e = 1
    (224.0, 126),           # 224 <= 448 * 2^-1: e = -1
    (_up(224.0), 127),      # just above 224: e = 0
    (1.0, 119),             # 448 * 2^-9 = 0.875 < 1 <= 1.75 = 448 * 2^-8: e = -8
    (1.75, 119),            # 1.75 = 448 * 2^-8 exactly: e = -8
    (_up(1.75), 120),       # e = -7
    (0.0, 0),               # every e satisfies the bound: the least, -127
    (1e-40, 0),             # below 448 * 2^-127 ~ 2.6e-36: clamped to -127
    (448.0 * 2.0 ** -127, 0),          # exactly the bound at -127
    (_up(448.0 * 2.0 ** -127), 1),     # e = -126
    (F32_MAX, 247),         # FLT_MAX ~ 1.99 * 2^127 > 1.75 * 2^127 = 448 * 2^119: e = 120
    (3.0, 120),             # 1.75 < 3 <= 3.5 = 448 * 2^-7: e = -7
]


def test_e8m0_decode_pins(orc):
    assert orc.e8m0_value(127) == 1.0
    assert orc.e8m0_value(128) == 2.0
    assert orc.e8m0_value(126) == 0.5
    assert orc.e8m0_value(0) == 2.0 ** -127
    assert orc.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(orc.e8m0_value(255))
    t = orc.e8m0_decode(np.arange(255, dtype=np.uint8))
    assert t.dtype == np.float32
    assert np.array_equal(t.astype(np.float64), np.exp2(np.arange(255) - 127.0))


@pytest.mark.parametrize("amax,byte", HAND)
def test_exponent_hand_table(orc, amax, byte):
    assert orc.e8m0_exponent(amax) + 127 == byte
    # through both quantizers, with the maximum on a negative element
    x = np.zeros((2, 256), np.float32)
    x[1, 130] = -np.float32(amax)
    x[1, 131] = np.float32(amax) / 3
    _, s = orc.quantize_per_token_e8m0(x)
    assert s[1, 1] == byte and s[1, 0] == 0 and s[0, 0] == 0 and s.shape == (2, 4)
    _, sb = orc.quantize_per_block_e8m0(x)
    assert sb[0, 1] == byte and sb.shape == (1, 4)


def _blocks_x(M, K, seed):
    rng = np.random.default_rng(seed)
    # block magnitudes spread over 2^-120 .. 2^100
    mag = np.exp2(rng.integers(-120, 100, (M, K // 128))).repeat(128, axis=1)
    return (rng.standard_normal((M, K)) * mag).astype(np.float32)


@pytest.mark.parametrize("M,K", [(3, 128), (33, 640), (64, 1024)])
def test_per_token_codes_against_torch_cast(orc, M, K):
    x = _blocks_x(M, K, M + K)
    q, s = orc.quantize_per_token_e8m0(x)
    KB = K // 128
    assert s.shape == (M, (KB + 3) // 4 * 4) and (s[:, KB:] == 0).all()
    e = s[:, :KB].astype(np.int64) - 127
    inv = np.exp2(-e).repeat(128, axis=1).astype(np.float32)       # exact powers of two
    ref = (torch.from_numpy(x) * torch.from_numpy(inv)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert _same_codes(q, ref)


@pytest.mark.parametrize("N,K", [(128, 128), (200, 384), (300, 512)])
def test_per_block_codes_against_torch_cast(orc, N, K):
    x = _blocks_x(N, K, N * 3 + K)
    q, s = orc.quantize_per_block_e8m0(x)
    NB, KB = (N + 127) // 128, K // 128
    assert s.shape == (NB, (KB + 3) // 4 * 4)
    e = np.repeat(s[:, :KB].astype(np.int64) - 127, 128, axis=0)[:N]
    inv = np.exp2(-e).repeat(128, axis=1).astype(np.float32)
    ref = (torch.from_numpy(x) * torch.from_numpy(inv)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert _same_codes(q, ref)


def test_exponent_invariants(orc):
    """For every block above the clamp, amax * 2^-e lies in (224, 448]: the
    scale is the least power of two that keeps the block in range; clamped
    blocks stay within 448 as well."""
    x = _blocks_x(64, 1024, 5)
    _, s = orc.quantize_per_token_e8m0(x)
    e = s[:, :8].astype(np.int64) - 127
    amax = np.abs(x).reshape(64, 8, 128).max(axis=2).astype(np.float64)
    r = amax * np.exp2(-e.astype(np.float64))
    free = e > -127
    assert free.sum() > 400 and (~free).sum() > 0
    assert ((r[free] > 224.0) & (r[free] <= 448.0)).all()
    assert (r[~free] <= 448.0).all()
    # and the round trip is within half an e4m3 step of the block's grid
    q, _ = orc.quantize_per_token_e8m0(x)
    back = dec(q).reshape(64, 8, 128) * np.exp2(e.astype(np.float64))[:, :, None]
    err = np.abs(back - x.reshape(64, 8, 128).astype(np.float64))
    # e4m3 spacing at magnitude |v| * 2^-e is at most 2^(floor(log2)-3)
    vs = np.abs(x.reshape(64, 8, 128).astype(np.float64)) * np.exp2(-e.astype(np.float64))[:, :, None]
    step = np.exp2(np.floor(np.log2(np.maximum(vs, 2.0 ** -6))) - 3)
    assert (err <= 0.5 * step * np.exp2(e.astype(np.float64))[:, :, None] * (1 + 1e-12)).all()


def _rand_e8m0_case(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = rng.integers(0, 256, (M, K), dtype=np.uint8)
    B = rng.integers(0, 256, (N, K), dtype=np.uint8)
    A[(A & 0x7F) == 0x7F] = 0x3F                                  # no NaN codes
    B[(B & 0x7F) == 0x7F] = 0x3F
    KB, KBp, NB = K // 128, (K // 128 + 3) // 4 * 4, (N + 127) // 128
    sa = np.zeros((M, KBp), np.uint8); sb = np.zeros((NB, KBp), np.uint8)
    sa[:, :KB] = rng.integers(117, 138, (M, KB))
    sb[:, :KB] = rng.integers(117, 138, (NB, KB))
    return A, sa, B, sb


@pytest.mark.parametrize("M,N,K", [(9, 136, 256), (40, 264, 640)])
def test_gemm_e8m0_exact_against_torch(orc, M, N, K):
    """Power-of-two scales keep every term exact in fp64, so torch's
    per-block fp64 reference rounds to the same bf16 bits; a wrong exponent
    bias, a wrong sb row or a transposed scale fails."""
    A, sa, B, sb = _rand_e8m0_case(M, N, K, M * N + K)
    KB = K // 128
    sa_f = np.exp2(sa[:, :KB].astype(np.float64) - 127).astype(np.float32)
    sb_f = np.exp2(sb[:, :KB].astype(np.float64) - 127).astype(np.float32)
    V = _per_kb_reference(A, sa_f, B, sb_f)
    ref = np.vectorize(orc.bf16_from_double, otypes=[np.uint16])(V)
    assert np.array_equal(orc.gemm_nt_e8m0(A, sa, B, sb), ref)


def test_gemm_e8m0_brute_force_rational(orc):
    """A few elements as exact rationals straight from the definition."""
    A, sa, B, sb = _rand_e8m0_case(3, 130, 384, 77)
    D = orc.gemm_nt_e8m0(A, sa, B, sb)
    a, b = dec(A), dec(B)
    for m, n in [(0, 0), (1, 129), (2, 64)]:
        v = Fraction(0)
        for kb in range(3):
            part = sum(Fraction(a[m, k]) * Fraction(b[n, k]) for k in range(128 * kb, 128 * kb + 128))
            v += Fraction(2) ** (int(sa[m, kb]) - 127) * Fraction(2) ** (int(sb[n // 128, kb]) - 127) * part
        assert D[m, n] == bf16_bits_of_fraction(v), (m, n)


def test_grouped_e8m0_forms_compose(orc):
    """The grouped forms with exponent scales are the dense form per group."""
    G, N, K = 2, 136, 256
    A, sa, _, _ = _rand_e8m0_case(256, N, K, 12)
    Bs = [_rand_e8m0_case(1, N, K, 20 + g) for g in range(G)]
    B = np.stack([b[2] for b in Bs]); sb = np.stack([b[3] for b in Bs])
    layout = np.repeat(np.array([1, 0], np.int32), 128)
    layout[5] = -1
    D = orc.gemm_grouped_contiguous_e8m0(A, sa, B, sb, layout)
    for g in range(G):
        rows = np.nonzero(layout == g)[0]
        assert np.array_equal(D[rows], orc.gemm_nt_e8m0(A, sa, B[g], sb[g], rows=rows))
    assert (D[5] == 0xFFFF).all()
    mm = np.array([100, 3], np.int32)
    Dm = orc.gemm_grouped_masked_e8m0(A.reshape(G, 128, K), sa.reshape(G, 128, -1), B, sb, mm)
    for g in range(G):
        ref = orc.gemm_nt_e8m0(A[g * 128:(g + 1) * 128], sa[g * 128:(g + 1) * 128], B[g], sb[g])
        assert np.array_equal(Dm[g, :mm[g]], ref[:mm[g]])
        assert (Dm[g, mm[g]:] == 0xFFFF).all()
