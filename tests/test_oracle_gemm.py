"""Pins for the oracle's block-scaled GEMM in its three forms.

Every check compares the oracle with something it does not share code with:
a hand-worked fixture, torch's fp64 matmul of torch-decoded operands (exact
when scales are 1 or powers of two), brute force in exact rational
arithmetic, integer matmul, an identity operand, scale linearity, and the
composition of the grouped forms from the dense one."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests.bf16_ref import bf16_bits_of_fraction, bf16_value
from fp8_block_scaled_gemm_amd.inputs import e4m3_pattern_matrix

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dec(q: np.ndarray) -> np.ndarray:
    """torch's own e4m3fn decode, as fp64."""
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16_to_f64(d: np.ndarray) -> np.ndarray:
    return torch.from_numpy(d.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def read_golden(name):
    A = B = sa = sb = None
    D = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].split()
        if not line:
            continue
        if line[0] == "shape":
            M, N, K = map(int, line[1:])
            A = np.zeros((M, K), np.uint8); B = np.zeros((N, K), np.uint8)
            sa = np.zeros((M, K // 128), np.float32); sb = np.zeros(((N + 127) // 128, K // 128), np.float32)
        elif line[0] in ("A", "B"):
            mat = A if line[0] == "A" else B
            r = int(line[1]); i = 2
            while i < len(line):
                if line[i] == "fill":
                    mat[r, :] = int(line[i + 1], 16); i += 2
                else:
                    mat[r, int(line[i + 1])] = int(line[i + 2], 16); i += 3
        elif line[0] in ("sa", "sb"):
            mat = sa if line[0] == "sa" else sb
            mat[int(line[1])] = [float(v) for v in line[2:]]
        elif line[0] == "D":
            D[(int(line[1]), int(line[2]))] = int(line[3], 16)
    return A, sa, B, sb, D


def test_handworked_fixture(orc):
    A, sa, B, sb, expected = read_golden("dense_handworked.txt")
    D = orc.gemm_nt(A, sa, B, sb)
    assert len(expected) == D.size
    for (m, n), bits in expected.items():
        assert D[m, n] == bits, (m, n, hex(D[m, n]), hex(bits))


def _rand_case(M, N, K, seed, scale_kind):
    rng = np.random.default_rng(seed)
    A = e4m3_pattern_matrix(M, K, seed)
    B = e4m3_pattern_matrix(N, K, seed + 1)
    KB, NB = K // 128, (N + 127) // 128
    if scale_kind == "unit":
        sa = np.ones((M, KB), np.float32); sb = np.ones((NB, KB), np.float32)
    elif scale_kind == "pow2":
        sa = np.exp2(rng.integers(-2, 3, (M, KB))).astype(np.float32)
        sb = np.exp2(rng.integers(-2, 3, (NB, KB))).astype(np.float32)
    else:
        sa = (rng.uniform(0.5, 2.0, (M, KB)) * 1e-2).astype(np.float32)
        sb = (rng.uniform(0.5, 2.0, (NB, KB)) * 1e-2).astype(np.float32)
    return A, sa, B, sb


def _per_kb_reference(A, sa, B, sb):
    """fp64 sum over K blocks of (sa * sb) * (A_blk @ B_blk^T), via torch."""
    M, K = A.shape
    N = B.shape[0]
    a = torch.from_numpy(dec(A)).reshape(M, K // 128, 128)
    b = torch.from_numpy(dec(B)).reshape(N, K // 128, 128)
    partial = torch.einsum("mkc,nkc->kmn", a, b)                     # [KB][M][N]
    sbn = torch.from_numpy(sb.astype(np.float64))[torch.arange(N) // 128]   # [N][KB]
    scale = torch.from_numpy(sa.astype(np.float64)).T[:, :, None] * sbn.T[:, None, :]
    return (scale * partial).sum(0).numpy()


@pytest.mark.parametrize("M,N,K", [(5, 24, 128), (33, 200, 384), (64, 256, 1024)])
def test_unit_scales_equal_fp64_matmul(orc, M, N, K):
    """All scales 1: V is the plain dot product, exact in fp64 in any order,
    so bf16(torch fp64 matmul) must match bit for bit.  A transposed operand
    or a dropped block would fail this."""
    A, sa, B, sb = _rand_case(M, N, K, M + N + K, "unit")
    V = torch.from_numpy(dec(A)) @ torch.from_numpy(dec(B)).T
    D = orc.gemm_nt(A, sa, B, sb)
    ref = np.array([[orc.bf16_from_double(float(v)) for v in row] for row in V.numpy()], np.uint16)
    assert np.array_equal(D, ref)


@pytest.mark.parametrize("M,N,K", [(17, 136, 256), (40, 264, 512)])
def test_pow2_scales_exact(orc, M, N, K):
    """Power-of-two scales keep every term exact, so the per-block torch
    reference is exact too and the bf16 results agree bit for bit.  A wrong
    sb row (n/128) or a swapped sa index fails here."""
    A, sa, B, sb = _rand_case(M, N, K, 3 * M + K, "pow2")
    V = _per_kb_reference(A, sa, B, sb)
    D = orc.gemm_nt(A, sa, B, sb)
    ref = np.vectorize(orc.bf16_from_double, otypes=[np.uint16])(V)
    assert np.array_equal(D, ref)


def test_general_scales_close(orc):
    A, sa, B, sb = _rand_case(48, 200, 640, 99, "general")
    V = _per_kb_reference(A, sa, B, sb)
    D = orc.gemm_nt(A, sa, B, sb)
    ref = np.vectorize(orc.bf16_from_double, otypes=[np.uint16])(V)
    diff = D != ref
    # only values within 1e-12 relative of a bf16 midpoint may differ, by one step
    assert diff.mean() < 1e-3
    got = bf16_to_f64(D[diff]); exp = bf16_to_f64(ref[diff])
    assert (np.abs(got - exp) <= np.abs(exp) * 2.0 ** -7 * 1.01).all()


def test_brute_force_rational_tiny(orc):
    """Triple loop in exact rationals, applying sa*sb to each product rather
    than to each block sum (a different association), then exact bf16."""
    M, N, K = 3, 9, 256
    A, sa, B, sb = _rand_case(M, N, K, 5, "general")
    D = orc.gemm_nt(A, sa, B, sb)
    da, db = dec(A), dec(B)
    for m in range(M):
        for n in range(N):
            v = Fraction(0)
            for k in range(K):
                s = Fraction(float(sa[m, k // 128])) * Fraction(float(sb[n // 128, k // 128]))
                v += s * Fraction(da[m, k]) * Fraction(db[n, k])
            # fp64 accumulation over 2 blocks can differ from the exact sum
            # only by rounding far below bf16 resolution
            assert D[m, n] == bf16_bits_of_fraction(v), (m, n)


def test_exact_integer_case(orc):
    """Scales 1, entries in -4..4 (exact in e4m3): V is an integer equal to
    the int64 matmul; with |V| <= 256 the bf16 result is exact."""
    rng = np.random.default_rng(1)
    M, N, K = 16, 32, 256
    ia = rng.integers(-4, 5, (M, K)); ib = rng.integers(-4, 5, (N, K))
    # keep |dot| <= 256: zero all but 16 entries per row of A
    mask = np.zeros((M, K), bool)
    for m in range(M):
        mask[m, rng.choice(K, 16, replace=False)] = True
    ia = np.where(mask, ia, 0)
    to_code = lambda v: torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    A, B = to_code(ia), to_code(ib)
    D = orc.gemm_nt(A, np.ones((M, 2), np.float32), B, np.ones((1, 2), np.float32))
    V = ia.astype(np.int64) @ ib.astype(np.int64).T
    assert np.abs(V).max() <= 256
    assert np.array_equal(bf16_to_f64(D), V.astype(np.float64))


def test_identity_b(orc):
    """B = I (code 0x38 on the diagonal), sb = 1: D[m,n] = bf16(sa[m, n/128] * A[m,n])."""
    M, K = 8, 256
    A = e4m3_pattern_matrix(M, K, 21)
    B = np.zeros((K, K), np.uint8); np.fill_diagonal(B, 0x38)
    rng = np.random.default_rng(2)
    sa = rng.uniform(0.1, 3.0, (M, 2)).astype(np.float32)
    D = orc.gemm_nt(A, sa, B, np.ones((2, 2), np.float32))
    exp = dec(A) * sa.astype(np.float64)[:, np.arange(K) // 128]
    ref = np.vectorize(orc.bf16_from_double, otypes=[np.uint16])(exp)
    # a -0 code times a scale is -0, while the block sum of the oracle starts
    # from +0: compare values, so that the two zeros are one
    assert np.array_equal(bf16_to_f64(D), bf16_to_f64(ref))


def test_scale_linearity(orc):
    """Doubling sa doubles D exactly; zeroing sa[:, kb] equals removing
    block kb from A."""
    A, sa, B, sb = _rand_case(12, 136, 512, 77, "general")
    D1 = orc.gemm_nt(A, sa, B, sb)
    D2 = orc.gemm_nt(A, (sa * 2).astype(np.float32), B, sb)
    assert np.array_equal(bf16_to_f64(D2), 2 * bf16_to_f64(D1))
    sa0 = sa.copy(); sa0[:, 2] = 0
    A0 = A.copy(); A0[:, 256:384] = 0
    assert np.array_equal(orc.gemm_nt(A, sa0, B, sb), orc.gemm_nt(A0, sa, B, sb))


def test_sb_row_selection_partial_block(orc):
    """N = 200: columns 0..127 use sb row 0 and 128..199 use row 1."""
    M, N, K = 4, 200, 128
    A = np.full((M, K), 0x38, np.uint8)
    B = np.full((N, K), 0x38, np.uint8)
    D = orc.gemm_nt(A, np.ones((M, 1), np.float32), B, np.array([[0.5], [4.0]], np.float32))
    v = bf16_to_f64(D)
    assert (v[:, :128] == 64.0).all() and (v[:, 128:] == 512.0).all()


def test_rows_variant_matches_full(orc):
    A, sa, B, sb = _rand_case(30, 72, 256, 8, "general")
    D = orc.gemm_nt(A, sa, B, sb)
    rows = np.array([29, 0, 7, 7], np.int64)
    assert np.array_equal(orc.gemm_nt(A, sa, B, sb, rows=rows), D[rows])


def test_contiguous_composes_from_dense(orc):
    G, N, K = 3, 72, 256
    sizes = [100, 0, 160]
    padded = [((s + 127) // 128) * 128 for s in sizes]
    layout = np.full(sum(padded), -1, np.int32)
    off = 0
    for g, (s, p) in enumerate(zip(sizes, padded)):
        layout[off:off + s] = g; off += p
    layout[5] = 7                      # out-of-range id: treated as padding
    M = layout.size
    A, sa, _, _ = _rand_case(M, N, K, 4, "general")
    Bs = [_rand_case(1, N, K, 10 + g, "general") for g in range(G)]
    B = np.stack([b[2] for b in Bs]); sb = np.stack([b[3] for b in Bs])
    D = orc.gemm_grouped_contiguous(A, sa, B, sb, layout)
    for r in range(M):
        g = layout[r]
        if 0 <= g < G:
            assert np.array_equal(D[r], orc.gemm_nt(A[r:r + 1], sa[r:r + 1], B[g], sb[g])[0])
        else:
            assert (D[r] == 0xFFFF).all()
    rows = np.array([0, 5, 101, M - 1], np.int64)
    assert np.array_equal(orc.gemm_grouped_contiguous(A, sa, B, sb, layout, rows=rows), D[rows])


def test_masked_composes_from_dense(orc):
    G, M_max, N, K = 4, 40, 24, 256
    masked = np.array([0, 40, 17, -3], np.int32)
    A = np.stack([_rand_case(M_max, N, K, 30 + g, "general")[0] for g in range(G)])
    sa = np.stack([_rand_case(M_max, N, K, 30 + g, "general")[1] for g in range(G)])
    B = np.stack([_rand_case(1, N, K, 50 + g, "general")[2] for g in range(G)])
    sb = np.stack([_rand_case(1, N, K, 50 + g, "general")[3] for g in range(G)])
    D = orc.gemm_grouped_masked(A, sa, B, sb, masked)
    for g in range(G):
        valid = min(max(int(masked[g]), 0), M_max)
        if valid:
            assert np.array_equal(D[g, :valid], orc.gemm_nt(A[g, :valid], sa[g, :valid], B[g], sb[g]))
        assert (D[g, valid:] == 0xFFFF).all()
    rows = np.array([0, 40 + 39, 80 + 16, 80 + 17], np.int64)
    out = orc.gemm_grouped_masked(A, sa, B, sb, masked, rows=rows)
    assert np.array_equal(out, D.reshape(-1, N)[rows])


def test_untouched_rows_keep_prefill(orc):
    G, M_max, N, K = 2, 8, 16, 128
    A = np.zeros((G, M_max, K), np.uint8); sa = np.ones((G, M_max, 1), np.float32)
    B = np.zeros((G, N, K), np.uint8); sb = np.ones((G, 1, 1), np.float32)
    D = np.full((G, M_max, N), 0x1234, np.uint16)
    orc.gemm_grouped_masked(A, sa, B, sb, np.zeros(G, np.int32), D=D)
    assert (D == 0x1234).all()
    lay = np.full(128, -1, np.int32)
    D2 = np.full((128, N), 0x4321, np.uint16)
    orc.gemm_grouped_contiguous(np.zeros((128, K), np.uint8), np.ones((128, 1), np.float32),
                                B, sb, lay, D=D2)
    assert (D2 == 0x4321).all()


# ---------------------------------------------------------------- accumulate
def test_acc_with_zero_addend_is_the_dense_form(orc):
    A = e4m3_pattern_matrix(12, 256, 31)
    B = e4m3_pattern_matrix(40, 256, 32)
    rng = np.random.default_rng(33)
    sa = rng.uniform(0.5, 2, (12, 2)).astype(np.float32)
    sb = rng.uniform(0.5, 2, (1, 2)).astype(np.float32)
    C = np.zeros((12, 40), np.float32)
    assert np.array_equal(orc.gemm_nt_acc(A, sa, B, sb, C), orc.gemm_nt(A, sa, B, sb))


def test_acc_with_zero_product_rounds_the_addend(orc):
    """A = 0: D is C rounded to bf16 (torch's fp32 -> bf16 cast, nearest even)."""
    rng = np.random.default_rng(34)
    C = (rng.standard_normal((9, 24)) * 10.0 ** rng.integers(-30, 30, (9, 24))).astype(np.float32)
    A = np.zeros((9, 128), np.uint8)
    B = e4m3_pattern_matrix(24, 128, 35)
    D = orc.gemm_nt_acc(A, np.ones((9, 1), np.float32), B, np.ones((1, 1), np.float32), C)
    ref = torch.from_numpy(C).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(D, ref)


def test_acc_exact_integer_case(orc):
    """Small integers in A, B and C with unit scales: D equals the int64
    matmul plus C exactly while |V + C| <= 256."""
    rng = np.random.default_rng(36)
    M, N, K = 16, 24, 128
    ia = rng.integers(-3, 4, (M, K)); ib = rng.integers(-3, 4, (N, K))
    mask = np.zeros((M, K), bool)
    for m in range(M):
        mask[m, rng.choice(K, 8, replace=False)] = True
    ia = np.where(mask, ia, 0)
    ic = rng.integers(-150, 151, (M, N))
    to_code = lambda v: torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    D = orc.gemm_nt_acc(to_code(ia), np.ones((M, 1), np.float32), to_code(ib),
                        np.ones((1, 1), np.float32), ic.astype(np.float32))
    V = ia.astype(np.int64) @ ib.astype(np.int64).T + ic
    assert np.abs(V).max() <= 256
    assert np.array_equal(bf16_to_f64(D), V.astype(np.float64))


def test_acc_brute_force_rational(orc):
    """Exact rational sum plus C, rounded once, against the oracle."""
    rng = np.random.default_rng(37)
    M, N, K = 3, 5, 256
    A = e4m3_pattern_matrix(M, K, 38); B = e4m3_pattern_matrix(N, K, 39)
    sa = rng.uniform(0.1, 3, (M, 2)).astype(np.float32)
    sb = rng.uniform(0.1, 3, (1, 2)).astype(np.float32)
    C = (rng.standard_normal((M, N)) * 50).astype(np.float32)
    D = orc.gemm_nt_acc(A, sa, B, sb, C)
    da, db = dec(A), dec(B)
    for m in range(M):
        for n in range(N):
            v = Fraction(float(C[m, n]))
            for k in range(K):
                s = Fraction(float(sa[m, k // 128])) * Fraction(float(sb[0, k // 128]))
                v += s * Fraction(da[m, k]) * Fraction(db[n, k])
            assert D[m, n] == bf16_bits_of_fraction(v), (m, n)
