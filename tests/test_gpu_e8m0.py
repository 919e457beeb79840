"""GPU parity of the power-of-two (E8M0) scale path.

The quantizers must equal the oracle's bit for bit (codes with +0 and -0
counted as one, exponent bytes exactly, padding bytes untouched).  The three
GEMM forms run on inputs quantized by the oracle's own E8M0 quantizer and
must agree with the oracle to the workload tolerance on every routed element
of the call (the full-size workloads included), with every unrouted row left
at its 0xFFFF pre-fill."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_gemm_amd as dg
from fp8_block_scaled_gemm_amd.inputs import contiguous_case, dense_case, masked_case, workload
from tests.gpu_util import SENTINEL, assert_close_bf16, check_call, same_codes, to_dev
from tests.test_oracle_e8m0 import HAND

pytestmark = pytest.mark.gpu

PAD = 0xA5  # pre-fill of scale padding bytes, which no call may write


def _spread(rows: int, K: int, seed: int, lo: int = -120, hi: int = 100) -> np.ndarray:
    """Blocks of standard normals times 2^u, u uniform in [lo, hi), plus an
    all-zero block, a block of fp32 subnormals and a block of negative zeros."""
    rng = np.random.default_rng(seed)
    mag = np.exp2(rng.integers(lo, hi, (rows, K // 128)).astype(np.float64)).repeat(128, axis=1)
    x = (rng.standard_normal((rows, K)) * mag).astype(np.float32)
    if rows >= 3:
        x[0, :128] = 0.0
        x[1, -128:] = (rng.standard_normal(128) * 1e-40).astype(np.float32)
        x[2, :128] = -0.0
    return x


def _quant_token(orc, x: np.ndarray):
    M, K = x.shape
    KB = K // 128
    s = torch.full((M, dg.e8m0_pitch(KB)), PAD, dtype=torch.uint8, device="cuda")
    q, s = dg.dg_quantize_fp8_per_token_e8m0(to_dev(x), s=s)
    torch.cuda.synchronize()
    rq, rs = orc.quantize_per_token_e8m0(x)
    q, s = q.cpu().numpy(), s.cpu().numpy()
    assert same_codes(q, rq)
    assert np.array_equal(s[:, :KB], rs[:, :KB])
    assert (s[:, KB:] == PAD).all(), "a padding byte was written"
    return s


def _quant_block(orc, x: np.ndarray):
    N, K = x.shape
    KB = K // 128
    s = torch.full(((N + 127) // 128, dg.e8m0_pitch(KB)), PAD, dtype=torch.uint8, device="cuda")
    q, s = dg.dg_quantize_fp8_per_block_e8m0(to_dev(x), s=s)
    torch.cuda.synchronize()
    rq, rs = orc.quantize_per_block_e8m0(x)
    q, s = q.cpu().numpy(), s.cpu().numpy()
    assert same_codes(q, rq)
    assert np.array_equal(s[:, :KB], rs[:, :KB])
    assert (s[:, KB:] == PAD).all(), "a padding byte was written"
    return s


# --------------------------------------------------------------- quantize

@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (257, 1024), (4096, 2048)])
def test_per_token_e8m0_matches_oracle(orc, M, K):
    _quant_token(orc, _spread(M, K, M + K))
    _quant_token(orc, dense_case(M, 8, K, seed=M + K).x_a.numpy())


@pytest.mark.parametrize("N,K", [(8, 128), (200, 256), (2112, 1024), (7168, 2048)])
def test_per_block_e8m0_matches_oracle(orc, N, K):
    _quant_block(orc, _spread(N, K, 3 * N + K))
    _quant_block(orc, dense_case(8, N, K, seed=N * 3 + K).x_b.numpy())


def test_e8m0_hand_table(orc):
    """Every hand-worked exponent of the oracle pins, on the GPU: row i of a
    per-token input and row block i of a per-block input have amax HAND[i]."""
    x = np.zeros((len(HAND), 128), np.float32)
    w = np.zeros((128 * len(HAND), 128), np.float32)
    for i, (amax, _) in enumerate(HAND):
        x[i, 7] = -np.float32(amax)
        x[i, 9] = np.float32(amax) / 3
        w[128 * i + 5, 100] = np.float32(amax)
    s = _quant_token(orc, x)
    assert [int(b) for b in s[:, 0]] == [b for _, b in HAND]
    sb = _quant_block(orc, w)
    assert [int(b) for b in sb[:, 0]] == [b for _, b in HAND]


# -------------------------------------------------------------------- GEMM

def _prepared(orc, case):
    K = case.K
    qa, sa = orc.quantize_per_token_e8m0(case.x_a.numpy().reshape(-1, K))
    qa = qa.reshape(case.x_a.shape)
    sa = sa.reshape(*case.x_a.shape[:-1], -1)
    xb = case.x_b.numpy()
    if xb.ndim == 2:
        qb, sb = orc.quantize_per_block_e8m0(xb)
    else:
        parts = [orc.quantize_per_block_e8m0(np.ascontiguousarray(xb[g])) for g in range(xb.shape[0])]
        qb = np.stack([p[0] for p in parts]); sb = np.stack([p[1] for p in parts])
    return qa, sa, qb, sb


def _run(case, qa, sa, qb, sb):
    A, SA, B, SB = to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb)
    if case.form == "dense":
        D = torch.full((case.M, case.N), SENTINEL, dtype=torch.int16, device=A.device)
        dg.dg_fp8_gemm_nt_e8m0(A, SA, B, SB, D)
    elif case.form == "contiguous":
        D = torch.full((case.M, case.N), SENTINEL, dtype=torch.int16, device=A.device)
        dg.dg_fp8_gemm_grouped_contiguous_e8m0(A, SA, B, SB, D, to_dev(case.layout.numpy()))
    else:
        D = torch.full((case.G, case.M, case.N), SENTINEL, dtype=torch.int16, device=A.device)
        dg.dg_fp8_gemm_grouped_masked_e8m0(A, SA, B, SB, D, to_dev(case.masked_m.numpy()))
    torch.cuda.synchronize()
    return D.cpu().numpy().view(np.uint16).reshape(-1, case.N)


def _oracle(orc, case, qa, sa, qb, sb, rows=None):
    if case.form == "dense":
        return orc.gemm_nt_e8m0(qa, sa, qb, sb, rows=rows)
    if case.form == "contiguous":
        return orc.gemm_grouped_contiguous_e8m0(qa, sa, qb, sb, case.layout.numpy(), rows=rows)
    return orc.gemm_grouped_masked_e8m0(qa, sa, qb, sb, case.masked_m.numpy(), rows=rows)


def _routed(case) -> np.ndarray:
    if case.form == "dense":
        return np.arange(case.M)
    if case.form == "contiguous":
        lay = case.layout.numpy()
        return np.nonzero((lay >= 0) & (lay < case.G))[0]
    mm = np.clip(case.masked_m.numpy(), 0, case.M)
    return np.concatenate([g * case.M + np.arange(mm[g]) for g in range(case.G)]).astype(np.int64)


def _check_full(orc, case):
    qa, sa, qb, sb = _prepared(orc, case)
    got = _run(case, qa, sa, qb, sb)
    ref = _oracle(orc, case, qa, sa, qb, sb).reshape(-1, case.N)
    check_call(got, ref, _routed(case), case.name)
    return got


@pytest.mark.parametrize("tile", ["256x256", "256x224", "256x192", "256x160", "128x256", "128x128", "128x64", "128x32", "256x256t"])
@pytest.mark.parametrize("M,N,K", [(300, 712, 1024), (129, 136, 256), (64, 528, 384),
                                   (1, 8, 128), (257, 264, 1152)])
def test_dense_e8m0_parity(orc, monkeypatch, tile, M, N, K):
    monkeypatch.setenv("DG_FP8_DENSE_TILE", tile)
    _check_full(orc, dense_case(M, N, K, seed=M * 5 + N + K))


def test_dense_e8m0_wide_exponents(orc):
    """Block magnitudes from 2^-30 to 2^30: per-block exponent bytes far from
    127 on both operands, so a wrong bias, a swapped operand scale or a scale
    applied to the wrong row or K block shows at once."""
    M, N, K = 200, 392, 768
    case = dense_case(M, N, K, seed=8)
    case.x_a = torch.from_numpy(_spread(M, K, 81, -30, 30))
    case.x_b = torch.from_numpy(_spread(N, K, 82, -30, 30))
    _check_full(orc, case)


def test_grouped_e8m0_with_one_k_block(orc):
    _check_full(orc, contiguous_case(3, 136, 128, 33, sizes=[130, 0, 256]))
    _check_full(orc, masked_case(3, 192, 264, 128, 34, masked=[192, 5, 0]))


@pytest.mark.parametrize("sizes", [[100, 0, 260], [128, 1, 255, 3]])
def test_contiguous_e8m0_parity(orc, sizes):
    _check_full(orc, contiguous_case(len(sizes), 264, 384, 7, sizes=sizes))


def test_e8m0_with_more_slots_than_cus(orc):
    _check_full(orc, dense_case(4352, 4352, 256, seed=82))
    mm = np.random.default_rng(83).integers(0, 257, 70).astype(np.int32)
    _check_full(orc, masked_case(70, 256, 2048, 256, seed=83, masked=mm.tolist()))


def test_contiguous_e8m0_mixed_blocks_route_every_id(orc):
    # blocks whose rows carry several valid ids, across several column tiles
    case = contiguous_case(3, 600, 256, 9, sizes=[128, 128, 128])
    lay = case.layout.clone()
    lay[5:9] = 2
    lay[70:72] = 1
    lay[200:210] = 0
    lay[211] = -1
    case.layout = lay
    got = _check_full(orc, case)
    assert (got[211] == 0xFFFF).all()


@pytest.mark.parametrize("masked", [[0, 200, 37, 129], [1, 0, 128, 2]])
def test_masked_e8m0_parity(orc, masked):
    _check_full(orc, masked_case(len(masked), 256, 392, 640, 9, masked=masked))


@pytest.mark.parametrize("name", ["dense_e8m0_4096x7168x2048", "dense_e8m0_4096x24576x1536",
                                  "contiguous_e8m0_8x4096x7168", "masked_e8m0_16x256x4096x7168"])
def test_e8m0_full_size_every_routed_element(orc, name):
    got = _check_full(orc, workload(name))
    assert got.size
