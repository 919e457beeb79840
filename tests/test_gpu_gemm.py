"""GPU parity of the three GEMM forms against the CPU oracle.

Inputs are seeded fp32 draws quantized by the oracle's own quantizer (the GPU
quantizer is checked separately, bit for bit), so no oracle input comes from
the HIP path.  Every case, the full-size named workloads included, compares
every routed element of D with the oracle's whole-call result (RMS taken over
all routed elements of the call) and every unrouted row of D with its
untouched 0xFFFF pre-fill."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_gemm_amd as dg
from fp8_block_scaled_gemm_amd.inputs import (contiguous_case, dense_case, masked_case,
                                              workload)
from tests.gpu_util import SENTINEL, assert_close_bf16, check_call, to_dev

pytestmark = pytest.mark.gpu


def _quant_a(orc, x_a: np.ndarray):
    K = x_a.shape[-1]
    q, s = orc.quantize_per_token(x_a.reshape(-1, K))
    return q.reshape(x_a.shape), s.reshape(*x_a.shape[:-1], K // 128)


def _quant_b(orc, x_b: np.ndarray):
    if x_b.ndim == 2:
        return orc.quantize_per_block(x_b)
    qs = [orc.quantize_per_block(np.ascontiguousarray(x_b[g])) for g in range(x_b.shape[0])]
    return np.stack([q for q, _ in qs]), np.stack([s for _, s in qs])


def _prepared(orc, case):
    qa, sa = _quant_a(orc, case.x_a.numpy())
    qb, sb = _quant_b(orc, case.x_b.numpy())
    return qa, sa, qb, sb


def _run(case, qa, sa, qb, sb):
    A, SA, B, SB = to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb)
    if case.form == "dense":
        D = torch.full((case.M, case.N), SENTINEL, dtype=torch.int16, device=A.device)
        dg.dg_fp8_gemm_nt(A, SA, B, SB, D)
    elif case.form == "dense_acc":
        D = torch.full((case.M, case.N), SENTINEL, dtype=torch.int16, device=A.device)
        dg.dg_fp8_gemm_nt_acc(A, SA, B, SB, to_dev(case.x_c.numpy()), D)
    elif case.form == "contiguous":
        D = torch.full((case.M, case.N), SENTINEL, dtype=torch.int16, device=A.device)
        dg.dg_fp8_gemm_grouped_contiguous(A, SA, B, SB, D, to_dev(case.layout.numpy()))
    else:
        D = torch.full((case.G, case.M, case.N), SENTINEL, dtype=torch.int16, device=A.device)
        dg.dg_fp8_gemm_grouped_masked(A, SA, B, SB, D, to_dev(case.masked_m.numpy()))
    torch.cuda.synchronize()
    return D.cpu().numpy().view(np.uint16)


def _oracle_full(orc, case, qa, sa, qb, sb):
    if case.form == "dense":
        return orc.gemm_nt(qa, sa, qb, sb)
    if case.form == "dense_acc":
        return orc.gemm_nt_acc(qa, sa, qb, sb, case.x_c.numpy())
    if case.form == "contiguous":
        return orc.gemm_grouped_contiguous(qa, sa, qb, sb, case.layout.numpy())
    return orc.gemm_grouped_masked(qa, sa, qb, sb, case.masked_m.numpy())


def _routed_rows(case) -> np.ndarray:
    """Flat row indices (into D viewed as [rows][N]) the call must write."""
    if case.form in ("dense", "dense_acc"):
        return np.arange(case.M)
    if case.form == "contiguous":
        lay = case.layout.numpy()
        return np.nonzero((lay >= 0) & (lay < case.G))[0]
    mm = np.clip(case.masked_m.numpy(), 0, case.M)
    return np.concatenate([g * case.M + np.arange(mm[g]) for g in range(case.G)]).astype(np.int64)


def _check_full(orc, case):
    qa, sa, qb, sb = _prepared(orc, case)
    got = _run(case, qa, sa, qb, sb).reshape(-1, case.N)
    ref = _oracle_full(orc, case, qa, sa, qb, sb).reshape(-1, case.N)
    check_call(got, ref, _routed_rows(case), case.name)
    return got


# ------------------------------------------------------------ small/medium

@pytest.mark.parametrize("M,N,K", [
    (128, 512, 512),      # the smallest named workload
    (1, 8, 128),          # minimal sizes
    (300, 712, 1024),     # ragged M and N tails, several tiles
    (129, 136, 256),      # one row / one 8-column group past a tile
    (64, 2112 // 4, 384), # N % 128 == 16: partial last scale block
    (257, 264, 1152),     # odd K-block count
])
def test_dense_parity(orc, M, N, K):
    _check_full(orc, dense_case(M, N, K, seed=M * 7 + N + K, name=f"dense_{M}x{N}x{K}"))


@pytest.mark.parametrize("tile", ["256x256", "256x224", "256x192", "256x160", "128x256", "128x128", "128x64", "128x32", "256x256t"])
@pytest.mark.parametrize("M,N,K", [(300, 488, 384), (512, 448, 256), (40, 200, 128)])
def test_dense_tile_shapes(orc, monkeypatch, tile, M, N, K):
    # every dense tile shape on ragged and exact sizes: several tiles, a
    # partial last tile in M and N, tiles straddling column-scale blocks
    monkeypatch.setenv("DG_FP8_DENSE_TILE", tile)
    _check_full(orc, dense_case(M, N, K, seed=M + N + K))


@pytest.mark.parametrize("M,N,K", [
    (40, 24, 1 << 20),     # 8192 K blocks: long K loop, per-lane offsets near 2^28
    (3, 1 << 20, 128),     # 4096 column tiles: large column offsets into B and D
    (1 << 17, 8, 256),     # 512 row tiles of a single 8-column group
])
def test_dense_extreme_extents(orc, M, N, K):
    _check_full(orc, dense_case(M, N, K, seed=M + N % 1000 + K % 1000, name=f"dense_{M}x{N}x{K}"))


def test_dense_parity_scaled_rows(orc):
    """Rows with very different magnitudes: per-row scales span 2^-20..2^20."""
    case = dense_case(200, 264, 512, seed=5)
    case.x_a *= torch.exp2(torch.linspace(-20, 20, 200)).unsqueeze(1)
    _check_full(orc, case)


@pytest.mark.parametrize("sizes", [[100, 0, 260], [128, 1, 255, 3]])
def test_contiguous_parity(orc, sizes):
    case = contiguous_case(len(sizes), 264, 512, seed=sum(sizes) + 1, sizes=sizes)
    _check_full(orc, case)


def test_zero_rows_are_a_no_op(orc):
    """M = 0 (dense), M_sum = 0 (contiguous) and M_max = 0 (masked) enqueue
    nothing and return success; a neighbouring buffer stays untouched."""
    dev = torch.device("cuda:0")
    K, N, G = 256, 64, 2
    A = torch.zeros((0, K), dtype=torch.uint8, device=dev)
    SA = torch.zeros((0, K // 128), dtype=torch.float32, device=dev)
    B = torch.zeros((G, N, K), dtype=torch.uint8, device=dev)
    SB = torch.ones((G, N // 128 + 1, K // 128), dtype=torch.float32, device=dev)
    guard = torch.full((16, N), SENTINEL, dtype=torch.int16, device=dev)
    D = guard[:0]
    dg.dg_fp8_gemm_nt(A, SA, B[0], SB[0], D)
    dg.dg_fp8_gemm_grouped_contiguous(A, SA, B, SB, D, torch.zeros(0, dtype=torch.int32, device=dev))
    dg.dg_fp8_gemm_grouped_masked(A.reshape(G, 0, K), SA.reshape(G, 0, K // 128), B, SB,
                                  guard[:0].reshape(G, 0, N),
                                  torch.zeros(G, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert (guard.cpu().numpy().view(np.uint16) == 0xFFFF).all()


def test_grouped_forms_with_one_k_block(orc):
    # K = 128: the pipeline's second prologue block and every refill are
    # empty loads
    _check_full(orc, contiguous_case(3, 136, 128, seed=31, sizes=[130, 0, 256]))
    _check_full(orc, masked_case(3, 192, 264, 128, seed=32, masked=[192, 5, 0]))


def test_contiguous_out_of_range_ids_are_padding(orc):
    case = contiguous_case(3, 136, 256, seed=12, sizes=[200, 50, 128])
    lay = case.layout.clone()
    lay[3] = 3          # id == G: not a group
    lay[130] = 99
    case.layout = lay
    _check_full(orc, case)


@pytest.mark.parametrize("sizes", [
    [1, 128, 100, 128, 50, 128, 127],   # every 256-row tile holds two groups
    [128, 0, 128, 128, 128, 0, 5],      # split, whole and ragged-last tiles
    [256, 130, 126, 300],               # a tile holds the ends of two groups
])
def test_contiguous_split_tiles(orc, sizes):
    # 256-row tiles whose two 128-row blocks carry different groups: one
    # workgroup per block, each with its own group's B
    _check_full(orc, contiguous_case(len(sizes), 264, 384, seed=len(sizes) + sum(sizes),
                                     sizes=sizes))


def test_contiguous_mixed_blocks_route_every_id(orc):
    # a 128-row block whose rows carry several valid ids is run once per id,
    # so every row is computed with its own group's B, as the oracle does;
    # padding rows (-1) and ids outside [0, G) inside such blocks stay
    # untouched
    case = contiguous_case(3, 136, 256, seed=21, sizes=[128, 128, 128])
    lay = case.layout.clone()
    lay[140:150] = 0    # block 1 (group 1) with some rows of group 0
    lay[150:152] = -1   # and two padding rows
    lay[260:270] = 2    # block 2 is group 2 already: no change in routing
    lay[10:20] = 2      # block 0 (group 0) with rows of group 2 ...
    lay[30:33] = 1      # ... and of group 1: three passes
    lay[40] = 3         # an id past G is not routed
    case.layout = lay
    qa, sa, qb, sb = _prepared(orc, case)
    got = _run(case, qa, sa, qb, sb).reshape(-1, case.N)
    ref = _oracle_full(orc, case, qa, sa, qb, sb).reshape(-1, case.N)
    routed = ((lay >= 0) & (lay < 3)).numpy()
    assert (~routed).sum() == 3
    assert (got[~routed] == 0xFFFF).all()
    assert_close_bf16(got[routed], ref[routed], "mixed blocks")


def test_contiguous_all_padding_leaves_d_untouched(orc):
    case = contiguous_case(2, 64, 256, seed=13, sizes=[0, 0])
    case.layout = torch.full((256,), -1, dtype=torch.int32)
    case.M = 256
    case.x_a = torch.randn(256, 256, generator=torch.Generator().manual_seed(13))
    got = _check_full(orc, case)
    assert (got == 0xFFFF).all()


@pytest.mark.parametrize("masked", [[0, 200, 37, 129], [200, 200, 200, 200], [1, 0, 128, 2]])
def test_masked_parity(orc, masked):
    _check_full(orc, masked_case(4, 200, 136, 384, seed=sum(masked), masked=masked))


def test_masked_out_of_range_counts_are_clamped(orc):
    _check_full(orc, masked_case(3, 64, 24, 256, seed=2, masked=[-5, 1000, 64]))


def test_masked_many_groups(orc):
    # more (group, m-block) pairs than lanes in a wave, with ties and empty groups
    rng = np.random.default_rng(70)
    masked = [int(x) for x in rng.integers(0, 41, size=70)]
    masked[3] = masked[9] = 40
    masked[5] = 0
    _check_full(orc, masked_case(70, 40, 136, 256, seed=70, masked=masked))


def test_masked_several_m_blocks(orc):
    # groups taller than one tile: a group's m-blocks carry different costs
    _check_full(orc, masked_case(3, 600, 136, 256, seed=600, masked=[600, 257, 513]))


def test_masked_all_zero_leaves_d_untouched(orc):
    got = _check_full(orc, masked_case(3, 64, 24, 256, seed=3, masked=[0, 0, 0]))
    assert (got == 0xFFFF).all()


def test_epilogue_rounding_is_exact(orc, monkeypatch):
    """Small-integer operands and unit scales make every block sum exact in
    fp32, so D differs from the exact value only by the bf16 rounding; many
    sums fall on ties (odd multiples of half a bf16 step), which must round
    to even.  Bit-exact against the oracle, every dense tile shape."""
    rng = np.random.default_rng(257)
    M, N, K = 256, 256, 256
    code = {v: orc.e4m3_from_float(float(v)) for v in range(0, 9)}
    a_val = rng.integers(0, 9, size=(M, K))
    b_val = rng.integers(0, 9, size=(N, K))
    qa = np.vectorize(code.get)(a_val).astype(np.uint8)
    qb = np.vectorize(code.get)(b_val).astype(np.uint8)
    sa = np.ones((M, K // 128), np.float32)
    sb = np.ones((N // 128, K // 128), np.float32)
    exact = (a_val @ b_val.T).astype(np.int64)
    step = 2 ** (np.floor(np.log2(np.maximum(exact, 1))).astype(np.int64) - 7)
    ties = (exact >= 256) & (exact % step == step // 2)
    assert ties.sum() > 1000
    ref = orc.gemm_nt(qa, sa, qb, sb)
    case = dense_case(M, N, K, seed=0)
    for tile in ("256x256", "256x224", "256x192", "256x160", "128x256", "128x128", "128x64", "128x32"):
        monkeypatch.setenv("DG_FP8_DENSE_TILE", tile)
        got = _run(case, qa, sa, qb, sb).reshape(M, N)
        assert np.array_equal(got, ref), tile


def test_launches_with_more_slots_than_cus(orc):
    """Launches with more tile slots than the device has CUs, in full: 289
    dense tiles, about 600 contiguous tiles with a mixed block and padding
    blocks, and 560 masked slots over 70 groups, some of them empty."""
    _check_full(orc, dense_case(4352, 4352, 256, seed=77))
    case = contiguous_case(5, 4096, 256, seed=78, m_lo=600, m_hi=1100)
    lay = case.layout.clone()
    lay[5:9] = (int(lay[0]) + 1) % 5   # one mixed block
    case.layout = lay
    _check_full(orc, case)
    mm = np.random.default_rng(79).integers(0, 257, 70).astype(np.int32)
    mm[::9] = 0
    _check_full(orc, masked_case(70, 256, 2048, 256, seed=79, masked=mm.tolist()))


def test_acc_with_more_slots_than_cus(orc):
    M, N, K = 4352, 4352, 256
    case = dense_case(M, N, K, seed=80)
    qa, sa, qb, sb = _prepared(orc, case)
    C = (np.random.default_rng(81).standard_normal((M, N)) * np.sqrt(K)).astype(np.float32)
    D = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_fp8_gemm_nt_acc(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), to_dev(C), D)
    torch.cuda.synchronize()
    check_call(D.cpu().numpy().view(np.uint16), orc.gemm_nt_acc(qa, sa, qb, sb, C),
               np.arange(M), "acc, 289 tiles")


@pytest.mark.parametrize("tile", ["256x256", "256x224", "256x192", "256x160", "128x256", "128x128", "128x64", "128x32", None])
@pytest.mark.parametrize("M,N,K", [(300, 488, 384), (64, 256, 128), (512, 520, 256)])
def test_dense_acc_parity(orc, monkeypatch, tile, M, N, K):
    """D = bf16(C + dense sum) against the oracle; C of the product's size
    and, in every other row, a hundred times larger (a dropped or doubled
    addend fails)."""
    if tile:
        monkeypatch.setenv("DG_FP8_DENSE_TILE", tile)
    case = dense_case(M, N, K, seed=M * 7 + N + K)
    qa, sa, qb, sb = _prepared(orc, case)
    rng = np.random.default_rng(M + N)
    C = (rng.standard_normal((M, N)) * np.where(np.arange(M)[:, None] % 2, 100.0, 1.0)
         * np.sqrt(K)).astype(np.float32)
    D = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda")
    dg.dg_fp8_gemm_nt_acc(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), to_dev(C), D)
    torch.cuda.synchronize()
    got = D.cpu().numpy().view(np.uint16)
    ref = orc.gemm_nt_acc(qa, sa, qb, sb, C)
    assert_close_bf16(got, ref, f"acc {M}x{N}x{K} {tile}")


def test_zero_scale_block(orc):
    """A zero block of A (amax 0, scale 0) contributes nothing."""
    case = dense_case(130, 136, 512, seed=17)
    case.x_a[:, 128:256] = 0
    case.x_a[5] = 0
    _check_full(orc, case)


def test_gemm_is_deterministic(orc):
    case = dense_case(300, 712, 1024, seed=4)
    qa, sa, qb, sb = _prepared(orc, case)
    a = _run(case, qa, sa, qb, sb)
    b = _run(case, qa, sa, qb, sb)
    assert np.array_equal(a, b)


# --------------------------------------------------------------- full size

FULL = ["dense_128x512x512", "dense_4096x7168x2048", "dense_64x7168x2048",
        "dense_128x7168x2048", "dense_4096x24576x1536", "dense_4096x2112x7168",
        "dense_acc_4096x7168x2048", "contiguous_8x4096x7168", "masked_16x256x4096x7168",
        "masked_16x256x7168x2048"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_every_routed_element(orc, name):
    """The named workloads at their full sizes, in the launch configuration
    the benchmark times: the oracle computes the whole call and every routed
    element is compared."""
    got = _check_full(orc, workload(name))
    assert got.size
