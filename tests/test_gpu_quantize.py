"""GPU parity of the quantize helpers: codes and scales must equal the
oracle's bit for bit (+0 and -0 codes counted as one)."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_gemm_amd as dg
from fp8_block_scaled_gemm_amd.inputs import dense_case, workload
from tests.gpu_util import same_codes, to_dev

pytestmark = pytest.mark.gpu


def _per_token(orc, x: np.ndarray):
    q, s = dg.dg_quantize_fp8_per_token(to_dev(x))
    torch.cuda.synchronize()
    rq, rs = orc.quantize_per_token(x)
    assert same_codes(q.cpu().numpy(), rq)
    assert np.array_equal(s.cpu().numpy(), rs)


def _per_token_bf16(orc, bits: np.ndarray):
    xb = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    q, s = dg.dg_quantize_fp8_per_token_bf16(xb)
    torch.cuda.synchronize()
    rq, rs = orc.quantize_per_token_bf16(bits)
    assert same_codes(q.cpu().numpy(), rq)
    assert np.array_equal(s.cpu().numpy(), rs)


def _per_block(orc, x: np.ndarray):
    q, s = dg.dg_quantize_fp8_per_block(to_dev(x))
    torch.cuda.synchronize()
    rq, rs = orc.quantize_per_block(x)
    assert same_codes(q.cpu().numpy(), rq)
    assert np.array_equal(s.cpu().numpy(), rs)


@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (257, 1024), (4096, 2048)])
def test_per_token_matches_oracle(orc, M, K):
    x = dense_case(M, 8, K, seed=M + K).x_a.numpy()
    _per_token(orc, x)


@pytest.mark.parametrize("N,K", [(8, 128), (200, 256), (2112, 1024), (7168, 2048)])
def test_per_block_matches_oracle(orc, N, K):
    x = dense_case(8, N, K, seed=N * 3 + K).x_b.numpy()
    _per_block(orc, x)


def _edge_matrix():
    """Blocks whose amax is 448 (scale exactly 1), so x/scale == x and every
    e4m3 midpoint, subnormal and signed zero is hit exactly; plus an all-zero
    block and blocks at extreme magnitudes."""
    codes = torch.arange(0x7F, dtype=torch.uint8)
    grid = codes.view(torch.float8_e4m3fn).float().numpy()
    mids = ((grid[:-1].astype(np.float64) + grid[1:]) / 2).astype(np.float32)
    vals = np.concatenate([grid, mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(1e9)),
                           np.float32([0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -10, 1e-30])])
    vals = np.concatenate([vals, -vals])
    n_blocks = (vals.size + 126) // 127
    rows = []
    for b in range(n_blocks):
        chunk = vals[b * 127:(b + 1) * 127]
        row = np.zeros(128, np.float32)
        row[0] = 448.0
        row[1:1 + chunk.size] = chunk
        rows.append(row)
    rows.append(np.zeros(128, np.float32))                            # amax 0
    rows.append((np.full(128, 3e38) * np.where(np.arange(128) % 2, 1, -1)).astype(np.float32))
    rows.append(np.linspace(-1e-38, 1e-38, 128).astype(np.float32))  # fp32 subnormal scale
    rows.append(np.random.default_rng(0).standard_normal(128).astype(np.float32) * 1e-20)
    return np.stack(rows).astype(np.float32)


def test_per_token_edge_values(orc):
    x = _edge_matrix()
    _per_token(orc, x)
    # the same rows as a per-block matrix: pad to one 128-row block with zeros
    _per_token(orc, np.concatenate([x, x[::-1]], axis=1))


def test_per_block_edge_values(orc):
    x = _edge_matrix()
    _per_block(orc, np.ascontiguousarray(np.concatenate([x, x], axis=1)))


def test_quantize_workload_activations_and_weights(orc):
    """The masked decode workload's A slabs and one expert's B, as the bench
    quantizes them."""
    case = workload("masked_16x256x7168x2048")
    _per_token(orc, case.x_a.reshape(-1, case.K)[:1024].numpy())
    _per_block(orc, case.x_b[3].numpy())


@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (257, 1024), (4096, 2048)])
def test_per_token_bf16_matches_oracle(orc, M, K):
    x = dense_case(M, 8, K, seed=M + K + 1).x_a
    _per_token_bf16(orc, x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_per_token_bf16_all_bit_patterns(orc):
    """Every finite bf16 bit pattern, 128 to a block (blocks of one binade
    and sign, so tiny and huge amax both occur)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    bits = bits[: bits.size // 128 * 128].reshape(-1, 128)
    _per_token_bf16(orc, bits)


def test_quantize_is_deterministic():
    x = to_dev(dense_case(512, 8, 2048, seed=9).x_a.numpy())
    q1, s1 = dg.dg_quantize_fp8_per_token(x)
    q2, s2 = dg.dg_quantize_fp8_per_token(x)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
