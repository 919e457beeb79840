"""Seeded random shapes for every form and both scale kinds, each compared
element by element with the oracle (and unrouted rows checked untouched).
The shapes are drawn once from a fixed seed: ragged M and N (N a multiple
of 8), K from one to twelve 128-wide blocks, random group sizes and masks,
so the sweep crosses tile, scale-block and group boundaries the fixed cases
do not pick.  Every fourth dense shape also runs the fp32-addend form."""
import numpy as np
import pytest

from fp8_block_scaled_gemm_amd.inputs import (contiguous_case, dense_acc_case, dense_case,
                                              masked_case)
from tests import test_gpu_e8m0 as e8
from tests import test_gpu_gemm as f32

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261202)
# keep each case's oracle work (rows x N x K) small enough for seconds on the host
_BUDGET = 1.5e8


def _mnk(max_m):
    while True:
        M = int(_rng.integers(1, max_m + 1))
        N = 8 * int(_rng.integers(1, 130))
        K = 128 * int(_rng.integers(1, 13))
        if M * N * K <= _BUDGET:
            return M, N, K


DENSE = [_mnk(700) for _ in range(40)]
CONTIG = []
for _ in range(12):
    G = int(_rng.integers(1, 6))
    sizes = [int(x) for x in _rng.integers(0, 300, size=G)]
    N = 8 * int(_rng.integers(1, 70))
    K = 128 * int(_rng.integers(1, 9))
    CONTIG.append((sizes, N, K))
MASKED = []
for _ in range(12):
    G = int(_rng.integers(1, 7))
    M_max = int(_rng.integers(1, 300))
    masked = [int(x) for x in _rng.integers(-3, M_max + 5, size=G)]
    N = 8 * int(_rng.integers(1, 70))
    K = 128 * int(_rng.integers(1, 9))
    MASKED.append((masked, M_max, N, K))


@pytest.mark.parametrize("i", range(len(DENSE)))
def test_dense_sweep(orc, i):
    M, N, K = DENSE[i]
    f32._check_full(orc, dense_case(M, N, K, seed=1000 + i))
    e8._check_full(orc, dense_case(M, N, K, seed=2000 + i))
    if i % 4 == 0:
        f32._check_full(orc, dense_acc_case(M, N, K, seed=7000 + i))


@pytest.mark.parametrize("i", range(len(CONTIG)))
def test_contiguous_sweep(orc, i):
    sizes, N, K = CONTIG[i]
    if sum(sizes) == 0:
        sizes = sizes + [1]
    f32._check_full(orc, contiguous_case(len(sizes), N, K, seed=3000 + i, sizes=sizes))
    e8._check_full(orc, contiguous_case(len(sizes), N, K, seed=4000 + i, sizes=sizes))


@pytest.mark.parametrize("i", range(len(MASKED)))
def test_masked_sweep(orc, i):
    masked, M_max, N, K = MASKED[i]
    G = len(masked)
    f32._check_full(orc, masked_case(G, M_max, N, K, seed=5000 + i, masked=masked))
    e8._check_full(orc, masked_case(G, M_max, N, K, seed=6000 + i, masked=masked))
