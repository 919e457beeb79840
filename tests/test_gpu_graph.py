"""The GEMM entry points inside a captured HIP graph: each replay, with the
program's own eager work and synchronizations between replays, must leave
exactly what an eager call leaves (the entry points allocate, synchronize
and memset nothing, so they can be captured)."""
import numpy as np
import pytest
import torch

import fp8_block_scaled_gemm_amd as dg
from fp8_block_scaled_gemm_amd.inputs import contiguous_case, dense_case, masked_case
from tests.gpu_util import SENTINEL, to_dev

pytestmark = pytest.mark.gpu


def _operands(orc, case):
    K = case.K
    qa, sa = orc.quantize_per_token(case.x_a.numpy().reshape(-1, K))
    xb = case.x_b.numpy()
    if xb.ndim == 2:
        qb, sb = orc.quantize_per_block(xb)
    else:
        parts = [orc.quantize_per_block(np.ascontiguousarray(xb[g])) for g in range(xb.shape[0])]
        qb = np.stack([p[0] for p in parts]); sb = np.stack([p[1] for p in parts])
    qa = qa.reshape(case.x_a.shape)
    sa = sa.reshape(*case.x_a.shape[:-1], K // 128)
    return to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb)


@pytest.mark.parametrize("form", ["dense", "masked", "contiguous", "dense_acc"])
def test_graph_replays_match_eager(orc, form):
    extra = ()
    if form in ("dense", "dense_acc"):
        case = dense_case(300, 520, 768, seed=91)
        call = dg.dg_fp8_gemm_nt
        shape = (case.M, case.N)
        if form == "dense_acc":
            call = dg.dg_fp8_gemm_nt_acc
            C = np.random.default_rng(93).standard_normal(shape).astype(np.float32) * 20
            extra = (to_dev(C),)
    elif form == "masked":
        case = masked_case(3, 200, 264, 640, 92, masked=[150, 0, 200])
        call = dg.dg_fp8_gemm_grouped_masked
        shape = (case.G, case.M, case.N)
        extra = (to_dev(case.masked_m.numpy()),)
    else:
        # one block mixes two ids: the call's second launch has work too
        case = contiguous_case(3, 264, 384, 94, sizes=[128, 200, 100])
        lay = case.layout.clone()
        lay[3:7] = 2
        case.layout = lay
        call = dg.dg_fp8_gemm_grouped_contiguous
        shape = (case.M, case.N)
        extra = (to_dev(case.layout.numpy()),)
    A, SA, B, SB = _operands(orc, case)
    if form == "dense_acc":
        # the binding takes C before D
        acc_call = call
        C_dev = extra[0]
        call = lambda a, sa, b, sb, d: acc_call(a, sa, b, sb, C_dev, d)  # noqa: E731
        extra = ()

    eager = torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda")
    call(A, SA, B, SB, eager, *extra)
    torch.cuda.synchronize()

    out = torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(A, SA, B, SB, out, *extra)
    other = torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda")
    for rep in range(3):
        out.fill_(SENTINEL)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
        # eager work between replays, on other buffers
        call(A, SA, B, SB, other, *extra)
        torch.cuda.synchronize()
        assert torch.equal(other, eager)


@pytest.mark.parametrize("kind", ["per_token", "per_token_bf16", "per_block",
                                  "per_token_e8m0", "per_block_e8m0"])
def test_quantizer_graph_replays_match_eager(kind):
    # bench.py times the quantizers as captured graphs: every replay, with
    # eager work between replays, must give the eager call's codes and scales
    g = torch.Generator().manual_seed(93)
    x = torch.randn(260, 640, generator=g).cuda()
    if kind.endswith("bf16"):
        x = x.to(torch.bfloat16)
    fn = getattr(dg, "dg_quantize_fp8_" + kind)
    eq, es = fn(x)
    torch.cuda.synchronize()
    q, s = torch.empty_like(eq), torch.empty_like(es)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn(x, q, s)
    for rep in range(3):
        q.fill_(0)
        s.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(q, eq) and torch.equal(s, es), f"replay {rep} differs from the eager call"
        oq, os_ = fn(x)          # eager work between replays, on other buffers
        torch.cuda.synchronize()
        assert torch.equal(oq, eq) and torch.equal(os_, es)
