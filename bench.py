"""Benchmark of the FP8 block-scaled NT GEMM on one MI355X.

A step is one call of the GEMM entry point (tile scheduling, operand and
scale staging, FP8 MFMA per 128-wide K block, promotion, bf16 epilogue) on
inputs already quantized and resident in HBM.  The default workload is the
dense M=4096, N=7168, K=2048 projection.  Inputs rotate over enough copies
(more than 512 MiB in total) that the 256 MiB last-level cache cannot serve
them from one step to the next.

Prints one JSON line:
  value        TFLOPS over the timed steps (2*rows*N*K per step / wall time)
  roofline     the GEMM kernel against the dense FP8 MFMA peak (or HBM for
               bandwidth-bound workloads), from HIP events on the launch
               stream around the timed graph replay (one GEMM per step)
  cpu_baseline the CPU oracle on a bounded sample of the same workload
  same_buffer  the same steps on one input set (warm caches), for comparison
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
ROTATE_BYTES = 512 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dense_4096x7168x2048")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the K steps as eager launches instead of one captured HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the CPU-oracle sample")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the GEMM, time a plain device copy of this many bytes "
                         "(the reference kernel for scaling HBM byte counters)")
    return ap.parse_args()


def copy_reference(nbytes: int, steps: int, warmup: int):
    """A plain device-to-device copy of known size, for calibrating the
    FETCH_SIZE / WRITE_SIZE counters against bytes actually moved."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_bytes": nbytes, "steps": steps, "us_per_copy": round(dt * 1e6, 2),
                      "GB/s (read+write)": round(2 * nbytes / dt / 1e9, 1)}), flush=True)


def algorithmic(case):
    """FLOP and HBM bytes the method must move per call (unrouted rows and
    groups without rows excluded)."""
    rows = case.valid_rows
    KB, NB = case.K // 128, (case.N + 127) // 128
    flop = 2.0 * rows * case.N * case.K
    groups = case.active_groups
    byts = (rows * case.K                     # A codes
            + groups * case.N * case.K        # B codes of groups in use
            + (1 if case.scales == "e8m0" else 4) * (rows * KB + groups * NB * KB)   # scales
            + 2 * rows * case.N)              # bf16 D
    if case.x_c is not None:
        byts += 4 * rows * case.N             # fp32 C
    return flop, float(byts)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_block_scaled_gemm_amd", "csrc")
    for f in ("gemm.hip", "device_common.h", "launch.h"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_gemm_{workload}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*(\w+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def make_inputs(case, dev, dg):
    import torch
    x_a = case.x_a.to(dev)
    x_b = case.x_b.to(dev)
    K = case.K
    e8 = case.scales == "e8m0"
    q_token = dg.dg_quantize_fp8_per_token_e8m0 if e8 else dg.dg_quantize_fp8_per_token
    q_block = dg.dg_quantize_fp8_per_block_e8m0 if e8 else dg.dg_quantize_fp8_per_block
    qa, sa = q_token(x_a.reshape(-1, K))
    qa = qa.reshape(x_a.shape)
    sa = sa.reshape(*x_a.shape[:-1], sa.shape[-1])
    if x_b.dim() == 2:
        qb, sb = q_block(x_b)
    else:
        parts = [q_block(x_b[g].contiguous()) for g in range(x_b.shape[0])]
        qb = torch.stack([p[0] for p in parts])
        sb = torch.stack([p[1] for p in parts])
    aux = None
    if case.form == "contiguous":
        aux = case.layout.to(dev)
    elif case.form == "masked":
        aux = case.masked_m.to(dev)
    if case.form == "masked":
        D = torch.empty((case.G, case.M, case.N), dtype=torch.bfloat16, device=dev)
    else:
        D = torch.empty((case.M, case.N), dtype=torch.bfloat16, device=dev)
    C = case.x_c.to(dev) if case.x_c is not None else None
    return {"A": qa, "sa": sa, "B": qb, "sb": sb, "C": C, "D": D, "aux": aux, "x_a": x_a,
            "x_b": x_b}


def gemm_call(case, dg, t):
    if case.scales == "e8m0":
        if case.form == "dense":
            dg.dg_fp8_gemm_nt_e8m0(t["A"], t["sa"], t["B"], t["sb"], t["D"])
        elif case.form == "contiguous":
            dg.dg_fp8_gemm_grouped_contiguous_e8m0(t["A"], t["sa"], t["B"], t["sb"], t["D"], t["aux"])
        else:
            dg.dg_fp8_gemm_grouped_masked_e8m0(t["A"], t["sa"], t["B"], t["sb"], t["D"], t["aux"])
        return
    if case.form == "dense":
        dg.dg_fp8_gemm_nt(t["A"], t["sa"], t["B"], t["sb"], t["D"])
    elif case.form == "dense_acc":
        dg.dg_fp8_gemm_nt_acc(t["A"], t["sa"], t["B"], t["sb"], t["C"], t["D"])
    elif case.form == "contiguous":
        dg.dg_fp8_gemm_grouped_contiguous(t["A"], t["sa"], t["B"], t["sb"], t["D"], t["aux"])
    else:
        dg.dg_fp8_gemm_grouped_masked(t["A"], t["sa"], t["B"], t["sb"], t["D"], t["aux"])


def same_buffer_rate(case, dg, inputs, steps, flop):
    """The same K steps on one input set (warm: operands may stay in the
    last-level cache between steps), as a captured graph, for comparison
    with the rotated-input figure that `value` reports."""
    import torch
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            gemm_call(case, dg, inputs)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    return {"kernel_us": round(us, 2), "TFLOPS": round(flop / (us * 1e-6) / 1e12, 1)}


def time_quantize(dg, t, case, reps=20):
    """Average time of the per-token quantization of A (the activation side,
    re-done every step in use), from fp32 and from bf16 input, and of the
    per-block quantization of one B matrix; reported beside the GEMM.

    Each is timed with HIP events around one replay of a captured graph of
    `reps` calls (these kernels take a few microseconds, about what one call
    through the Python binding costs on the host, so eager launches would
    time the host).  The calls rotate over distinct input and output buffers
    totalling more than 512 MiB, so every call reads its input from HBM and
    not from the 256 MiB last-level cache."""
    import torch
    x = t["x_a"].reshape(-1, case.K)
    w = t["x_b"].reshape(-1, case.K) if t["x_b"].dim() == 2 else t["x_b"][0]
    KB, SP = case.K // 128, dg.e8m0_pitch(case.K // 128)
    NB = (w.shape[0] + 127) // 128

    def buffers(src, s_shape, s_dtype, in_dtype):
        """Copies of (input, codes, scales), enough of them to exceed the
        rotation size."""
        src = src.to(in_dtype)
        one = src.numel() * (src.element_size() + 1) + 4 * s_shape[0] * s_shape[1]
        n = max(2, -(-ROTATE_BYTES // one))
        return [(src.clone(), torch.empty(src.shape, dtype=torch.uint8, device=src.device),
                 torch.zeros(s_shape, dtype=s_dtype, device=src.device)) for _ in range(n)]

    def timed(fn, bufs):
        for i in range(3):
            fn(*bufs[i % len(bufs)])
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(reps):
                fn(*bufs[i % len(bufs)])
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps, len(bufs)

    res = {}
    tok32 = buffers(x, (x.shape[0], KB), torch.float32, torch.float32)
    ms, n_tok = timed(dg.dg_quantize_fp8_per_token, tok32)
    del tok32
    ms_b, _ = timed(dg.dg_quantize_fp8_per_token_bf16,
                    buffers(x, (x.shape[0], KB), torch.float32, torch.bfloat16))
    ms_e, _ = timed(dg.dg_quantize_fp8_per_token_e8m0,
                    buffers(x, (x.shape[0], SP), torch.uint8, torch.float32))
    ms_w, n_blk = timed(dg.dg_quantize_fp8_per_block,
                        buffers(w, (NB, KB), torch.float32, torch.float32))
    ms_we, _ = timed(dg.dg_quantize_fp8_per_block_e8m0,
                     buffers(w, (NB, SP), torch.uint8, torch.float32))
    torch.cuda.empty_cache()
    byts = x.numel() * 5 + x.shape[0] * KB * 4
    byts_b = x.numel() * 3 + x.shape[0] * KB * 4
    byts_e = x.numel() * 5 + x.shape[0] * KB
    byts_w = w.numel() * 5 + NB * KB * 4
    byts_we = w.numel() * 5 + NB * KB

    def gbs(b, m):
        return round(b / (m * 1e-3) / 1e9, 1)

    res.update({"kernel": "quantize_per_token", "rows": int(x.shape[0]), "K": case.K,
                "rotated_buffers": n_tok,
                "us": round(ms * 1e3, 2), "GB/s": gbs(byts, ms),
                "bf16_input_us": round(ms_b * 1e3, 2), "bf16_input_GB/s": gbs(byts_b, ms_b),
                "e8m0_us": round(ms_e * 1e3, 2), "e8m0_GB/s": gbs(byts_e, ms_e),
                "per_block_rows": int(w.shape[0]), "per_block_rotated_buffers": n_blk,
                "per_block_us": round(ms_w * 1e3, 2), "per_block_GB/s": gbs(byts_w, ms_w),
                "per_block_e8m0_us": round(ms_we * 1e3, 2),
                "per_block_e8m0_GB/s": gbs(byts_we, ms_we)})
    return res


def cpu_baseline(case, target_s: float):
    """The CPU oracle (untuned) on a bounded sample of rows of the same
    workload; TFLOPS scaled to the sample's own FLOP count."""
    import numpy as np
    import oracle

    K = case.K
    e8 = case.scales == "e8m0"
    q_token = oracle.quantize_per_token_e8m0 if e8 else oracle.quantize_per_token
    q_block = oracle.quantize_per_block_e8m0 if e8 else oracle.quantize_per_block
    dense = oracle.gemm_nt_e8m0 if e8 else oracle.gemm_nt
    contiguous = oracle.gemm_grouped_contiguous_e8m0 if e8 else oracle.gemm_grouped_contiguous
    masked = oracle.gemm_grouped_masked_e8m0 if e8 else oracle.gemm_grouped_masked
    xa = case.x_a.reshape(-1, K).numpy()
    if case.form in ("dense", "dense_acc"):
        qb, sb = q_block(case.x_b.numpy())
        routed = np.arange(case.M)
    elif case.form == "contiguous":
        parts = [q_block(np.ascontiguousarray(case.x_b[g].numpy())) for g in range(case.G)]
        qb = np.stack([p[0] for p in parts]); sb = np.stack([p[1] for p in parts])
        lay = case.layout.numpy()
        routed = np.nonzero((lay >= 0) & (lay < case.G))[0]
    else:
        parts = [q_block(np.ascontiguousarray(case.x_b[g].numpy())) for g in range(case.G)]
        qb = np.stack([p[0] for p in parts]); sb = np.stack([p[1] for p in parts])
        mm = np.clip(case.masked_m.numpy(), 0, case.M)
        routed = np.concatenate([g * case.M + np.arange(mm[g]) for g in range(case.G)])
    qa, sa = q_token(xa)

    def run(rows):
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        t0 = time.perf_counter()
        if case.form == "dense":
            dense(qa, sa, qb, sb, rows=rows)
        elif case.form == "dense_acc":
            oracle.gemm_nt_acc(qa[rows], sa[rows], qb, sb, case.x_c.numpy()[rows])
        elif case.form == "contiguous":
            contiguous(qa, sa, qb, sb, case.layout.numpy(), rows=rows)
        else:
            masked(qa.reshape(case.G, case.M, K), sa.reshape(case.G, case.M, -1),
                   qb, sb, case.masked_m.numpy(), rows=rows)
        return time.perf_counter() - t0

    threads = oracle.num_threads()
    probe = routed[:max(threads, 8)]
    t_probe = run(probe)
    per_row = t_probe / len(probe)
    n_rows = int(min(len(routed), max(len(probe), target_s / max(per_row, 1e-9))))
    sample = routed[np.linspace(0, len(routed) - 1, n_rows).astype(np.int64)]
    t = run(sample)
    flop = 2.0 * len(sample) * case.N * K
    return {"value": round(flop / t / 1e12, 5), "unit": "TFLOPS", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(sample)} of {len(routed)} routed rows of {case.name} "
                      f"(all N={case.N} columns, K={K}), {t:.2f} s wall",
            "cpu_model": cpu_model(),
            "one_core": one_core_baselines()}


def cpu_model() -> str:
    """The host CPU's model name as the kernel reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def one_core_baselines(target_s: float = 3.0):
    """The oracle on one thread: the whole 128 x 512 x 512 workload, and a
    bounded sample of rows of 4096 x 7168 x 2048 (TFLOPS scaled to the
    sample's own FLOP count)."""
    import numpy as np
    import oracle
    from fp8_block_scaled_gemm_amd.inputs import workload

    threads = oracle.num_threads()
    out = {}
    oracle.set_num_threads(1)
    try:
        for name in ("dense_128x512x512", "dense_4096x7168x2048"):
            case = workload(name)
            qa, sa = oracle.quantize_per_token(case.x_a.numpy())
            qb, sb = oracle.quantize_per_block(case.x_b.numpy())
            t0 = time.perf_counter()
            oracle.gemm_nt(qa, sa, qb, sb, rows=np.arange(min(8, case.M)))
            per_row = (time.perf_counter() - t0) / min(8, case.M)
            n = int(min(case.M, max(8, target_s / max(per_row, 1e-9))))
            rows = np.linspace(0, case.M - 1, n).astype(np.int64)
            t0 = time.perf_counter()
            oracle.gemm_nt(qa, sa, qb, sb, rows=rows)
            t = time.perf_counter() - t0
            out[name] = {"TFLOPS": round(2.0 * n * case.N * case.K / t / 1e12, 6),
                         "rows": f"{n} of {case.M}", "s": round(t, 3)}
    finally:
        oracle.set_num_threads(threads)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding of this path is a design note, not a measured path",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_bytes:
        copy_reference(args.copy_bytes, args.steps, args.warmup)
        return

    import torch
    import fp8_block_scaled_gemm_amd as dg
    from fp8_block_scaled_gemm_amd.inputs import workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = workload(args.workload)
    flop, byts = algorithmic(case)
    base = make_inputs(case, dev, dg)
    torch.cuda.synchronize()

    in_bytes = sum(base[k].numel() * base[k].element_size() for k in ("A", "sa", "B", "sb", "C", "D")
                   if base[k] is not None)
    copies = max(1, -(-ROTATE_BYTES // in_bytes))
    sets = [base]
    for _ in range(copies - 1):
        sets.append({k: (v.clone() if (v is not None and k not in ("x_a", "x_b")) else v)
                     for k, v in base.items()})
    torch.cuda.synchronize()

    for i in range(args.warmup):
        gemm_call(case, dg, sets[i % copies])
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    if args.no_graph:
        # eager launches, each bracketed by events on the launch stream
        t0 = time.perf_counter()
        for i in range(args.steps):
            starts[i].record(stream)
            gemm_call(case, dg, sets[i % copies])
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kernel_ms = sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / args.steps
    else:
        # The K timed steps are one captured HIP graph (the entry points
        # allocate, synchronize and memset nothing, so they capture), which
        # takes the host's per-call launch cost out of the step rate.  The
        # per-kernel duration is the HIP-event time of that replay on the
        # launch stream over K (the graph holds one GEMM kernel per step).
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                gemm_call(case, dg, sets[i % copies])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        starts[0].record(stream)
        graph.replay()
        ends[0].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kernel_ms = starts[0].elapsed_time(ends[0]) / args.steps
        # the replay must leave what an eager call writes, bit for bit (rows
        # a call does not route stay as they were in both)
        replayed = sets[0]["D"].clone()
        gemm_call(case, dg, sets[0])
        torch.cuda.synchronize()
        if not torch.equal(replayed.view(torch.int16), sets[0]["D"].view(torch.int16)):
            raise RuntimeError("graph replay of the GEMM differs from an eager call")

    ms_per_step = wall * 1e3 / args.steps
    value = flop / (ms_per_step * 1e-3) / 1e12
    intensity = flop / byts
    if intensity >= PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = flop / (kernel_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4)}
    else:
        achieved = byts / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["traffic"] = traffic_from_profiles(case.name)
    roof["kernel"] = f"gemm_kernel ({case.form}, {case.scales} scales)"
    roof["kernel_us"] = round(kernel_ms * 1e3, 2)
    roof["algorithmic_flop"] = flop
    roof["algorithmic_bytes"] = byts

    warm = None if args.no_graph else same_buffer_rate(case, dg, sets[0], args.steps, flop)
    quant = time_quantize(dg, base, case)
    cpu = None if args.no_cpu_baseline else cpu_baseline(case, args.cpu_seconds)

    line = {
        "metric": "FP8 block-scaled GEMM TFLOPS (and % of FP8 MFMA peak) at M=4096,N=7168,K=2048",
        "value": round(value, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": case.name, "form": case.form, "scales": case.scales,
                   "M": case.M, "N": case.N,
                   "K": case.K, "G": case.G, "valid_rows": case.valid_rows,
                   "rotated_input_sets": copies},
        "roofline": roof,
        "cpu_baseline": cpu,
        "same_buffer": warm,
        "quantize": quant,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
