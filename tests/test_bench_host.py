"""Host logic of bench.py (CPU only): the one-GPU guard, the algorithmic
work figures the roofline divides by, and the gate that keeps a committed
HBM-traffic figure out of the report once the kernel source has changed."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from fp8_block_scaled_gemm_amd.inputs import dense_case, masked_case  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_work_of_the_default_workload():
    # M=4096, N=7168, K=2048: K/128 = 16 scale columns, N/128 = 56 scale rows
    case = dense_case(4096, 7168, 2048, seed=2)
    flop, byts = bench.algorithmic(case)
    assert flop == 2 * 4096 * 7168 * 2048 == 120259084288
    a_codes, b_codes = 4096 * 2048, 7168 * 2048
    scales = 4 * (4096 * 16 + 56 * 16)
    d_bf16 = 2 * 4096 * 7168
    assert byts == a_codes + b_codes + scales + d_bf16 == 82054656


def test_algorithmic_work_counts_routed_rows_and_used_groups_only():
    # 4 slabs of 64 rows, N=256, K=384; masked_m = 0, 10, 64, 100 (clamped
    # to 64): 138 routed rows, 3 groups whose B is read
    case = masked_case(4, 64, 256, 384, seed=3, masked=[0, 10, 64, 100])
    flop, byts = bench.algorithmic(case)
    rows, groups, KB, NB = 138, 3, 3, 2
    assert flop == 2 * rows * 256 * 384
    assert byts == rows * 384 + groups * 256 * 384 + 4 * (rows * KB + groups * NB * KB) + 2 * rows * 256


def _write_traffic(root, workload, src_hash, nbytes):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", f"traffic_gemm_{workload}.txt"), "w") as f:
        f.write(f"kernel_source_sha256_16: {src_hash}\nhbm_bytes_per_launch: {nbytes}\n")


def test_traffic_is_reported_only_for_the_profiled_kernel_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0123456789abcdef")
    assert bench.traffic_from_profiles("w") is None            # no summary
    _write_traffic(str(tmp_path), "w", "0123456789abcdef", 1.5e8)
    assert bench.traffic_from_profiles("w") == pytest.approx(1.5e8)
    _write_traffic(str(tmp_path), "w", "fedcba9876543210", 1.5e8)
    assert bench.traffic_from_profiles("w") is None            # taken on other source


def test_kernel_source_hash_covers_the_gemm_sources():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
