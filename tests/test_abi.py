"""CPU tests of the C-ABI library: it loads, exports every function the
header declares, and rejects bad arguments on the host before touching the
GPU (these calls return from host-side checks, so no GPU is needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg_fp8.h")

DG_OK, DG_ERR_NULL, DG_ERR_SHAPE, DG_ERR_ALIGN = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import fp8_block_scaled_gemm_amd as dg
    path = dg.library_path()
    if not os.path.exists(path):
        from fp8_block_scaled_gemm_amd import build
        build.build()
    return dg.load_library()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "dg_fp8_gemm_nt", "dg_fp8_gemm_nt_acc", "dg_fp8_gemm_grouped_contiguous",
        "dg_fp8_gemm_grouped_masked", "dg_quantize_fp8_per_token", "dg_quantize_fp8_per_token_bf16",
        "dg_quantize_fp8_per_block", "dg_status_string",
        "dg_fp8_gemm_nt_e8m0", "dg_fp8_gemm_grouped_contiguous_e8m0",
        "dg_fp8_gemm_grouped_masked_e8m0", "dg_quantize_fp8_per_token_e8m0",
        "dg_quantize_fp8_per_block_e8m0"])


def test_library_exports_every_declared_symbol(lib):
    import fp8_block_scaled_gemm_amd as dg
    out = subprocess.run(["nm", "-D", "--defined-only", dg.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_library_has_gfx950_code_object():
    import fp8_block_scaled_gemm_amd as dg
    data = open(dg.library_path(), "rb").read()
    assert b"gfx950" in data


def test_status_strings(lib):
    import fp8_block_scaled_gemm_amd as dg
    for s in range(6):
        assert isinstance(dg.dg_status_string(s), str) and dg.dg_status_string(s)
    assert dg.dg_status_string(0) == "ok"


FAKE = 0x10000  # 16-byte aligned, never dereferenced: the checks reject first


def _gemm_nt(lib, A=FAKE, sa=FAKE, B=FAKE, sb=FAKE, D=FAKE, M=4, N=8, K=128):
    return lib.dg_fp8_gemm_nt(A, sa, B, sb, D, M, N, K, None)


def test_dense_rejects_bad_shapes(lib):
    assert _gemm_nt(lib, K=100) == DG_ERR_SHAPE
    assert _gemm_nt(lib, K=0) == DG_ERR_SHAPE
    assert _gemm_nt(lib, N=12) == DG_ERR_SHAPE
    assert _gemm_nt(lib, N=0) == DG_ERR_SHAPE
    assert _gemm_nt(lib, M=-1) == DG_ERR_SHAPE
    assert _gemm_nt(lib, M=1 << 40, N=1 << 30) == DG_ERR_SHAPE
    assert _gemm_nt(lib, K=1 << 24) == DG_ERR_SHAPE          # 32-bit tile offsets


def test_dense_rejects_null_and_misaligned(lib):
    assert _gemm_nt(lib, A=None) == DG_ERR_NULL
    assert _gemm_nt(lib, D=None) == DG_ERR_NULL
    assert _gemm_nt(lib, sb=FAKE + 4) == DG_ERR_ALIGN
    assert _gemm_nt(lib, B=FAKE + 8) == DG_ERR_ALIGN


def test_zero_rows_is_a_no_op(lib):
    assert _gemm_nt(lib, A=None, sa=None, D=None, M=0) == DG_OK
    assert lib.dg_fp8_gemm_grouped_contiguous(None, None, None, None, None, None,
                                              0, 8, 128, 2, None) == DG_OK
    assert lib.dg_fp8_gemm_grouped_masked(None, None, None, None, None, None,
                                          3, 0, 8, 128, None) == DG_OK
    assert lib.dg_quantize_fp8_per_token(None, 0, 128, None, None, None) == DG_OK
    assert lib.dg_quantize_fp8_per_token_bf16(None, 0, 128, None, None, None) == DG_OK
    assert lib.dg_quantize_fp8_per_block(None, 0, 128, None, None, None) == DG_OK


def test_acc_rejections(lib):
    f = lib.dg_fp8_gemm_nt_acc
    assert f(None, None, None, None, None, None, 0, 8, 128, None) == DG_OK          # M = 0
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 8, 128, None) == DG_ERR_NULL     # C
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE, 4, 8, 128, None) == DG_ERR_ALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 12, 128, None) == DG_ERR_SHAPE  # N % 8
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 100, None) == DG_ERR_SHAPE   # K % 128
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1 << 22, 128, None) == DG_ERR_SHAPE  # N


def test_e8m0_rejections(lib):
    """The exponent-scale entry points apply the same host checks."""
    f = lib.dg_fp8_gemm_nt_e8m0
    assert f(None, None, None, None, None, 0, 8, 128, None) == DG_OK                # M = 0
    assert f(FAKE, None, FAKE, FAKE, FAKE, 4, 8, 128, None) == DG_ERR_NULL
    assert f(FAKE, FAKE + 4, FAKE, FAKE, FAKE, 4, 8, 128, None) == DG_ERR_ALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 12, 128, None) == DG_ERR_SHAPE       # N % 8
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 200, None) == DG_ERR_SHAPE        # K % 128
    c = lib.dg_fp8_gemm_grouped_contiguous_e8m0
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 8, 128, 2, None) == DG_ERR_SHAPE
    assert c(FAKE, FAKE, FAKE, FAKE, FAKE, None, 128, 8, 128, 2, None) == DG_ERR_NULL
    m = lib.dg_fp8_gemm_grouped_masked_e8m0
    assert m(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 16, 8, 128, None) == DG_ERR_SHAPE
    assert m(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0, 8, 128, None) == DG_OK      # no rows
    for q in (lib.dg_quantize_fp8_per_token_e8m0, lib.dg_quantize_fp8_per_block_e8m0):
        assert q(FAKE, 4, 100, FAKE, FAKE, None) == DG_ERR_SHAPE
        assert q(FAKE, 4, 128, FAKE, None, None) == DG_ERR_NULL
        assert q(FAKE, 0, 128, None, None, None) == DG_OK
    assert lib.dg_quantize_fp8_per_block_e8m0(FAKE, 128 * 65536, 128, FAKE, FAKE, None) == DG_ERR_SHAPE


def test_grouped_rejections(lib):
    f = lib.dg_fp8_gemm_grouped_contiguous
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 8, 128, 2, None) == DG_ERR_SHAPE  # M_sum % 128
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 128, 8, 128, 0, None) == DG_ERR_SHAPE  # G < 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, 128, 8, 128, 2, None) == DG_ERR_NULL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4, 128, 8, 128, 2, None) == DG_ERR_ALIGN
    g = lib.dg_fp8_gemm_grouped_masked
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 16, 8, 128, None) == DG_ERR_SHAPE    # G < 1
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, -1, 8, 128, None) == DG_ERR_SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 16, 8, 96, None) == DG_ERR_SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, None, 2, 16, 8, 128, None) == DG_ERR_NULL


def test_quantize_rejections(lib):
    assert lib.dg_quantize_fp8_per_token(FAKE, 4, 100, FAKE, FAKE, None) == DG_ERR_SHAPE
    assert lib.dg_quantize_fp8_per_token(FAKE, -1, 128, FAKE, FAKE, None) == DG_ERR_SHAPE
    assert lib.dg_quantize_fp8_per_token(None, 4, 128, FAKE, FAKE, None) == DG_ERR_NULL
    assert lib.dg_quantize_fp8_per_token_bf16(FAKE, 4, 100, FAKE, FAKE, None) == DG_ERR_SHAPE
    assert lib.dg_quantize_fp8_per_token_bf16(FAKE, 4, 128, None, FAKE, None) == DG_ERR_NULL
    assert lib.dg_quantize_fp8_per_token_bf16(FAKE + 2, 4, 128, FAKE, FAKE, None) == DG_ERR_ALIGN
    assert lib.dg_quantize_fp8_per_block(FAKE, 4, 128, FAKE + 1, FAKE, None) == DG_ERR_ALIGN
    assert lib.dg_quantize_fp8_per_block(FAKE, 4, 0, FAKE, FAKE, None) == DG_ERR_SHAPE


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import fp8_block_scaled_gemm_amd as dg
    monkeypatch.setattr(dg, "_lib", None)
    monkeypatch.setattr(dg, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        dg.load_library()


def test_product_path_does_not_touch_the_oracle():
    """The package's sources never import or load the CPU oracle."""
    pkg = os.path.join(ROOT, "fp8_block_scaled_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "liborc" not in text, f


def test_binding_refuses_tensors_on_two_devices():
    import torch
    import fp8_block_scaled_gemm_amd as dg
    a, b = torch.zeros(4), torch.zeros(4, device="meta")
    assert dg._device_of(a, a) == a.device
    with pytest.raises(ValueError, match="one device"):
        dg._device_of(a, b)


def test_launch_limits_are_shape_errors(lib):
    """Sizes that pass the per-call rules but would need more than 2^31
    workgroups are rejected as DG_ERR_SHAPE before anything is enqueued."""
    g = lib.dg_fp8_gemm_grouped_masked
    # 2^20 slabs of one 256-row block times 4096 column blocks: 2^32 tiles
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 256, 1 << 20, 128, None) == DG_ERR_SHAPE
    # 2^37 (row, K block) pairs over 32 per workgroup: 2^32 workgroups
    assert lib.dg_quantize_fp8_per_token(FAKE, 1 << 30, 1 << 14, FAKE, FAKE, None) == DG_ERR_SHAPE
    assert lib.dg_quantize_fp8_per_token_e8m0(FAKE, 1 << 30, 1 << 14, FAKE, FAKE, None) == DG_ERR_SHAPE
    # dense: 2^23 x 2^12 tiles of 256 x 256
    assert _gemm_nt(lib, M=(1 << 31) - 1, N=1 << 20) == DG_ERR_SHAPE
