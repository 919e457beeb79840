"""MI355X (gfx950) FP8 block-scaled NT GEMM: thin Python binding.

Every function here has the name of the C-ABI entry point it calls
(include/dg_fp8.h) and only marshals arguments: it checks torch tensor
dtypes, shapes and devices, passes raw device pointers and the current HIP
stream, and raises ``DGError`` on a nonzero status.  All arithmetic runs in
the HIP kernels of ``libdgfp8.so``; there is no CPU fallback, and importing a
function fails loudly when the library has not been built
(``python -m fp8_block_scaled_gemm_amd.build``).

Tensor conventions: e4m3 codes are ``torch.uint8`` (or
``torch.float8_e4m3fn``, viewed as bytes), scales ``torch.float32``, group
arrays ``torch.int32``, and D is ``torch.bfloat16`` (or ``torch.uint16`` /
``torch.int16`` holding bf16 bit patterns).  All tensors live on the GPU,
are contiguous and 16-byte aligned.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "DGError", "library_path", "load_library",
    "dg_fp8_gemm_nt", "dg_fp8_gemm_nt_acc", "dg_fp8_gemm_grouped_contiguous",
    "dg_fp8_gemm_grouped_masked",
    "dg_quantize_fp8_per_token", "dg_quantize_fp8_per_token_bf16", "dg_quantize_fp8_per_block",
    "dg_fp8_gemm_nt_e8m0", "dg_fp8_gemm_grouped_contiguous_e8m0", "dg_fp8_gemm_grouped_masked_e8m0",
    "dg_quantize_fp8_per_token_e8m0", "dg_quantize_fp8_per_block_e8m0", "e8m0_pitch",
    "dg_status_string",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdgfp8.so")
_lib = None

DG_OK = 0


class DGError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed with status {status}: {dg_status_string(status)}")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libdgfp8.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m fp8_block_scaled_gemm_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    for name, args in [
        ("dg_fp8_gemm_nt", [p, p, p, p, p, i64, i64, i64, p]),
        ("dg_fp8_gemm_nt_acc", [p, p, p, p, p, p, i64, i64, i64, p]),
        ("dg_fp8_gemm_grouped_contiguous", [p, p, p, p, p, p, i64, i64, i64, i64, p]),
        ("dg_fp8_gemm_grouped_masked", [p, p, p, p, p, p, i64, i64, i64, i64, p]),
        ("dg_quantize_fp8_per_token", [p, i64, i64, p, p, p]),
        ("dg_quantize_fp8_per_token_bf16", [p, i64, i64, p, p, p]),
        ("dg_quantize_fp8_per_block", [p, i64, i64, p, p, p]),
        ("dg_fp8_gemm_nt_e8m0", [p, p, p, p, p, i64, i64, i64, p]),
        ("dg_fp8_gemm_grouped_contiguous_e8m0", [p, p, p, p, p, p, i64, i64, i64, i64, p]),
        ("dg_fp8_gemm_grouped_masked_e8m0", [p, p, p, p, p, p, i64, i64, i64, i64, p]),
        ("dg_quantize_fp8_per_token_e8m0", [p, i64, i64, p, p, p]),
        ("dg_quantize_fp8_per_block_e8m0", [p, i64, i64, p, p, p]),
    ]:
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.dg_status_string.argtypes = [ctypes.c_int]
    lib.dg_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def dg_status_string(status: int) -> str:
    return load_library().dg_status_string(int(status)).decode()


def _stream_ptr(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _bytes(t: torch.Tensor, what: str) -> torch.Tensor:
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"{what} must be uint8 or float8_e4m3fn codes, got {t.dtype}")
    return t


def _check(t: torch.Tensor, what: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{what} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")


_D_TYPES = (torch.bfloat16, torch.uint16, torch.int16)


def _device_of(*tensors) -> torch.device:
    """The one device all of a call's tensors live on; a call whose tensors
    span devices is refused (the kernels would read another GPU's memory)."""
    dev = tensors[0].device
    for t in tensors[1:]:
        if t.device != dev:
            raise ValueError(f"all tensors of a call must be on one device, got {dev} and {t.device}")
    return dev


def _call(dev: torch.device, name: str, *args):
    # the library launches on the current device, with the stream passed in
    with torch.cuda.device(dev):
        status = getattr(load_library(), name)(*args)
    if status != DG_OK:
        raise DGError(name, status)


def dg_fp8_gemm_nt(A, sa, B, sb, D):
    """Dense: D[M][N] = bf16(sum_kb sa[m,kb]*sb[n/128,kb] * A_blk @ B_blk^T)."""
    A, B = _bytes(A, "A"), _bytes(B, "B")
    M, K = A.shape
    N = B.shape[0]
    KB, NB = K // 128, (N + 127) // 128
    _check(A, "A"); _check(B, "B", shape=(N, K))
    _check(sa, "sa", torch.float32, (M, KB)); _check(sb, "sb", torch.float32, (NB, KB))
    _check(D, "D", _D_TYPES, (M, N))
    _call(_device_of(A, sa, B, sb, D), "dg_fp8_gemm_nt",
          A.data_ptr(), sa.data_ptr(), B.data_ptr(), sb.data_ptr(),
          D.data_ptr(), M, N, K, _stream_ptr(D))
    return D


def dg_fp8_gemm_nt_acc(A, sa, B, sb, C, D):
    """Dense with an fp32 addend: D[M][N] = bf16(C + the dense sum)."""
    A, B = _bytes(A, "A"), _bytes(B, "B")
    M, K = A.shape
    N = B.shape[0]
    KB, NB = K // 128, (N + 127) // 128
    _check(A, "A"); _check(B, "B", shape=(N, K))
    _check(sa, "sa", torch.float32, (M, KB)); _check(sb, "sb", torch.float32, (NB, KB))
    _check(C, "C", torch.float32, (M, N))
    _check(D, "D", _D_TYPES, (M, N))
    _call(_device_of(A, sa, B, sb, C, D), "dg_fp8_gemm_nt_acc",
          A.data_ptr(), sa.data_ptr(), B.data_ptr(), sb.data_ptr(),
          C.data_ptr(), D.data_ptr(), M, N, K, _stream_ptr(D))
    return D


def dg_fp8_gemm_grouped_contiguous(A, sa, B, sb, D, grouped_layout):
    """Contiguous-grouped: row r of D uses B[grouped_layout[r]]; rows whose
    id is outside [0, G) are not written."""
    A, B = _bytes(A, "A"), _bytes(B, "B")
    M_sum, K = A.shape
    G, N, _ = B.shape
    KB, NB = K // 128, (N + 127) // 128
    _check(A, "A"); _check(B, "B", shape=(G, N, K))
    _check(sa, "sa", torch.float32, (M_sum, KB)); _check(sb, "sb", torch.float32, (G, NB, KB))
    _check(D, "D", _D_TYPES, (M_sum, N))
    _check(grouped_layout, "grouped_layout", torch.int32, (M_sum,))
    _call(_device_of(A, sa, B, sb, D, grouped_layout), "dg_fp8_gemm_grouped_contiguous",
          A.data_ptr(), sa.data_ptr(), B.data_ptr(),
          sb.data_ptr(), D.data_ptr(), grouped_layout.data_ptr(), M_sum, N, K, G, _stream_ptr(D))
    return D


def dg_fp8_gemm_grouped_masked(A, sa, B, sb, D, masked_m):
    """Masked-grouped: rows r < masked_m[g] of slab g use B[g]; other rows
    of D are not written."""
    A, B = _bytes(A, "A"), _bytes(B, "B")
    G, M_max, K = A.shape
    _, N, _ = B.shape
    KB, NB = K // 128, (N + 127) // 128
    _check(A, "A"); _check(B, "B", shape=(G, N, K))
    _check(sa, "sa", torch.float32, (G, M_max, KB)); _check(sb, "sb", torch.float32, (G, NB, KB))
    _check(D, "D", _D_TYPES, (G, M_max, N))
    _check(masked_m, "masked_m", torch.int32, (G,))
    _call(_device_of(A, sa, B, sb, D, masked_m), "dg_fp8_gemm_grouped_masked",
          A.data_ptr(), sa.data_ptr(), B.data_ptr(),
          sb.data_ptr(), D.data_ptr(), masked_m.data_ptr(), G, M_max, N, K, _stream_ptr(D))
    return D


def dg_quantize_fp8_per_token(x, q=None, s=None):
    """x[M][K] fp32 -> (q[M][K] uint8 e4m3 codes, s[M][K/128] fp32)."""
    _check(x, "x", torch.float32)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    q = _bytes(q, "q")
    _check(q, "q", shape=(M, K)); _check(s, "s", torch.float32, (M, K // 128))
    _call(_device_of(x, q, s), "dg_quantize_fp8_per_token",
          x.data_ptr(), M, K, q.data_ptr(), s.data_ptr(),
          _stream_ptr(x))
    return q, s


def dg_quantize_fp8_per_token_bf16(x, q=None, s=None):
    """x[M][K] bf16 -> (q[M][K] uint8 e4m3 codes, s[M][K/128] fp32)."""
    _check(x, "x", torch.bfloat16)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    q = _bytes(q, "q")
    _check(q, "q", shape=(M, K)); _check(s, "s", torch.float32, (M, K // 128))
    _call(_device_of(x, q, s), "dg_quantize_fp8_per_token_bf16",
          x.data_ptr(), M, K, q.data_ptr(), s.data_ptr(),
          _stream_ptr(x))
    return q, s


def dg_quantize_fp8_per_block(x, q=None, s=None):
    """x[N][K] fp32 -> (q[N][K] uint8, s[ceil(N/128)][K/128] fp32)."""
    _check(x, "x", torch.float32)
    N, K = x.shape
    NB = (N + 127) // 128
    if q is None:
        q = torch.empty((N, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((NB, K // 128), dtype=torch.float32, device=x.device)
    q = _bytes(q, "q")
    _check(q, "q", shape=(N, K)); _check(s, "s", torch.float32, (NB, K // 128))
    _call(_device_of(x, q, s), "dg_quantize_fp8_per_block",
          x.data_ptr(), N, K, q.data_ptr(), s.data_ptr(),
          _stream_ptr(x))
    return q, s


# ------------------------------------------------ power-of-two (E8M0) scales

def e8m0_pitch(kb: int) -> int:
    """Bytes per row of E8M0 scales: K/128 rounded up to a multiple of 4."""
    return (kb + 3) // 4 * 4


def dg_fp8_gemm_nt_e8m0(A, sa, B, sb, D):
    """Dense form with E8M0 scales sa[M][SP], sb[ceil(N/128)][SP] (uint8)."""
    A, B = _bytes(A, "A"), _bytes(B, "B")
    M, K = A.shape
    N = B.shape[0]
    SP, NB = e8m0_pitch(K // 128), (N + 127) // 128
    _check(A, "A"); _check(B, "B", shape=(N, K))
    _check(sa, "sa", torch.uint8, (M, SP)); _check(sb, "sb", torch.uint8, (NB, SP))
    _check(D, "D", _D_TYPES, (M, N))
    _call(_device_of(A, sa, B, sb, D), "dg_fp8_gemm_nt_e8m0",
          A.data_ptr(), sa.data_ptr(), B.data_ptr(), sb.data_ptr(),
          D.data_ptr(), M, N, K, _stream_ptr(D))
    return D


def dg_fp8_gemm_grouped_contiguous_e8m0(A, sa, B, sb, D, grouped_layout):
    """Contiguous-grouped form with E8M0 scales sa[M_sum][SP], sb[G][NB][SP]."""
    A, B = _bytes(A, "A"), _bytes(B, "B")
    M_sum, K = A.shape
    G, N, _ = B.shape
    SP, NB = e8m0_pitch(K // 128), (N + 127) // 128
    _check(A, "A"); _check(B, "B", shape=(G, N, K))
    _check(sa, "sa", torch.uint8, (M_sum, SP)); _check(sb, "sb", torch.uint8, (G, NB, SP))
    _check(D, "D", _D_TYPES, (M_sum, N))
    _check(grouped_layout, "grouped_layout", torch.int32, (M_sum,))
    _call(_device_of(A, sa, B, sb, D, grouped_layout), "dg_fp8_gemm_grouped_contiguous_e8m0",
          A.data_ptr(), sa.data_ptr(), B.data_ptr(),
          sb.data_ptr(), D.data_ptr(), grouped_layout.data_ptr(), M_sum, N, K, G, _stream_ptr(D))
    return D


def dg_fp8_gemm_grouped_masked_e8m0(A, sa, B, sb, D, masked_m):
    """Masked-grouped form with E8M0 scales sa[G][M_max][SP], sb[G][NB][SP]."""
    A, B = _bytes(A, "A"), _bytes(B, "B")
    G, M_max, K = A.shape
    _, N, _ = B.shape
    SP, NB = e8m0_pitch(K // 128), (N + 127) // 128
    _check(A, "A"); _check(B, "B", shape=(G, N, K))
    _check(sa, "sa", torch.uint8, (G, M_max, SP)); _check(sb, "sb", torch.uint8, (G, NB, SP))
    _check(D, "D", _D_TYPES, (G, M_max, N))
    _check(masked_m, "masked_m", torch.int32, (G,))
    _call(_device_of(A, sa, B, sb, D, masked_m), "dg_fp8_gemm_grouped_masked_e8m0",
          A.data_ptr(), sa.data_ptr(), B.data_ptr(),
          sb.data_ptr(), D.data_ptr(), masked_m.data_ptr(), G, M_max, N, K, _stream_ptr(D))
    return D


def dg_quantize_fp8_per_token_e8m0(x, q=None, s=None):
    """x[M][K] fp32 -> (q[M][K] uint8 codes, s[M][SP] uint8 E8M0 exponents).
    A newly allocated s has zero padding bytes; the kernel never writes them."""
    _check(x, "x", torch.float32)
    M, K = x.shape
    SP = e8m0_pitch(K // 128)
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.zeros((M, SP), dtype=torch.uint8, device=x.device)
    q = _bytes(q, "q")
    _check(q, "q", shape=(M, K)); _check(s, "s", torch.uint8, (M, SP))
    _call(_device_of(x, q, s), "dg_quantize_fp8_per_token_e8m0",
          x.data_ptr(), M, K, q.data_ptr(), s.data_ptr(),
          _stream_ptr(x))
    return q, s


def dg_quantize_fp8_per_block_e8m0(x, q=None, s=None):
    """x[N][K] fp32 -> (q[N][K] uint8, s[ceil(N/128)][SP] uint8 E8M0 exponents)."""
    _check(x, "x", torch.float32)
    N, K = x.shape
    NB, SP = (N + 127) // 128, e8m0_pitch(K // 128)
    if q is None:
        q = torch.empty((N, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.zeros((NB, SP), dtype=torch.uint8, device=x.device)
    q = _bytes(q, "q")
    _check(q, "q", shape=(N, K)); _check(s, "s", torch.uint8, (NB, SP))
    _call(_device_of(x, q, s), "dg_quantize_fp8_per_block_e8m0",
          x.data_ptr(), N, K, q.data_ptr(), s.data_ptr(),
          _stream_ptr(x))
    return q, s
