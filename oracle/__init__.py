"""CPU oracle for the FP8 block-scaled NT GEMM (test infrastructure).

Test infrastructure only: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product library and
its Python binding never import this package, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over output
rows); this module compiles it with gcc and marshals numpy arrays into it.
What each function computes, and the passage of DeepGEMM's ``fp8_gemm.cuh``
it follows, is stated in the C source next to each function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liborc.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liborc.so with gcc (no fused multiply-add)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", _SRC, "-o", _LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_value.restype = ctypes.c_double
    lib.orc_e4m3_from_float.argtypes = [ctypes.c_float]
    lib.orc_e4m3_from_float.restype = ctypes.c_uint8
    lib.orc_bf16_from_double.argtypes = [ctypes.c_double]
    lib.orc_bf16_from_double.restype = ctypes.c_uint16
    lib.orc_quantize_per_token.argtypes = [p, i64, i64, p, p]
    lib.orc_quantize_per_token.restype = None
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_value.restype = ctypes.c_float
    lib.orc_quantize_per_token_bf16.argtypes = [p, i64, i64, p, p]
    lib.orc_quantize_per_token_bf16.restype = None
    lib.orc_quantize_per_block.argtypes = [p, i64, i64, p, p]
    lib.orc_quantize_per_block.restype = None
    lib.orc_e8m0_value.argtypes = [ctypes.c_uint8]
    lib.orc_e8m0_value.restype = ctypes.c_double
    lib.orc_e8m0_exponent.argtypes = [ctypes.c_float]
    lib.orc_e8m0_exponent.restype = ctypes.c_int
    lib.orc_quantize_per_token_e8m0.argtypes = [p, i64, i64, p, p]
    lib.orc_quantize_per_token_e8m0.restype = None
    lib.orc_quantize_per_block_e8m0.argtypes = [p, i64, i64, p, p]
    lib.orc_quantize_per_block_e8m0.restype = None
    lib.orc_gemm_nt.argtypes = [p, p, p, p, p, i64, i64, i64]
    lib.orc_gemm_nt.restype = None
    lib.orc_gemm_nt_acc.argtypes = [p, p, p, p, p, p, i64, i64, i64]
    lib.orc_gemm_nt_acc.restype = None
    lib.orc_gemm_nt_rows.argtypes = [p, p, p, p, i64, i64, i64, p, i64, p]
    lib.orc_gemm_nt_rows.restype = None
    lib.orc_gemm_grouped_contiguous.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64]
    lib.orc_gemm_grouped_contiguous.restype = None
    lib.orc_gemm_grouped_contiguous_rows.argtypes = [p, p, p, p, p, i64, i64, i64, i64, p, i64, p]
    lib.orc_gemm_grouped_contiguous_rows.restype = None
    lib.orc_gemm_grouped_masked.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64]
    lib.orc_gemm_grouped_masked.restype = None
    lib.orc_gemm_grouped_masked_rows.argtypes = [p, p, p, p, p, i64, i64, i64, i64, p, i64, p]
    lib.orc_gemm_grouped_masked_rows.restype = None
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_set_num_threads.argtypes = [ctypes.c_int]
    lib.orc_set_num_threads.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, f"expected {dtype}, got {a.dtype}"
    return a


# ----------------------------------------------------------------- scalars

def e4m3_value(code: int) -> float:
    """OCP E4M3FN decode of one byte code."""
    return _load().orc_e4m3_value(int(code) & 0xFF)


def e4m3_table() -> np.ndarray:
    """fp64 value of each of the 256 codes (NaN for the two NaN codes)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_from_float(v: float) -> int:
    """Round an fp32 value to e4m3: nearest, ties to even, saturating at 448."""
    return int(_load().orc_e4m3_from_float(float(np.float32(v))))


def bf16_from_double(v: float) -> int:
    """Round an fp64 value to a bf16 bit pattern: nearest, ties to even."""
    return int(_load().orc_bf16_from_double(float(v)))


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's later parallel loops (1 times one core)."""
    _load().orc_set_num_threads(int(n))


# ---------------------------------------------------------------- quantize

def quantize_per_token(x: np.ndarray):
    """x[M][K] fp32 -> (q[M][K] uint8 e4m3 codes, s[M][K/128] fp32)."""
    x = _c(x, np.float32)
    M, K = x.shape
    assert K % 128 == 0
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // 128), dtype=np.float32)
    _load().orc_quantize_per_token(_ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def bf16_value(bits: int) -> float:
    """The fp32 value of a bf16 bit pattern."""
    return float(_load().orc_bf16_value(int(bits)))


def quantize_per_token_bf16(x_bits: np.ndarray):
    """x[M][K] bf16 bit patterns (uint16) -> (q[M][K] uint8, s[M][K/128] fp32)."""
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    assert K % 128 == 0
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // 128), dtype=np.float32)
    _load().orc_quantize_per_token_bf16(_ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def quantize_per_block(x: np.ndarray):
    """x[N][K] fp32 -> (q[N][K] uint8, s[ceil(N/128)][K/128] fp32)."""
    x = _c(x, np.float32)
    N, K = x.shape
    assert K % 128 == 0
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty(((N + 127) // 128, K // 128), dtype=np.float32)
    _load().orc_quantize_per_block(_ptr(x), N, K, _ptr(q), _ptr(s))
    return q, s


# ------------------------------------------------------ power-of-two scales

def e8m0_pitch(kb: int) -> int:
    """Bytes per row of exponent scales: K/128 rounded up to a multiple of 4."""
    return (kb + 3) // 4 * 4


def e8m0_value(b: int) -> float:
    """2^(b - 127) for an E8M0 byte b; NaN for 255."""
    return float(_load().orc_e8m0_value(int(b) & 0xFF))


def e8m0_exponent(amax: float) -> int:
    """Smallest e >= -127 with amax <= 448 * 2^e (amax taken as fp32)."""
    return int(_load().orc_e8m0_exponent(float(np.float32(amax))))


def e8m0_decode(s: np.ndarray) -> np.ndarray:
    """fp32 values of E8M0 bytes (exact: 2^-127 is an fp32 subnormal), with
    the 256 values taken from the C decode above."""
    table = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64).astype(np.float32)
    return table[np.asarray(s, dtype=np.uint8)]


def quantize_per_token_e8m0(x: np.ndarray):
    """x[M][K] fp32 -> (q[M][K] uint8 codes, s[M][KBp] uint8 exponents);
    padding bytes of s are zero."""
    x = _c(x, np.float32)
    M, K = x.shape
    assert K % 128 == 0
    q = np.empty((M, K), dtype=np.uint8)
    s = np.zeros((M, e8m0_pitch(K // 128)), dtype=np.uint8)
    _load().orc_quantize_per_token_e8m0(_ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def quantize_per_block_e8m0(x: np.ndarray):
    """x[N][K] fp32 -> (q[N][K] uint8, s[ceil(N/128)][KBp] uint8 exponents)."""
    x = _c(x, np.float32)
    N, K = x.shape
    assert K % 128 == 0
    q = np.empty((N, K), dtype=np.uint8)
    s = np.zeros(((N + 127) // 128, e8m0_pitch(K // 128)), dtype=np.uint8)
    _load().orc_quantize_per_block_e8m0(_ptr(x), N, K, _ptr(q), _ptr(s))
    return q, s


def _e8m0_scales(s: np.ndarray, KB: int) -> np.ndarray:
    return np.ascontiguousarray(e8m0_decode(np.asarray(s)[..., :KB]))


def gemm_nt_e8m0(A, sa, B, sb, rows=None):
    """Dense form with exponent-byte scales sa[M][KBp], sb[ceil(N/128)][KBp]:
    the definition of gemm_nt with sa, sb replaced by their powers of two."""
    KB = A.shape[-1] // 128
    return gemm_nt(A, _e8m0_scales(sa, KB), B, _e8m0_scales(sb, KB), rows=rows)


def gemm_grouped_contiguous_e8m0(A, sa, B, sb, layout, rows=None):
    """Contiguous-grouped form with exponent-byte scales."""
    KB = A.shape[-1] // 128
    return gemm_grouped_contiguous(A, _e8m0_scales(sa, KB), B, _e8m0_scales(sb, KB), layout,
                                   rows=rows)


def gemm_grouped_masked_e8m0(A, sa, B, sb, masked_m, rows=None):
    """Masked-grouped form with exponent-byte scales."""
    KB = A.shape[-1] // 128
    return gemm_grouped_masked(A, _e8m0_scales(sa, KB), B, _e8m0_scales(sb, KB), masked_m,
                               rows=rows)


# -------------------------------------------------------------------- GEMM

def gemm_nt(A, sa, B, sb, D=None, rows=None):
    """Dense form.  A[M][K], sa[M][K/128], B[N][K], sb[ceil(N/128)][K/128]
    (uint8 codes / fp32 scales) -> D[M][N] as uint16 bf16 bit patterns.

    With ``rows`` (int64 indices) only those rows are computed and the
    result has shape [len(rows)][N]."""
    A = _c(A, np.uint8); sa = _c(sa, np.float32); B = _c(B, np.uint8); sb = _c(sb, np.float32)
    M, K = A.shape
    N = B.shape[0]
    assert K % 128 == 0 and B.shape[1] == K
    assert sa.shape == (M, K // 128) and sb.shape == ((N + 127) // 128, K // 128)
    lib = _load()
    if rows is not None:
        rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < M)
        out = np.full((rows.size, N), 0xFFFF, dtype=np.uint16)
        lib.orc_gemm_nt_rows(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), M, N, K,
                             _ptr(rows), rows.size, _ptr(out))
        return out
    if D is None:
        D = np.full((M, N), 0xFFFF, dtype=np.uint16)
    assert D.dtype == np.uint16 and D.shape == (M, N) and D.flags["C_CONTIGUOUS"]
    lib.orc_gemm_nt(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(D), M, N, K)
    return D



def gemm_nt_acc(A, sa, B, sb, C):
    """Dense form with an fp32 addend: D = bf16(C + the dense sum), C[M][N]
    fp32 joining the fp64 sum before the single rounding."""
    A = _c(A, np.uint8); sa = _c(sa, np.float32); B = _c(B, np.uint8); sb = _c(sb, np.float32)
    C = _c(C, np.float32)
    M, K = A.shape
    N = B.shape[0]
    assert K % 128 == 0 and B.shape[1] == K and C.shape == (M, N)
    assert sa.shape == (M, K // 128) and sb.shape == ((N + 127) // 128, K // 128)
    D = np.full((M, N), 0xFFFF, dtype=np.uint16)
    _load().orc_gemm_nt_acc(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(C), _ptr(D), M, N, K)
    return D

def gemm_grouped_contiguous(A, sa, B, sb, layout, D=None, rows=None):
    """Contiguous-grouped form.  A[M_sum][K], sa[M_sum][K/128],
    B[G][N][K], sb[G][ceil(N/128)][K/128], layout[M_sum] int32.
    Rows whose id is outside [0, G) are left as they were in D (or in the
    0xFFFF-filled result when D is not given)."""
    A = _c(A, np.uint8); sa = _c(sa, np.float32); B = _c(B, np.uint8); sb = _c(sb, np.float32)
    layout = _c(layout, np.int32)
    M_sum, K = A.shape
    G, N, K2 = B.shape
    assert K2 == K and K % 128 == 0 and layout.shape == (M_sum,)
    assert sa.shape == (M_sum, K // 128) and sb.shape == (G, (N + 127) // 128, K // 128)
    lib = _load()
    if rows is not None:
        rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
        out = np.full((rows.size, N), 0xFFFF, dtype=np.uint16)
        lib.orc_gemm_grouped_contiguous_rows(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(layout),
                                             M_sum, N, K, G, _ptr(rows), rows.size, _ptr(out))
        return out
    if D is None:
        D = np.full((M_sum, N), 0xFFFF, dtype=np.uint16)
    assert D.dtype == np.uint16 and D.shape == (M_sum, N) and D.flags["C_CONTIGUOUS"]
    lib.orc_gemm_grouped_contiguous(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(D), _ptr(layout),
                                    M_sum, N, K, G)
    return D


def gemm_grouped_masked(A, sa, B, sb, masked_m, D=None, rows=None):
    """Masked-grouped form.  A[G][M_max][K], sa[G][M_max][K/128],
    B[G][N][K], sb[G][ceil(N/128)][K/128], masked_m[G] int32.
    Rows r >= clamp(masked_m[g], 0, M_max) are left as they were.
    ``rows`` are flat indices g*M_max + r."""
    A = _c(A, np.uint8); sa = _c(sa, np.float32); B = _c(B, np.uint8); sb = _c(sb, np.float32)
    masked_m = _c(masked_m, np.int32)
    G, M_max, K = A.shape
    G2, N, K2 = B.shape
    assert G2 == G and K2 == K and K % 128 == 0 and masked_m.shape == (G,)
    assert sa.shape == (G, M_max, K // 128) and sb.shape == (G, (N + 127) // 128, K // 128)
    lib = _load()
    if rows is not None:
        rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
        out = np.full((rows.size, N), 0xFFFF, dtype=np.uint16)
        lib.orc_gemm_grouped_masked_rows(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(masked_m),
                                         G, M_max, N, K, _ptr(rows), rows.size, _ptr(out))
        return out
    if D is None:
        D = np.full((G, M_max, N), 0xFFFF, dtype=np.uint16)
    assert D.dtype == np.uint16 and D.shape == (G, M_max, N) and D.flags["C_CONTIGUOUS"]
    lib.orc_gemm_grouped_masked(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(D), _ptr(masked_m),
                                G, M_max, N, K)
    return D
