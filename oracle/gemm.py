"""W4A4 GEMM oracle: int64 accumulation + float32 dequant (test infrastructure).

Abstract / page "SpinQuant, Reproduced" Q7-Q8: weights and activations are
4-bit.  Readings:
  * acc[m][n] = sum_k qx[m][k] * qw[n][k] in int64 (C routine, gemm_int64.c);
    the library accumulates in int32, so |acc| < 2^31 is asserted;
  * dequant Y[m][n] = fl32(fl32(float32(acc) * s_x[m]) * s_w[n]) — token scale
    first, then channel scale, each product rounded to float32.

A second, independent route (``gemm_int_codes_blas``) forms the same integer
product with float64 BLAS; it is exact because every partial sum is an
integer far below 2^53, and the tests use it to pin the C routine.
"""

import ctypes
import os

import numpy as np

from . import build as _build
from .quant import unpack_int4

__all__ = ["w4a8_gemm", "gemm_int_codes", "gemm_rows", "gemm_int_codes_blas", "dequant", "w4a4_gemm",
           "num_threads"]

_lib = None


def _load():
    global _lib
    if _lib is None:
        # ORACLE_GEMM_LIBRARY names another build of gemm_int64.c (the
        # sanitized one of the sanitizer tests)
        path = os.environ.get("ORACLE_GEMM_LIBRARY") or _build.LIB
        if path == _build.LIB and (not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
            _build.build(force=True)
        lib = ctypes.CDLL(path)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i8p = ctypes.c_void_p
        lib.oracle_gemm_i64.argtypes = [i8p, i8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64p]
        lib.oracle_gemm_i64.restype = None
        lib.oracle_gemm_i64_rows.argtypes = [i8p, i8p, i64p, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, i64p]
        lib.oracle_gemm_i64_rows.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the C routine uses."""
    return int(_load().oracle_num_threads())


def gemm_int_codes(qx, qw) -> np.ndarray:
    """int64 acc [M, N] from int8 codes qx [M, K], qw [N, K] (C, int64 accumulate)."""
    qx = np.ascontiguousarray(qx, dtype=np.int8)
    qw = np.ascontiguousarray(qw, dtype=np.int8)
    M, K = qx.shape
    N, K2 = qw.shape
    if K != K2:
        raise ValueError("K mismatch")
    acc = np.empty((M, N), dtype=np.int64)
    _load().oracle_gemm_i64(qx.ctypes.data, qw.ctypes.data, M, N, K,
                            acc.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    return acc


def gemm_rows(qx, qw, rows) -> np.ndarray:
    """int64 acc for the listed rows only: [len(rows), N]."""
    qx = np.ascontiguousarray(qx, dtype=np.int8)
    qw = np.ascontiguousarray(qw, dtype=np.int8)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    M, K = qx.shape
    N = qw.shape[0]
    if rows.size and (rows.min() < 0 or rows.max() >= M):
        raise ValueError("row index out of range")
    acc = np.empty((rows.size, N), dtype=np.int64)
    _load().oracle_gemm_i64_rows(qx.ctypes.data, qw.ctypes.data,
                                 rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                 int(rows.size), N, K,
                                 acc.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    return acc


def gemm_int_codes_blas(qx, qw) -> np.ndarray:
    """Second route: the same integer product via float64 BLAS (exact below 2^53)."""
    a = np.asarray(qx, dtype=np.float64)
    b = np.asarray(qw, dtype=np.float64)
    if a.shape[1] * 64 >= 2 ** 53:
        raise ValueError("K too large for an exact float64 route")
    return np.rint(a @ b.T).astype(np.int64)


def dequant(acc, x_scale, w_scale) -> np.ndarray:
    """Y = fl32(fl32(float32(acc) * s_x[m]) * s_w[n]); asserts |acc| < 2^31."""
    acc = np.asarray(acc, dtype=np.int64)
    if acc.size and np.abs(acc).max() >= 2 ** 31:
        raise OverflowError("accumulator exceeds the int32 range")
    a32 = acc.astype(np.float32)                     # exact: |acc| < 2^24 at every size used
    t = a32 * np.asarray(x_scale, dtype=np.float32)[:, None]
    return (t * np.asarray(w_scale, dtype=np.float32)[None, :]).astype(np.float32)


def w4a4_gemm(Xq, x_scale, Wq, w_scale):
    """Full W4A4 product from packed operands: returns (Y float32 [M, N], acc int64)."""
    qx = unpack_int4(Xq)
    qw = unpack_int4(Wq)
    acc = gemm_int_codes(qx, qw)
    return dequant(acc, x_scale, w_scale), acc


def w4a8_gemm(Xq8, x_scale, Wq, w_scale):
    """The W4A8 product: int8 activation codes [M, K] against packed INT4
    weights [N, K/2]; int64 accumulation and the same float32 epilogue.
    Returns (Y float32 [M, N], acc int64)."""
    qx = np.asarray(Xq8, dtype=np.int8)
    qw = unpack_int4(Wq)
    acc = gemm_int_codes(qx, qw)
    return dequant(acc, x_scale, w_scale), acc
