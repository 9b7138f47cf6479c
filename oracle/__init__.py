"""CPU oracle for fp32 GEMM and GEMV (fp64 accumulation), loaded through ctypes.

TEST INFRASTRUCTURE. Only tests/, the smoke check in __graft_entry__ and the
benchmark's cpu_baseline / verification leg import this package. The GPU library
(tiled_gemm_gemv_amd) never imports it, and it never imports the GPU library.

The arithmetic lives in oracle.c; this module only marshals numpy arrays:

* gemm(A, B, rows=None, threads=None) -> (C64, S64)
    C64[r, j] = sum_k A[i, k] * B[k, j] for i = rows[r] (or i = r), in fp64,
    summed in ascending k; S64 = sum_k |A[i, k] * B[k, j]|.
    Definition: "Matrix Operations" (docs.vulkan.org ML-inference tutorial),
    section "Matrix-Matrix Multiplication (GEMM)".
* gemv(A, x, threads=None) -> (y64, s64)
    y64[i] = sum_j A[i, j] * x[j] in fp64, ascending j; s64 = sum_j |A[i, j] * x[j]|.
    Definition: same page, section "Matrix-Vector Multiplication".

Inputs must be float32, 2-D row-major with unit column stride (any row stride).
"""
import ctypes
import os

import numpy as np

from . import build as _build


def default_threads() -> int:
    """Host threads available to this process."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _row_major_f32(a, name):
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError(f"{name} must be float32, got {a.dtype}")
    if a.ndim != 2:
        raise ValueError(f"{name} must be 2-D")
    if a.shape[1] > 1 and a.strides[1] != 4:
        a = np.ascontiguousarray(a)
    if a.shape[0] > 1 and (a.strides[0] % 4 != 0 or a.strides[0] < 4 * a.shape[1]):
        a = np.ascontiguousarray(a)
    ld = a.strides[0] // 4 if a.shape[0] > 1 else max(1, a.shape[1])
    return a, max(ld, 1)


def _ptr(a):
    return a.ctypes.data if a is not None and a.size else None


class Oracle:
    """ctypes front end of one compiled copy of oracle.c."""

    def __init__(self, libpath: str):
        lib = ctypes.CDLL(libpath)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_gemm_f64.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, vp, i64,
                                        ctypes.c_int]
        lib.oracle_gemm_f64.restype = ctypes.c_int
        lib.oracle_gemv_f64.argtypes = [i64, i64, vp, i64, vp, vp, vp, ctypes.c_int]
        lib.oracle_gemv_f64.restype = ctypes.c_int
        self.lib = lib
        self.path = libpath

    def gemm(self, A, B, rows=None, threads=None):
        """fp64 reference of C = A @ B for all rows, or for the given row indices."""
        A, lda = _row_major_f32(A, "A")
        B, ldb = _row_major_f32(B, "B")
        M, K = A.shape
        K2, N = B.shape
        if K2 != K:
            raise ValueError(f"inner dimensions differ: A is {A.shape}, B is {B.shape}")
        if rows is None:
            rows_arr = None
            nrows = M
        else:
            rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            nrows = rows_arr.shape[0]
        # NaN-filled, so an output the library fails to write cannot pass for a result.
        C = np.full((nrows, N), np.nan, dtype=np.float64)
        S = np.full((nrows, N), np.nan, dtype=np.float64)
        rc = self.lib.oracle_gemm_f64(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(rows_arr), nrows,
                                      _ptr(C), _ptr(S), max(N, 1), threads or default_threads())
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_f64 failed with status {rc}")
        return C, S

    def gemv(self, A, x, threads=None):
        """fp64 reference of y = A @ x."""
        A, lda = _row_major_f32(A, "A")
        x = np.ascontiguousarray(np.asarray(x))
        if x.dtype != np.float32 or x.ndim != 1:
            raise TypeError("x must be a 1-D float32 array")
        M, N = A.shape
        if x.shape[0] != N:
            raise ValueError(f"x has {x.shape[0]} entries, A has {N} columns")
        y = np.full(M, np.nan, dtype=np.float64)
        s = np.full(M, np.nan, dtype=np.float64)
        rc = self.lib.oracle_gemv_f64(M, N, _ptr(A), lda, _ptr(x), _ptr(y), _ptr(s),
                                      threads or default_threads())
        if rc != 0:
            raise RuntimeError(f"oracle_gemv_f64 failed with status {rc}")
        return y, s


_default = None


def load() -> Oracle:
    """The oracle built from oracle.c, building liboracle.so first only if it is missing."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def gemm(A, B, rows=None, threads=None):
    return load().gemm(A, B, rows=rows, threads=threads)


def gemv(A, x, threads=None):
    return load().gemv(A, x, threads=threads)
