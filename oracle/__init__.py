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
* conv2d(x, w, stride, pad, dilation) -> (y64, s64)
    The 2-D convolution of a convolutional layer from its usual definition (see
    oracle.c; the pages only say it can be recast as a matrix product).

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
        lib.oracle_conv2d_f64.argtypes = [i64] * 13 + [vp, vp, vp, vp, ctypes.c_int]
        lib.oracle_conv2d_f64.restype = ctypes.c_int
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


    def conv2d(self, x, w, stride=(1, 1), pad=(0, 0), dilation=(1, 1), threads=None):
        """fp64 reference of the 2-D convolution: x is N x C x H x W, w is K x C x R x S
        (float32, packed); returns (y64, s64), each N x K x P x Q."""
        x = np.ascontiguousarray(np.asarray(x))
        w = np.ascontiguousarray(np.asarray(w))
        if x.dtype != np.float32 or w.dtype != np.float32 or x.ndim != 4 or w.ndim != 4:
            raise TypeError("x and w must be 4-D float32 arrays")
        N, C, H, W = x.shape
        K, C2, R, S = w.shape
        if C2 != C:
            raise ValueError(f"channel counts differ: x has {C}, w has {C2}")
        sh, sw = stride
        ph, pw = pad
        dh, dw = dilation
        P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
        Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
        if P < 1 or Q < 1:
            raise ValueError("the filter does not fit the padded input")
        y = np.full((N, K, P, Q), np.nan)
        s = np.full((N, K, P, Q), np.nan)
        rc = self.lib.oracle_conv2d_f64(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, _ptr(x),
                                        _ptr(w), _ptr(y), _ptr(s), threads or default_threads())
        if rc != 0:
            raise RuntimeError(f"oracle_conv2d_f64 failed with status {rc}")
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


def conv2d(x, w, stride=(1, 1), pad=(0, 0), dilation=(1, 1), threads=None):
    return load().conv2d(x, w, stride, pad, dilation, threads=threads)
