"""CPU oracle for single-precision GEMM, C = alpha*A*B + beta*C_in, in fp64.

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The GPU library never
imports or calls this package, and this package never imports the GPU
library; the two share no code.

The arithmetic lives in ``sgemm_oracle.c`` (plain C, fp64, k ascending,
parallel over rows only).  This module only marshals numpy arrays into it.
Definition followed: the problem statement of "Matmul I: tiling and shared
memory" (section 1) with the epilogue alpha*acc + beta*C of "2D Register
Tiling: The Outer Product" (The Kernel), and beta == 0 never reading C as in
"The Final Kernel" (Skipping The Read Of C).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_long)


def _ld(x, rows, cols, name):
    """Leading dimension (elements) of a row-major float32 2-D view."""
    if not isinstance(x, np.ndarray) or x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 numpy array")
    if x.shape != (rows, cols):
        raise ValueError(f"{name} has shape {x.shape}, expected {(rows, cols)}")
    if rows > 0 and cols > 1 and x.strides[1] != 4:
        raise ValueError(f"{name} must have unit column stride")
    if rows > 1:
        if x.strides[0] % 4 or x.strides[0] // 4 < cols:
            raise ValueError(f"{name} rows overlap or are misaligned")
        return x.strides[0] // 4
    return max(cols, 1)


def _ptr(x):
    return x.ctypes.data_as(_f32p)


class Oracle:
    """ctypes front end of one build of ``sgemm_oracle.c``."""

    def __init__(self, lib_path=None):
        if lib_path is None:
            lib_path = _build.LIB
            if not os.path.exists(lib_path) or (
                    os.path.getmtime(lib_path) < os.path.getmtime(_build.SRC)):
                _build.build()
        lib = ctypes.CDLL(lib_path)
        lib.oracle_sgemm_f64.restype = ctypes.c_int
        lib.oracle_sgemm_f64.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            _f32p, ctypes.c_long, _f32p, ctypes.c_long,
            ctypes.c_float, _f32p, ctypes.c_long, _f64p, ctypes.c_long]
        lib.oracle_sgemm_sampled.restype = ctypes.c_int
        lib.oracle_sgemm_sampled.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            _f32p, ctypes.c_long, _f32p, ctypes.c_long,
            ctypes.c_float, _f32p, ctypes.c_long,
            ctypes.c_long, _i64p, _i64p, _f64p]
        lib.oracle_version.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        self.lib = lib
        self.path = lib_path

    def set_threads(self, n: int) -> None:
        self.lib.oracle_set_threads(int(n))

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def _common(self, A, B, C_in, alpha, beta):
        M, K = A.shape
        K2, N = B.shape
        if K2 != K:
            raise ValueError("inner dimensions differ")
        lda = _ld(A, M, K, "A")
        ldb = _ld(B, K, N, "B")
        alpha = np.float32(alpha)
        beta = np.float32(beta)
        if beta != 0:
            if C_in is None:
                raise ValueError("C_in is required when beta != 0")
            ldc, cp = _ld(C_in, M, N, "C_in"), _ptr(C_in)
        elif C_in is not None:
            # Handed over so that a reading of C_in with beta == 0 would show.
            ldc, cp = _ld(C_in, M, N, "C_in"), _ptr(C_in)
        else:
            ldc, cp = max(N, 1), None
        return M, N, K, lda, ldb, float(alpha), float(beta), ldc, cp

    def sgemm_ref(self, A, B, C_in=None, alpha=1.0, beta=0.0):
        """Full fp64 product alpha*A@B + beta*C_in; A [M,K], B [K,N] float32.

        A, B and C_in may be row-major views with padded rows (unit column
        stride).  C_in is not read when beta == 0 and may then be None.
        Returns a fresh [M,N] float64 array.
        """
        M, N, K, lda, ldb, a, b, ldc, cp = self._common(A, B, C_in, alpha, beta)
        out = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_sgemm_f64(M, N, K, a, _ptr(A), lda, _ptr(B), ldb,
                                       b, cp, ldc, out.ctypes.data_as(_f64p), max(N, 1))
        if rc != 0:
            raise RuntimeError(f"oracle_sgemm_f64 returned {rc}")
        return out

    def sgemm_ref_sampled(self, A, B, I, J, C_in=None, alpha=1.0, beta=0.0):
        """fp64 entries C[I[s], J[s]] of alpha*A@B + beta*C_in, each computed
        with the same arithmetic as :meth:`sgemm_ref`."""
        M, N, K, lda, ldb, a, b, ldc, cp = self._common(A, B, C_in, alpha, beta)
        I = np.ascontiguousarray(I, dtype=np.int64)
        J = np.ascontiguousarray(J, dtype=np.int64)
        if I.shape != J.shape or I.ndim != 1:
            raise ValueError("I and J must be 1-D and of equal length")
        out = np.empty(I.shape[0], dtype=np.float64)
        rc = self.lib.oracle_sgemm_sampled(M, N, K, a, _ptr(A), lda, _ptr(B), ldb,
                                           b, cp, ldc, I.shape[0],
                                           I.ctypes.data_as(_i64p), J.ctypes.data_as(_i64p),
                                           out.ctypes.data_as(_f64p))
        if rc != 0:
            raise RuntimeError(f"oracle_sgemm_sampled returned {rc}")
        return out


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def sgemm_ref(A, B, C_in=None, alpha=1.0, beta=0.0):
    return default().sgemm_ref(A, B, C_in, alpha, beta)


def sgemm_ref_sampled(A, B, I, J, C_in=None, alpha=1.0, beta=0.0):
    return default().sgemm_ref_sampled(A, B, I, J, C_in, alpha, beta)


def set_threads(n: int) -> None:
    default().set_threads(n)


def max_threads() -> int:
    return default().max_threads()
