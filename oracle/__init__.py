"""CPU oracle for the row-major FP32 product C = A x B (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
``cpu_baseline`` leg are the only callers. The product path (the HIP library
and its Python binding) never imports this package, and this package never
imports the product path; the two share only the seeded input generators in
``gemm_inputs``.

The arithmetic lives in ``gemm_oracle.c`` (plain C, FP64 accumulation in
ascending k, one rounding to FP32); this module only marshals NumPy arrays to
it through ctypes. See the header of ``gemm_oracle.c`` for the definition and
the passages of the pages it follows (the problem statement of the yekq.top
LeetGPU matrix-multiplication walkthrough, section 1 of the hpc.payai.win
lesson 10 on shared-memory tiled GEMM).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

# Plain optimisation, no fast-math (it would allow the k-sum to be
# reassociated) and no FMA contraction (it cannot change the result, since
# every FP32 x FP32 product is exact in double, but keeping it off keeps the
# arithmetic literally what the source says).
GCC_FLAGS = ["-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
             "-std=c11", "-shared", "-fPIC"]


def build(force: bool = True, src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile gemm_oracle.c (or another copy of it) into a shared library (gcc)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class OracleLib:
    """ctypes view of one compiled copy of gemm_oracle.c."""

    def __init__(self, path: str = LIB_PATH):
        lib = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_gemm_f32.restype = ctypes.c_int
        lib.oracle_gemm_f32.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_int]
        lib.oracle_gemm_f32_entries.restype = ctypes.c_int
        lib.oracle_gemm_f32_entries.argtypes = [vp, vp, i64, i64, i64, vp, vp, i64,
                                                vp, vp, ctypes.c_int]
        lib.oracle_gemm_f32_general.restype = ctypes.c_int
        lib.oracle_gemm_f32_general.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                                ctypes.c_float, vp, i64, vp, i64,
                                                ctypes.c_float, vp, i64, vp, ctypes.c_int]
        lib.oracle_gemm_i64.restype = ctypes.c_int
        lib.oracle_gemm_i64.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int]
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        """Threads the oracle's parallel loops use (OpenMP's default team size)."""
        return int(self.lib.oracle_num_threads())

    def gemm(self, A: np.ndarray, B: np.ndarray, threads: int = 0):
        """Full product. Returns (C float32 M x N, S float64 M x N) where
        S[i, j] = sum_k |A[i, k] * B[k, j]|."""
        A = np.ascontiguousarray(A, dtype=np.float32)
        B = np.ascontiguousarray(B, dtype=np.float32)
        M, N, K = _shapes(A, B)
        C = np.empty((M, N), dtype=np.float32)
        S = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_gemm_f32(_ptr(A), _ptr(B), _ptr(C), _ptr(S), M, N, K, threads)
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_f32 failed: {rc}")
        return C, S

    def gemm_entries(self, A: np.ndarray, B: np.ndarray, rows, cols, threads: int = 0):
        """The product evaluated only at (rows[t], cols[t]); returns (values f32, S f64)."""
        A = np.ascontiguousarray(A, dtype=np.float32)
        B = np.ascontiguousarray(B, dtype=np.float32)
        M, N, K = _shapes(A, B)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape or rows.ndim != 1:
            raise ValueError("rows and cols must be 1-D and of equal length")
        out = np.empty(rows.shape, dtype=np.float32)
        S = np.empty(rows.shape, dtype=np.float64)
        rc = self.lib.oracle_gemm_f32_entries(_ptr(A), _ptr(B), M, N, K, _ptr(rows), _ptr(cols),
                                              rows.size, _ptr(out), _ptr(S), threads)
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_f32_entries failed: {rc}")
        return out, S

    def gemm_general(self, trans_a: bool, trans_b: bool, M: int, N: int, K: int, alpha: float,
                     A: np.ndarray, lda: int, B: np.ndarray, ldb: int, beta: float,
                     C: np.ndarray, ldc: int, threads: int = 0):
        """C <- alpha * op(A) op(B) + beta * C on strided row-major storage.

        A, B and C are the flat float32 storage arrays (padding included); the
        result is a new flat array (C's storage with the M x N elements
        replaced) and S (float64 M x N)."""
        A = np.ascontiguousarray(A, dtype=np.float32).ravel()
        B = np.ascontiguousarray(B, dtype=np.float32).ravel()
        out = np.array(C, dtype=np.float32).ravel()
        S = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_gemm_f32_general(int(bool(trans_a)), int(bool(trans_b)), M, N, K,
                                              alpha, _ptr(A), lda, _ptr(B), ldb, beta, _ptr(out),
                                              ldc, _ptr(S), threads)
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_f32_general failed: {rc}")
        return out, S

    def gemm_i64(self, A: np.ndarray, B: np.ndarray, threads: int = 0) -> np.ndarray:
        """Exact integer product of integer-valued matrices (int64 in, int64 out)."""
        A = np.ascontiguousarray(A, dtype=np.int64)
        B = np.ascontiguousarray(B, dtype=np.int64)
        M, N, K = _shapes(A, B)
        C = np.empty((M, N), dtype=np.int64)
        rc = self.lib.oracle_gemm_i64(_ptr(A), _ptr(B), _ptr(C), M, N, K, threads)
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_i64 failed: {rc}")
        return C


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


def _shapes(A: np.ndarray, B: np.ndarray):
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch: A{A.shape} x B{B.shape}")
    return A.shape[0], B.shape[1], A.shape[1]


_default = None


def _lib() -> OracleLib:
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build(force=True)
        _default = OracleLib(LIB_PATH)
    return _default


def num_threads() -> int:
    return _lib().num_threads()


def gemm(A: np.ndarray, B: np.ndarray, threads: int = 0):
    return _lib().gemm(A, B, threads)


def gemm_entries(A: np.ndarray, B: np.ndarray, rows, cols, threads: int = 0):
    return _lib().gemm_entries(A, B, rows, cols, threads)


def gemm_i64(A: np.ndarray, B: np.ndarray, threads: int = 0) -> np.ndarray:
    return _lib().gemm_i64(A, B, threads)


def gemm_general(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, threads=0):
    return _lib().gemm_general(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                               threads)


gemm.__doc__ = OracleLib.gemm.__doc__
gemm_entries.__doc__ = OracleLib.gemm_entries.__doc__
gemm_i64.__doc__ = OracleLib.gemm_i64.__doc__
gemm_general.__doc__ = OracleLib.gemm_general.__doc__
