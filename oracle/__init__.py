"""CPU oracle for the FP32 GEMM C = A.B -- TEST INFRASTRUCTURE, not part of the product.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py` may import
this package.  The GPU library never loads it and shares no code with it; the only thing
both sides share is the seeded input generator `tdb_inputs`, which holds none of the
product's arithmetic.

The arithmetic lives in `oracle_gemm.c` (plain i-k-j triple loop, FP64 accumulation, see
that file's header for the passages it follows); this module builds it with gcc, loads it
with ctypes and wraps it for numpy arrays.

Acceptance bound used by every parity check (elementwise, inclusive):
    |C[i][j] - C64[i][j]| <= 1e-5 * Bnd[i][j] + 1e-6,   Bnd = sum_k |A[i][k]| * |B[k][j]|.
`tolerance_ratio` returns max |C - C64| / (1e-5 * Bnd + 1e-6); a value <= 1 passes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle_gemm.c")
LIB = os.path.join(_HERE, "liboracle_gemm.so")

REL_TOL = 1e-5
ABS_TOL = 1e-6

_default = None


def build(force: bool = True, src: str = SRC, out: str = LIB) -> str:
    """Compile an oracle source (default oracle_gemm.c) into a shared library with gcc and
    OpenMP.  Returns the path of the library."""
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-Wall", "-Werror",
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _as_rows(X: np.ndarray, name: str):
    """A 2-D float32 array with unit column stride; returns (array, leading dimension)."""
    if not isinstance(X, np.ndarray) or X.dtype != np.float32 or X.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 numpy array")
    if X.shape[1] > 0 and X.strides[1] != 4:
        X = np.ascontiguousarray(X)
    ld = X.strides[0] // 4 if X.shape[0] > 1 else X.shape[1]
    return X, max(ld, X.shape[1], 1)


class OracleLib:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_gemm_f64.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, vp, i64]
        lib.oracle_gemm_f64.restype = ctypes.c_int
        lib.oracle_gemm_f64_sampled.argtypes = [i64, i64, i64, vp, i64, vp, i64, i64, vp,
                                                vp, vp, vp]
        lib.oracle_gemm_f64_sampled.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        self.path = path
        self._lib = lib

    def max_threads(self) -> int:
        return int(self._lib.oracle_max_threads())

    def set_threads(self, n: int) -> None:
        self._lib.oracle_set_threads(int(n))

    def gemm_f64(self, A: np.ndarray, B: np.ndarray):
        """Full oracle.  Returns (C64, Bnd), both M x N float64."""
        A, lda = _as_rows(A, "A")
        B, ldb = _as_rows(B, "B")
        M, K = A.shape
        K2, N = B.shape
        if K != K2:
            raise ValueError("inner dimensions differ")
        C64 = np.zeros((M, N), dtype=np.float64)
        Bnd = np.zeros((M, N), dtype=np.float64)
        if M == 0 or N == 0:
            return C64, Bnd
        rc = self._lib.oracle_gemm_f64(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
                                       C64.ctypes.data, Bnd.ctypes.data, N)
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_f64 failed ({rc})")
        return C64, Bnd

    def gemm_f64_sampled(self, A: np.ndarray, B: np.ndarray, rows, cols):
        """Sampled oracle at positions (rows[s], cols[s]).  Returns (c64, bnd) vectors."""
        A, lda = _as_rows(A, "A")
        B, ldb = _as_rows(B, "B")
        M, K = A.shape
        K2, N = B.shape
        if K != K2:
            raise ValueError("inner dimensions differ")
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape or rows.ndim != 1:
            raise ValueError("rows and cols must be 1-D and of equal length")
        n = rows.shape[0]
        c64 = np.zeros(n, dtype=np.float64)
        bnd = np.zeros(n, dtype=np.float64)
        rc = self._lib.oracle_gemm_f64_sampled(M, N, K, A.ctypes.data, lda, B.ctypes.data,
                                               ldb, n, rows.ctypes.data, cols.ctypes.data,
                                               c64.ctypes.data, bnd.ctypes.data)
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_f64_sampled failed ({rc})")
        return c64, bnd


def default() -> OracleLib:
    """The oracle built from oracle_gemm.c (built on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB):
            build()
        _default = OracleLib(LIB)
    return _default


def max_threads() -> int:
    return default().max_threads()


def set_threads(n: int) -> None:
    default().set_threads(n)


def gemm_f64(A: np.ndarray, B: np.ndarray):
    """Full oracle.  Returns (C64, Bnd), both M x N float64."""
    return default().gemm_f64(A, B)


def gemm_f64_sampled(A: np.ndarray, B: np.ndarray, rows, cols):
    """Sampled oracle at positions (rows[s], cols[s]).  Returns (c64, bnd) vectors."""
    return default().gemm_f64_sampled(A, B, rows, cols)


def tolerance_ratio(C, C64, Bnd) -> float:
    """max |C - C64| / (1e-5 * Bnd + 1e-6) over all elements (0.0 for empty input).

    A NaN or infinite C gives +inf, so it always fails."""
    C = np.asarray(C, dtype=np.float64)
    if C.size == 0:
        return 0.0
    err = np.abs(C - np.asarray(C64, dtype=np.float64))
    lim = REL_TOL * np.asarray(Bnd, dtype=np.float64) + ABS_TOL
    r = err / lim
    if not np.all(np.isfinite(r)):
        return float("inf")
    return float(r.max())


def within_tolerance(C, C64, Bnd) -> bool:
    return tolerance_ratio(C, C64, Bnd) <= 1.0
