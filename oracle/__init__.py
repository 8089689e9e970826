"""CPU oracle for C = A x B with FP32 operands and fp64 arithmetic.

TEST INFRASTRUCTURE ONLY: tests/, the smoke check in __graft_entry__.py and the
cpu_baseline leg of bench.py may import this package; the product path
(fp32_gemm_f32_amd) never does, and this package never imports the product.

The arithmetic lives in sgemm_oracle.c (the plain definition of the product, see that
file's header for the passages it follows); this module only builds it with gcc and
marshals numpy arrays to it. counting.py holds the pages' read-count model.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sgemm_oracle.c")
_LIB = os.path.join(_HERE, "_liboracle.so")
_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra"]

_lib = None


class OracleReport(ctypes.Structure):
    _fields_ = [("max_err", ctypes.c_double),
                ("arg_i", ctypes.c_int64), ("arg_j", ctypes.c_int64),
                ("n_checked", ctypes.c_int64), ("n_inexact", ctypes.c_int64),
                ("n_nonfinite", ctypes.c_int64), ("n_zero_den_bad", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


def build(src: str = _SRC, out: str = _LIB, extra: list[str] | None = None) -> str:
    """Compile the oracle with gcc (always; cheap). Returns the library path."""
    cmd = ["gcc", *_CFLAGS, *(extra or []), src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(lib):
    i64, dp = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_gemm_f64.argtypes = [i64, i64, i64, dp, i64, dp, i64, dp, i64]
    lib.oracle_gemm_f64.restype = ctypes.c_int
    lib.oracle_check.argtypes = [i64, i64, i64, dp, i64, dp, i64, dp, i64, dp, i64,
                                 ctypes.POINTER(OracleReport)]
    lib.oracle_check.restype = ctypes.c_int
    lib.oracle_sample.argtypes = [i64, i64, i64, dp, i64, dp, i64, i64, dp, dp, dp, dp]
    lib.oracle_sample.restype = ctypes.c_int
    lib.oracle_transpose.argtypes = [i64, i64, dp, i64, dp, i64]
    lib.oracle_transpose.restype = ctypes.c_int
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load the oracle library (building it first if it is missing)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _ld(x: np.ndarray) -> int:
    """Leading dimension (elements) of a row-major 2-D float32 view."""
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError("oracle operands are 2-D float32 arrays")
    if x.strides[1] != 4 or x.strides[0] % 4:
        raise ValueError("oracle operands must be row-major with unit column stride")
    return max(x.strides[0] // 4, x.shape[1], 1)


def _ptr(x: np.ndarray) -> int:
    return x.__array_interface__["data"][0]


def gemm_f64(A: np.ndarray, B: np.ndarray, lib=None) -> np.ndarray:
    """C_ref = A x B in double precision (the plain definition)."""
    lib = lib or load()
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C = np.empty((M, N), dtype=np.float64)
    rc = lib.oracle_gemm_f64(M, N, K, _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(C), max(N, 1))
    if rc:
        raise RuntimeError(f"oracle_gemm_f64 failed ({rc})")
    return C


def check(A: np.ndarray, B: np.ndarray, C: np.ndarray, rows=None, lib=None) -> dict:
    """Compare an FP32 result C against the oracle (all rows, or the listed rows)."""
    lib = lib or load()
    M, K = A.shape
    N = B.shape[1]
    if C.shape != (M, N):
        raise ValueError("C has the wrong shape")
    rep = OracleReport()
    if rows is None:
        rc = lib.oracle_check(M, N, K, _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(C), _ld(C),
                              None, 0, ctypes.byref(rep))
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        rc = lib.oracle_check(M, N, K, _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(C), _ld(C),
                              _ptr(r), r.size, ctypes.byref(rep))
    if rc:
        raise RuntimeError(f"oracle_check failed ({rc})")
    return rep.as_dict()


def sample(A: np.ndarray, B: np.ndarray, ii, jj, lib=None):
    """(ref, den) for the elements (ii[t], jj[t]) of A x B."""
    lib = lib or load()
    M, K = A.shape
    N = B.shape[1]
    ii = np.ascontiguousarray(np.asarray(ii, dtype=np.int64))
    jj = np.ascontiguousarray(np.asarray(jj, dtype=np.int64))
    if ii.shape != jj.shape:
        raise ValueError("index arrays differ in shape")
    ref = np.empty(ii.size, dtype=np.float64)
    den = np.empty(ii.size, dtype=np.float64)
    rc = lib.oracle_sample(M, N, K, _ptr(A), _ld(A), _ptr(B), _ld(B), ii.size,
                           _ptr(ii), _ptr(jj), _ptr(ref), _ptr(den))
    if rc:
        raise RuntimeError(f"oracle_sample failed ({rc})")
    return ref, den


def transpose(X: np.ndarray, lib=None) -> np.ndarray:
    """out = X^T (the LDS microbenchmark's result), as a new packed array."""
    lib = lib or load()
    rows, cols = X.shape
    out = np.empty((cols, rows), dtype=np.float32)
    rc = lib.oracle_transpose(rows, cols, _ptr(X), _ld(X), _ptr(out), max(rows, 1))
    if rc:
        raise RuntimeError(f"oracle_transpose failed ({rc})")
    return out


def threads(lib=None) -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return (lib or load()).oracle_threads()


def set_threads(n: int, lib=None) -> int:
    """Threads for the oracle's later parallel regions; returns the previous count."""
    return (lib or load()).oracle_set_threads(n)
