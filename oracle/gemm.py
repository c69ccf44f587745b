"""Integer GEMM of the oracle (test infrastructure only): a ctypes front end
to the plain C loops in int_gemm.c.  See that file for what is computed."""
from __future__ import annotations

import ctypes

import numpy as np

from .build import build

_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        for name in ("oracle_int_gemm_i32", "oracle_int_gemm_i64"):
            f = getattr(lib, name)
            f.restype = None
            f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3
        _lib = lib
    return _lib


def int_gemm_ref(a: np.ndarray, b: np.ndarray, acc: str = "i32") -> np.ndarray:
    """acc[m,n] = sum_k a[m,k] * b[n,k] for int8 a [M,K], b [N,K].

    ``acc="i32"`` accumulates modulo 2^32 (int32 result), ``acc="i64"`` in int64.
    """
    a = np.ascontiguousarray(a, dtype=np.int8)
    b = np.ascontiguousarray(b, dtype=np.int8)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("expected a [M,K] and b [N,K]")
    M, K = a.shape
    N = b.shape[0]
    lib = _load()
    if acc == "i32":
        c = np.empty((M, N), dtype=np.int32)
        lib.oracle_int_gemm_i32(a.ctypes.data, b.ctypes.data, c.ctypes.data, M, N, K)
    elif acc == "i64":
        c = np.empty((M, N), dtype=np.int64)
        lib.oracle_int_gemm_i64(a.ctypes.data, b.ctypes.data, c.ctypes.data, M, N, K)
    else:
        raise ValueError(acc)
    return c
