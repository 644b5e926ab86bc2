"""CPU oracle (test infrastructure only).

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.  The product path never does: the HIP
library and its Python binding share no code with it and fail loudly if the
HIP build is missing.

`gemm` / `gemm_entries` wrap `oracle_gemm.c` (binary64 accumulation over the
exact bf16 inputs, ascending k per element; MikPoly page, part 1 item 2, the
untiled triple loop).  `cost_model` holds the oracle of the page's
polymerization cost model.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_gemm.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               "-std=c11", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_gemm.argtypes = [i64, i64, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64, p, ctypes.c_int]
        lib.oracle_gemm.restype = ctypes.c_int
        lib.oracle_gemm_entries.argtypes = [i64, i64, i64, p, i64, i64, p, i64, i64, i64, p, p, p, p, p,
                                            ctypes.c_int]
        lib.oracle_gemm_entries.restype = ctypes.c_int
        lib.oracle_gemm_outer.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64]
        lib.oracle_gemm_outer.restype = ctypes.c_int
        lib.oracle_threads.argtypes = [ctypes.c_int]
        lib.oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def threads(requested: int = 0) -> int:
    return _load().oracle_threads(requested)


def gemm(a: np.ndarray, b: np.ndarray, with_abs: bool = False, nthreads: int = 0):
    """C = A.B in binary64 for bf16-bit operands of shape (M,K),(K,N) or batched
    (batch,M,K),(batch,K,N).  Returns C (and sum |a*b| if with_abs)."""
    lib = _load()
    a = np.ascontiguousarray(a, dtype=np.uint16)
    b = np.ascontiguousarray(b, dtype=np.uint16)
    squeeze = a.ndim == 2
    if squeeze:
        a, b = a[None], b[None]
    batch, M, K = a.shape
    Kb, N = b.shape[1:]
    assert Kb == K and b.shape[0] == batch
    c = np.empty((batch, M, N), dtype=np.float64)
    e = np.empty((batch, M, N), dtype=np.float64) if with_abs else None
    rc = lib.oracle_gemm(batch, M, N, K, _ptr(a), K, M * K, _ptr(b), N, K * N, _ptr(c), N, M * N,
                         _ptr(e), nthreads)
    if rc != 0:
        raise RuntimeError("oracle_gemm failed")
    if squeeze:
        c = c[0]
        e = e[0] if e is not None else None
    return (c, e) if with_abs else c


def gemm_entries(a: np.ndarray, b: np.ndarray, rows, cols, bidx=None, nthreads: int = 0):
    """Selected entries of A.B (binary64) and their sum |a*b|."""
    lib = _load()
    a = np.ascontiguousarray(a, dtype=np.uint16)
    b = np.ascontiguousarray(b, dtype=np.uint16)
    if a.ndim == 2:
        a, b = a[None], b[None]
    batch, M, K = a.shape
    N = b.shape[2]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    bi = None if bidx is None else np.ascontiguousarray(bidx, dtype=np.int64)
    out = np.empty(rows.shape[0], dtype=np.float64)
    outabs = np.empty(rows.shape[0], dtype=np.float64)
    rc = lib.oracle_gemm_entries(M, N, K, _ptr(a), K, M * K, _ptr(b), N, K * N, rows.shape[0],
                                 _ptr(bi), _ptr(rows), _ptr(cols), _ptr(out), _ptr(outabs), nthreads)
    if rc != 0:
        raise RuntimeError("oracle_gemm_entries failed")
    return out, outabs


def gemm_outer(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """A.B accumulated as K ascending rank-1 updates (oracle_gemm_outer)."""
    lib = _load()
    a = np.ascontiguousarray(a, dtype=np.uint16)
    b = np.ascontiguousarray(b, dtype=np.uint16)
    M, K = a.shape
    N = b.shape[1]
    c = np.empty((M, N), dtype=np.float64)
    if lib.oracle_gemm_outer(M, N, K, _ptr(a), K, _ptr(b), N, _ptr(c), N) != 0:
        raise RuntimeError("oracle_gemm_outer failed")
    return c


def error_bound(K: int, abs_sum: np.ndarray, slack: float = 2.0) -> np.ndarray:
    """Forward error bound of recursive binary32 summation of K exact products:
    |fl(sum) - sum| <= gamma_K * sum|a*b|, gamma_K = K u / (1 - K u), u = 2^-24
    (Higham, Accuracy and Stability of Numerical Algorithms, 2nd ed., sec. 3.1)."""
    u = 2.0 ** -24
    Ku = K * u
    return slack * (Ku / (1.0 - Ku)) * abs_sum
