"""CPU oracle for D = A * B^T in fp16 (fp64 accumulation, one RNE rounding).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
bench's CPU-baseline leg may import this package.  The product path (the HIP
library and its Python binding) never touches it, and it shares no code with
that path: its arithmetic lives in ``gemm_oracle.c`` (plain C, built with
gcc), loaded here through ctypes.

The definition it follows and the pages it cites are in the header comment
of ``gemm_oracle.c``.  Arrays cross this interface as numpy ``uint16`` fp16
bit patterns, row-major: A is M x K, B is N x K, D is M x N.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# Plain C: no fast-math, no FMA contraction, so the k-loop adds in order.
GCC_ARGS = ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
            "-fno-fast-math", "-o", _LIB, _SRC, "-lm"]

_lock = threading.Lock()
_lib = None


def build() -> str:
    """Compile liboracle.so from gemm_oracle.c (always recompiles)."""
    subprocess.run(GCC_ARGS, check=True)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if (not os.path.exists(_LIB)
                    or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
                build()
            L = ctypes.CDLL(_LIB)
            u16p = ctypes.POINTER(ctypes.c_uint16)
            f64p = ctypes.POINTER(ctypes.c_double)
            i64p = ctypes.POINTER(ctypes.c_int64)
            i64 = ctypes.c_int64
            L.oracle_f16_to_f64.restype = ctypes.c_double
            L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
            L.oracle_f64_to_f16.restype = ctypes.c_uint16
            L.oracle_f64_to_f16.argtypes = [ctypes.c_double]
            L.oracle_f16_to_f64_n.argtypes = [u16p, f64p, i64]
            L.oracle_f64_to_f16_n.argtypes = [f64p, u16p, i64]
            L.oracle_gemm_nt.restype = ctypes.c_int
            L.oracle_gemm_nt.argtypes = [i64, i64, i64, u16p, u16p, u16p, ctypes.c_int]
            L.oracle_gemm_nt_sampled.restype = ctypes.c_int
            L.oracle_gemm_nt_sampled.argtypes = [i64, i64, i64, u16p, u16p, i64,
                                                 i64p, i64p, u16p, ctypes.c_int]
            _lib = L
    return _lib


def _p(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _bits(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected fp16 bit patterns (uint16), got {a.dtype}")
    return np.ascontiguousarray(a)


def f16_to_f64(bits) -> np.ndarray:
    b = _bits(bits)
    out = np.empty(b.shape, dtype=np.float64)
    lib().oracle_f16_to_f64_n(_p(b, ctypes.c_uint16), _p(out, ctypes.c_double), b.size)
    return out


def f64_to_f16(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(a.shape, dtype=np.uint16)
    lib().oracle_f64_to_f16_n(_p(a, ctypes.c_double), _p(out, ctypes.c_uint16), a.size)
    return out


def gemm_nt(A, B, nthreads: int = 0):
    """Full D (uint16 bits, M x N) and the number of threads used."""
    A = _bits(A)
    B = _bits(B)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[1]:
        raise ValueError(f"shape mismatch A{A.shape} B{B.shape}")
    M, K = A.shape
    N = B.shape[0]
    D = np.empty((M, N), dtype=np.uint16)
    used = lib().oracle_gemm_nt(M, N, K, _p(A, ctypes.c_uint16), _p(B, ctypes.c_uint16),
                                _p(D, ctypes.c_uint16), int(nthreads))
    return D, used


def gemm_nt_sampled(A, B, rows, cols, nthreads: int = 0):
    """D[rows[i], cols[i]] for each i (uint16 bits) and the threads used."""
    A = _bits(A)
    B = _bits(B)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[1]:
        raise ValueError(f"shape mismatch A{A.shape} B{B.shape}")
    M, K = A.shape
    N = B.shape[0]
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    c = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    if r.shape != c.shape:
        raise ValueError("rows and cols differ in length")
    out = np.empty(r.shape, dtype=np.uint16)
    used = lib().oracle_gemm_nt_sampled(M, N, K, _p(A, ctypes.c_uint16), _p(B, ctypes.c_uint16),
                                        r.size, _p(r, ctypes.c_int64), _p(c, ctypes.c_int64),
                                        _p(out, ctypes.c_uint16), int(nthreads))
    if used < 0:
        raise IndexError("sample index out of range")
    return out, used
