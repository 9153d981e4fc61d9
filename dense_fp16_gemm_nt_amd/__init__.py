"""fp16 NT GEMM for MI355X (gfx950): D = A * B^T, fp32 accumulation, one
fp16 rounding at writeback.

Thin ctypes binding over ``libgemm_f16_nt.so`` (the C-ABI declared in
``include/gemm_f16_nt.h``): it checks tensor metadata, passes device
pointers and the current HIP stream, and raises on a non-zero status.  All
arithmetic runs in the library's HIP kernels; there is no fallback.  If the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgemm_f16_nt.so")

OK = 0
INVALID_ARG = -1
UNSUPPORTED = -2
LAUNCH = -3
DEVICE = -4

R1_SINGLE_TILE = 1
R2_KLOOP = 2
R3_GRID = 3
R4_RING = 4
R5_PERSISTENT_WS = 5
RUNGS = (R1_SINGLE_TILE, R2_KLOOP, R3_GRID, R4_RING, R5_PERSISTENT_WS)

_lock = threading.Lock()
_lib = None


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_string(status)})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m dense_fp16_gemm_nt_amd.build` (hipcc, gfx950)")
            L = ctypes.CDLL(LIB_PATH)
            i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
            i64p = ctypes.POINTER(ctypes.c_int64)
            L.gemm_f16_nt.restype = i32
            L.gemm_f16_nt.argtypes = [i64, i64, i64, vp, vp, vp, vp]
            L.gemm_f16_nt_rung.restype = i32
            L.gemm_f16_nt_rung.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp]
            L.gemm_f16_nt_persistent.restype = i32
            L.gemm_f16_nt_persistent.argtypes = [i64, i64, i64, vp, vp, vp, i64, vp]
            L.gemm_f16_nt_check.restype = i32
            L.gemm_f16_nt_check.argtypes = [i32, i64, i64, i64, vp, vp, vp]
            L.gemm_f16_nt_status_string.restype = ctypes.c_char_p
            L.gemm_f16_nt_status_string.argtypes = [i32]
            L.gemm_f16_nt_schedule.restype = i64
            L.gemm_f16_nt_schedule.argtypes = [i64, i64, i64, i64p, i64p, i64p, i64]
            L.gemm_f16_nt_ring_plan.restype = i32
            L.gemm_f16_nt_ring_plan.argtypes = [i32, i64, ctypes.POINTER(ctypes.c_int), i64p, i64p]
            _lib = L
    return _lib


def status_string(status: int) -> str:
    try:
        return lib().gemm_f16_nt_status_string(int(status)).decode()
    except RuntimeError:
        return "library not loaded"


def _operands(A, B, D):
    import torch

    if A.dtype != torch.float16 or B.dtype != torch.float16:
        raise TypeError("A and B must be torch.float16")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[1]:
        raise ValueError(f"A must be M x K and B N x K; got {tuple(A.shape)} and {tuple(B.shape)}")
    if not (A.is_cuda and B.is_cuda):
        raise ValueError("A and B must be device tensors")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous (row-major)")
    M, K = A.shape
    N = B.shape[0]
    if D is None:
        D = torch.empty((M, N), dtype=torch.float16, device=A.device)
    elif D.dtype != torch.float16 or tuple(D.shape) != (M, N) or not D.is_contiguous() or D.device != A.device:
        raise ValueError(f"D must be a contiguous float16 {M} x {N} tensor on {A.device}")
    return M, N, K, D


def _stream(A):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(A.device).cuda_stream)


def gemm_f16_nt(A, B, D=None):
    """D = A @ B.T (A: M x K, B: N x K, fp16) on the current stream."""
    M, N, K, D = _operands(A, B, D)
    st = lib().gemm_f16_nt(M, N, K, A.data_ptr(), B.data_ptr(), D.data_ptr(), _stream(A))
    if st != OK:
        raise GemmError(st, "gemm_f16_nt")
    return D


def gemm_f16_nt_rung(rung: int, A, B, D=None):
    """The same product on one rung of the kernel ladder (1..5)."""
    M, N, K, D = _operands(A, B, D)
    st = lib().gemm_f16_nt_rung(int(rung), M, N, K, A.data_ptr(), B.data_ptr(), D.data_ptr(), _stream(A))
    if st != OK:
        raise GemmError(st, f"gemm_f16_nt_rung({rung})")
    return D


def gemm_f16_nt_persistent(A, B, num_workgroups: int, D=None):
    """Rung 5 with an explicit persistent grid size."""
    M, N, K, D = _operands(A, B, D)
    st = lib().gemm_f16_nt_persistent(M, N, K, A.data_ptr(), B.data_ptr(), D.data_ptr(),
                                      int(num_workgroups), _stream(A))
    if st != OK:
        raise GemmError(st, "gemm_f16_nt_persistent")
    return D


def check(rung: int, M: int, N: int, K: int, A_ptr: int, B_ptr: int, D_ptr: int) -> int:
    """Validation status for raw arguments (no HIP call)."""
    return lib().gemm_f16_nt_check(int(rung), int(M), int(N), int(K), A_ptr, B_ptr, D_ptr)


def schedule(M: int, N: int, num_workgroups: int):
    """Host evaluation of the persistent rung's tile visits: (wg, tile_m, tile_n) lists."""
    import numpy as np

    L = lib()
    n = L.gemm_f16_nt_schedule(M, N, num_workgroups, None, None, None, 0)
    if n < 0:
        raise GemmError(int(n), "gemm_f16_nt_schedule")
    wg = np.empty(n, np.int64)
    tm = np.empty(n, np.int64)
    tn = np.empty(n, np.int64)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))  # noqa: E731
    L.gemm_f16_nt_schedule(M, N, num_workgroups, p(wg), p(tm), p(tn), n)
    return wg, tm, tn


def ring_plan(depth: int, steps: int):
    """Host evaluation of the operand ring: (stage, lap, refill) per k step."""
    import numpy as np

    stage = np.empty(steps, np.int32)
    lap = np.empty(steps, np.int64)
    refill = np.empty(steps, np.int64)
    st = lib().gemm_f16_nt_ring_plan(depth, steps, stage.ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
                                     lap.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                     refill.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    if st != OK:
        raise GemmError(st, "gemm_f16_nt_ring_plan")
    return stage, lap, refill
