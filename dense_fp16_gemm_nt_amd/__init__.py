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
SCRATCH = -5

R1_SINGLE_TILE = 1
R2_KLOOP = 2
R3_GRID = 3
R4_RING = 4
R5_PERSISTENT_WS = 5
R8_RING4_GAP = 8
R9_RING_SMALL = 9
R10_RING4_PAIRED = 10
R11_WIDE = 11
R12_SKINNY = 12
R13_KSPLIT = 13
RUNGS = (R1_SINGLE_TILE, R2_KLOOP, R3_GRID, R4_RING, R5_PERSISTENT_WS, R8_RING4_GAP,
         R9_RING_SMALL, R10_RING4_PAIRED, R11_WIDE, R12_SKINNY, R13_KSPLIT)

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
            L.gemm_f16_nt_strided_batched.restype = i32
            L.gemm_f16_nt_strided_batched.argtypes = [i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64, i64, vp]
            L.gemm_f16_nt_check_strided.restype = i32
            L.gemm_f16_nt_check_strided.argtypes = [i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64, i64]
            L.gemm_f16_nt_splitk.restype = i32
            L.gemm_f16_nt_splitk.argtypes = [i64, i64, i64, vp, vp, vp, i32, vp, i64, vp]
            L.gemm_f16_nt_splitk_noalloc.restype = i32
            L.gemm_f16_nt_splitk_noalloc.argtypes = [i64, i64, i64, vp, vp, vp, i32, vp]
            L.gemm_f16_nt_splitk_workspace.restype = i64
            L.gemm_f16_nt_splitk_workspace.argtypes = [i64, i64, i64, i32]
            L.gemm_f16_nt_check.restype = i32
            L.gemm_f16_nt_check.argtypes = [i32, i64, i64, i64, vp, vp, vp]
            L.gemm_f16_nt_status_string.restype = ctypes.c_char_p
            L.gemm_f16_nt_status_string.argtypes = [i32]
            L.gemm_f16_nt_schedule.restype = i64
            L.gemm_f16_nt_schedule.argtypes = [i64, i64, i64, i64p, i64p, i64p, i64]
            L.gemm_f16_nt_tile_walk.restype = i64
            L.gemm_f16_nt_tile_walk.argtypes = [i32, i64, i64, i32, i64p, i64p, i64p, i64]
            L.gemm_f16_nt_plan.restype = i32
            L.gemm_f16_nt_plan.argtypes = [i64, i64, i64, i32, ctypes.POINTER(ctypes.c_int), i64p,
                                           ctypes.POINTER(ctypes.c_int)]
            L.gemm_f16_nt_splitk_plan.restype = i32
            L.gemm_f16_nt_splitk_plan.argtypes = [i64, i64, i64, i32, i64p, i64p]
            L.gemm_f16_nt_ksplit_plan.restype = i32
            L.gemm_f16_nt_ksplit_plan.argtypes = [i32, i64, i64, i64, i32] + [ctypes.POINTER(ctypes.c_int)] * 4
            L.gemm_f16_nt_handoff_plan.restype = i32
            L.gemm_f16_nt_handoff_plan.argtypes = [i32, i32, i32, i64, ctypes.POINTER(ctypes.c_uint32),
                                                   ctypes.POINTER(ctypes.c_uint32)]
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
    """The same product on one rung of the kernel ladder (1-5, 8-13)."""
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


def _as_batched(X, name):
    """(batch or None, rows, cols, ld, stride) of a 2D or 3D fp16 device tensor
    whose last dimension is contiguous."""
    import torch

    if X.dtype != torch.float16 or not X.is_cuda:
        raise TypeError(f"{name} must be a float16 device tensor")
    if X.dim() == 2:
        if X.stride(1) != 1:
            raise ValueError(f"{name}: last dimension must be contiguous")
        return None, X.shape[0], X.shape[1], X.stride(0), 0
    if X.dim() == 3:
        if X.stride(2) != 1:
            raise ValueError(f"{name}: last dimension must be contiguous")
        return X.shape[0], X.shape[1], X.shape[2], X.stride(1), X.stride(0)
    raise ValueError(f"{name} must be 2D or 3D")


def gemm_f16_nt_strided_batched(A, B, D=None):
    """D[b] = A[b] @ B[b].T for 3D (or 2D, broadcast) fp16 tensors whose last
    dimension is contiguous; any leading dimension / batch stride the C-ABI
    accepts.  D defaults to a new contiguous (batch, M, N) tensor."""
    import torch

    ba, M, K, lda, sa = _as_batched(A, "A")
    bb, N, Kb, ldb, sb = _as_batched(B, "B")
    if Kb != K:
        raise ValueError(f"inner dimensions differ: {K} and {Kb}")
    if ba is not None and bb is not None and ba != bb:
        raise ValueError(f"batch sizes differ: {ba} and {bb}")
    batch = ba if ba is not None else (bb if bb is not None else 1)
    if A.device != B.device:
        raise ValueError("A and B on different devices")
    if D is None:
        D = torch.empty((batch, M, N), dtype=torch.float16, device=A.device)
    bd, Md, Nd, ldd, sd = _as_batched(D if D.dim() == 3 else D.unsqueeze(0), "D")
    if (bd, Md, Nd) != (batch, M, N):
        raise ValueError(f"D must be {batch} x {M} x {N}")
    st = lib().gemm_f16_nt_strided_batched(M, N, K, A.data_ptr(), lda, sa, B.data_ptr(), ldb, sb,
                                           D.data_ptr(), ldd, sd, batch, _stream(A))
    if st != OK:
        raise GemmError(st, "gemm_f16_nt_strided_batched")
    return D


def attention_scores(Q, Kt):
    """Unscaled attention scores S = Q @ K^T per head: Q (..., Sq, d) and
    K (..., Sk, d) with equal leading dimensions -> S (..., Sq, Sk), fp16
    (fp32 accumulation, one rounding), on the strided-batched kernel.  No
    scaling or softmax is applied."""
    import torch

    if Q.shape[:-2] != Kt.shape[:-2] or Q.shape[-1] != Kt.shape[-1]:
        raise ValueError(f"shapes {tuple(Q.shape)} and {tuple(Kt.shape)} do not match")
    lead = tuple(Q.shape[:-2])
    Sq, Sk = Q.shape[-2], Kt.shape[-2]
    S = torch.empty(lead + (Sq, Sk), dtype=torch.float16, device=Q.device)

    def as3(X):
        # collapse the leading dimensions when one stride describes them
        if X.dim() == 2:
            return X.unsqueeze(0)
        try:
            return X.view(-1, X.shape[-2], X.shape[-1])
        except RuntimeError:
            return None

    q3, k3, s3 = as3(Q), as3(Kt), as3(S)
    if q3 is not None and k3 is not None:
        gemm_f16_nt_strided_batched(q3, k3, s3)
        return S
    # leading dimensions not collapsible (e.g. heads interleaved in the
    # rows): one batched call per index of the outer dimensions
    for idx in torch.cartesian_prod(*[torch.arange(n) for n in lead[:-1]]).reshape(-1, len(lead) - 1).tolist() \
            if len(lead) > 1 else [[]]:
        sl = tuple(idx)
        gemm_f16_nt_strided_batched(Q[sl], Kt[sl], S[sl])
    return S


def plan(M: int, N: int, K: int, cus: int):
    """(rung_top, m_top, rung_rest) that gemm_f16_nt chooses for contiguous
    aligned operands on a device with `cus` compute units (host evaluation):
    rows [0, m_top) on rung_top, the rest on rung_rest (0: none)."""
    rt, mt, rr = ctypes.c_int(), ctypes.c_int64(), ctypes.c_int()
    st = lib().gemm_f16_nt_plan(int(M), int(N), int(K), int(cus), ctypes.byref(rt), ctypes.byref(mt), ctypes.byref(rr))
    if st != OK:
        raise GemmError(st, "gemm_f16_nt_plan")
    return rt.value, mt.value, rr.value


def splitk_plan(M: int, N: int, K: int, cus: int):
    """(m_top, splits) that gemm_f16_nt_splitk with splits = 0 chooses on a
    device with `cus` compute units (host evaluation, no GPU needed)."""
    m_top, splits = ctypes.c_int64(), ctypes.c_int64()
    st = lib().gemm_f16_nt_splitk_plan(int(M), int(N), int(K), int(cus), ctypes.byref(m_top), ctypes.byref(splits))
    if st != OK:
        raise GemmError(st, "gemm_f16_nt_splitk_plan")
    return m_top.value, splits.value


def ksplit_plan(rung: int, M: int, N: int, K: int, cus: int):
    """(mt, nf, db, waves): the workgroup tile rung 12 or 13 launches for
    an M x N x K product on a device with `cus` compute units (host
    evaluation): 16*mt rows of the side with fewer rows, 16*nf of the
    other, db load groups in flight per wave, `waves` waves splitting K."""
    mt, nf, db, nw = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    st = lib().gemm_f16_nt_ksplit_plan(int(rung), int(M), int(N), int(K), int(cus), ctypes.byref(mt),
                                       ctypes.byref(nf), ctypes.byref(db), ctypes.byref(nw))
    if st != OK:
        raise GemmError(st, "gemm_f16_nt_ksplit_plan")
    return mt.value, nf.value, db.value, nw.value


def splitk_workspace_bytes(M: int, N: int, K: int, splits: int = 0) -> int:
    n = lib().gemm_f16_nt_splitk_workspace(int(M), int(N), int(K), int(splits))
    if n < 0:
        raise GemmError(int(n), "gemm_f16_nt_splitk_workspace")
    return int(n)


def gemm_f16_nt_splitk(A, B, D=None, splits: int = 0, workspace=None):
    """D = A @ B.T with K cut into slices (fp32 partials in `workspace`, a
    byte tensor on A's device; allocated here when not given)."""
    import torch

    M, N, K, D = _operands(A, B, D)
    need = splitk_workspace_bytes(M, N, K, splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=A.device)
    st = lib().gemm_f16_nt_splitk(M, N, K, A.data_ptr(), B.data_ptr(), D.data_ptr(), int(splits),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(A))
    if st != OK:
        raise GemmError(st, "gemm_f16_nt_splitk")
    return D


def gemm_f16_nt_splitk_noalloc(A, B, D, splits: int = 0):
    """gemm_f16_nt_splitk with the library's own scratch array for the
    partial sums: nothing is allocated, D must be given."""
    if D is None:
        raise ValueError("gemm_f16_nt_splitk_noalloc writes into a given D (it allocates nothing)")
    M, N, K, D = _operands(A, B, D)
    st = lib().gemm_f16_nt_splitk_noalloc(M, N, K, A.data_ptr(), B.data_ptr(), D.data_ptr(), int(splits), _stream(A))
    if st != OK:
        raise GemmError(st, "gemm_f16_nt_splitk_noalloc")
    return D


def check(rung: int, M: int, N: int, K: int, A_ptr: int, B_ptr: int, D_ptr: int) -> int:
    """Validation status for raw arguments (no HIP call)."""
    return lib().gemm_f16_nt_check(int(rung), int(M), int(N), int(K), A_ptr, B_ptr, D_ptr)


def check_strided(M, N, K, A_ptr, lda, sa, B_ptr, ldb, sb, D_ptr, ldd, sd, batch) -> int:
    """Validation status of the strided form for raw arguments (no HIP call)."""
    return lib().gemm_f16_nt_check_strided(int(M), int(N), int(K), A_ptr, int(lda), int(sa), B_ptr, int(ldb),
                                           int(sb), D_ptr, int(ldd), int(sd), int(batch))


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


def tile_walk(rung: int, M: int, N: int, cus: int):
    """Host evaluation of a rung's tile walk on `cus` compute units:
    (wg, row0, col0) arrays, one entry per tile visit in workgroup-major
    visit order (the first output row and column of each tile)."""
    import numpy as np

    L = lib()
    n = L.gemm_f16_nt_tile_walk(rung, M, N, cus, None, None, None, 0)
    if n < 0:
        raise GemmError(int(n), "gemm_f16_nt_tile_walk")
    wg = np.empty(n, np.int64)
    r0 = np.empty(n, np.int64)
    c0 = np.empty(n, np.int64)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))  # noqa: E731
    L.gemm_f16_nt_tile_walk(rung, M, N, cus, p(wg), p(r0), p(c0), n)
    return wg, r0, c0


def handoff_plan(depth: int, producers: int, consumers: int, steps: int):
    """Host evaluation of rung 5's handoff counters: (ready_target,
    free_target) per k step."""
    import numpy as np

    rt = np.empty(steps, np.uint32)
    ft = np.empty(steps, np.uint32)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))  # noqa: E731
    st = lib().gemm_f16_nt_handoff_plan(depth, producers, consumers, steps, p(rt), p(ft))
    if st != OK:
        raise GemmError(st, "gemm_f16_nt_handoff_plan")
    return rt, ft


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
