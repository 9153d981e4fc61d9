"""gemm_f16_nt_splitk_noalloc (the split-K entry point that allocates
nothing: its fp32 partial sums live in the library's per-device scratch
array) against gemm_f16_nt_splitk with a caller workspace, through the
C-ABI: identical bits on two calls in a row, the second on a smaller
product (so the scratch array still holds the first call's partial sums),
and parity with the oracle at the stated tolerance."""
import sys

import numpy as np
import pytest

import dense_fp16_gemm_nt_amd as g
import oracle
from dense_fp16_gemm_nt_amd import inputs, workloads
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def host_bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def both(M, N, K, seed, splits=0):
    """D from the workspace entry point and from the no-allocation one
    (each into a NaN-poisoned output), and the oracle's D."""
    A, B = inputs.operands(M, N, K, seed, workloads.U11)
    dA = torch.from_numpy(A).to(DEV)
    dB = torch.from_numpy(B).to(DEV)
    ws_bytes = g.splitk_workspace_bytes(M, N, K, splits)
    assert 0 < ws_bytes <= 64 << 20, ws_bytes
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    D_ws = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    D_na = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    torch.cuda.synchronize()
    say(f"[gpu] splitk workspace M={M} N={N} K={K} splits={splits} ({ws_bytes} bytes)")
    g.gemm_f16_nt_splitk(dA, dB, D_ws, splits, ws)
    torch.cuda.synchronize()
    say(f"[gpu] splitk_noalloc M={M} N={N} K={K} splits={splits}")
    g.gemm_f16_nt_splitk_noalloc(dA, dB, D_na, splits)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm_nt(A, B)
    return host_bits(D_ws), host_bits(D_na), ref


def test_noalloc_matches_workspace_entry_on_two_calls():
    # first: 64 slices of 512 x 512 fp32 partial sums, the whole 64 MiB
    # array; second: a smaller product (16 slices of 256 x 256, 4 MiB, asked
    # for explicitly: the library's own choice runs it unsplit) over the
    # first call's leftovers
    for (M, N, K, seed, sp) in ((512, 512, 32768, 901, 0), (256, 256, 8192, 902, 16)):
        d_ws, d_na, ref = both(M, N, K, seed, sp)
        np.testing.assert_array_equal(d_na, d_ws)
        assert_parity(d_na, ref, K, f"noalloc {M}x{N}x{K}")


def test_noalloc_whole_rounds_plus_split_rows():
    # 6144^3: 21 tile rows run unsplit, the last 768 rows split K three
    # ways (56.6 MiB of partial sums); then a ragged tile-starved product
    for (M, N, K, seed, sp) in ((6144, 6144, 6144, 903, 0), (300, 260, 4104, 904, 5)):
        d_ws, d_na, ref = both(M, N, K, seed, sp)
        np.testing.assert_array_equal(d_na, d_ws)
        assert_parity(d_na, ref, K, f"noalloc {M}x{N}x{K}")
