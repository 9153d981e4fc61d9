"""GPU parity past 4 GiB: operands, outputs, batch strides and split-K
partial sums whose byte offsets do not fit in 32 bits.  Sampled outputs
(the rows and columns on both sides of each 2^31- and 2^32-byte offset
among them) against the CPU oracle, into NaN-poisoned outputs that must be
written everywhere.

The large operands repeat the rows of a small seeded pattern matrix P (row
r is P[(r + shift) % p], p prime, so a row read from a wrong address holds
other values); the oracle gets the same rows from P on the host.
"""
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
GIB4 = 1 << 32


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def bits(t) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def pattern(p: int, K: int, seed: int, stream: int) -> np.ndarray:
    return inputs.generate(p, K, seed, stream, workloads.U11)


def built(P: np.ndarray, rows: int, shift: int = 0):
    """The rows x K device operand whose row r is P[(r + shift) % len(P)]."""
    idx = inputs.periodic_index(rows, len(P), shift)
    return dev(P)[torch.from_numpy(idx).to(DEV)]


def crossing(count: int, row_bytes: int) -> list:
    """Indices on both sides of the 2^31- and 2^32-byte offsets (and their
    multiples) of a run of `count` items of `row_bytes` bytes each."""
    out = []
    for edge in range(1 << 31, count * row_bytes, 1 << 31):
        i = edge // row_bytes
        out += [i - 1, i, i + 1]
    return [i for i in out if 0 <= i < count]


def sample(M: int, N: int, count: int, seed: int, rows_extra=(), cols_extra=()):
    """Output positions (rows[i], cols[i]): the corners, each designed row
    with the first, last and a random column, each designed column with the
    first, last and a random row, and `count` random positions."""
    rng = np.random.default_rng(seed)
    rx, cx = list(rows_extra), list(cols_extra)
    rows = [0, 0, M - 1, M - 1] + rx * 3 + [0] * len(cx) + [M - 1] * len(cx) + list(rng.integers(0, M, len(cx)))
    cols = [0, N - 1, 0, N - 1] + [0] * len(rx) + [N - 1] * len(rx) + list(rng.integers(0, N, len(rx))) + cx * 3
    rows += list(rng.integers(0, M, count))
    cols += list(rng.integers(0, N, count))
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


def gathered(D, rows, cols) -> np.ndarray:
    r = torch.from_numpy(rows).to(DEV)
    c = torch.from_numpy(cols).to(DEV)
    return bits(D[r, c])


def all_written(D) -> bool:
    return not torch.isnan(D).any().item()


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_output_past_4gib():
    """D of 5.4 GB (65553 x 40968, ragged M): rows past the 2^31 and 2^32
    byte offsets, the library's choice."""
    M, N, K = 65553, 40968, 128
    A, B = inputs.operands(M, N, K, 71, workloads.U11)
    say(f"[gpu] output past 4 GiB: {M}x{N}x{K}, D {M * N * 2 / 2**30:.2f} GiB, plan {g.plan(M, N, K, 256)}")
    D = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    g.gemm_f16_nt(dev(A), dev(B), D)
    torch.cuda.synchronize()
    assert all_written(D), "output elements left unwritten"
    rows, cols = sample(M, N, 3000, 1, rows_extra=crossing(M, N * 2))
    want, _ = oracle.gemm_nt_sampled(A, B, rows, cols)
    assert_parity(gathered(D, rows, cols), want, K, "D past 4 GiB")
    del D
    free()


@pytest.mark.parametrize("side,small", [("A", 512), ("B", 512), ("A", 16), ("B", 16)])
def test_operand_past_4gib(side, small):
    """A (or B) of 4.6 GB: 1048876 rows of K = 2176, so row bases pass the
    2^31 and 2^32 byte offsets; the other operand has 512 rows (the
    four-wave ring) or 16 (rung 12, whose large side it is)."""
    big, K = 1048876, 2176
    P = pattern(997, K, 72, 0)
    S = inputs.generate(small, K, 72, 1, workloads.U11)
    shift = 13
    say(f"[gpu] {side} past 4 GiB: {big} rows x K={K}, {big * K * 2 / 2**30:.2f} GiB")
    Big = built(P, big, shift)
    extra = crossing(big, K * 2)
    if side == "A":
        M, N = big, small
        D = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        say(f"      plan {g.plan(M, N, K, 256)}")
        g.gemm_f16_nt(Big, dev(S), D)
        torch.cuda.synchronize()
        rows, cols = sample(M, N, 3000, 2, rows_extra=extra)
        want, _ = oracle.gemm_nt_sampled(P[inputs.periodic_index(M, len(P), shift)[rows]], S,
                                         np.arange(len(rows)), cols)
    else:
        M, N = small, big
        D = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        say(f"      plan {g.plan(M, N, K, 256)}")
        g.gemm_f16_nt(dev(S), Big, D)
        torch.cuda.synchronize()
        rows, cols = sample(M, N, 3000, 3, cols_extra=extra)
        want, _ = oracle.gemm_nt_sampled(S, P[inputs.periodic_index(N, len(P), shift)[cols]],
                                         rows, np.arange(len(cols)))
    assert all_written(D), "output elements left unwritten"
    assert_parity(gathered(D, rows, cols), want, K, f"{side} past 4 GiB")
    del Big, D
    free()


def test_strided_batch_past_4gib():
    """40 products of 8192 x 8192 x 128 in one strided-batched call: D is
    5 GiB, so batch entries from 32 on start past 2^32 bytes; each entry's
    A and B are shifted pattern rows."""
    batch, M, N, K = 40, 8192, 8192, 128
    P, Q = pattern(997, K, 73, 0), pattern(1009, K, 73, 1)
    say(f"[gpu] strided batch past 4 GiB: {batch} x {M}x{N}x{K}, D {batch * M * N * 2 / 2**30:.2f} GiB")
    A = torch.stack([built(P, M, 7 * b) for b in range(batch)])
    B = torch.stack([built(Q, N, 11 * b) for b in range(batch)])
    D = torch.full((batch, M, N), float("nan"), dtype=torch.float16, device=DEV)
    g.gemm_f16_nt_strided_batched(A, B, D)
    torch.cuda.synchronize()
    assert all_written(D), "output elements left unwritten"
    del A, B
    for b in range(batch):
        rows, cols = sample(M, N, 120, 100 + b)
        Ab = P[inputs.periodic_index(M, len(P), 7 * b)[rows]]
        Bb = Q[inputs.periodic_index(N, len(Q), 11 * b)[cols]]
        want, _ = oracle.gemm_nt_sampled(Ab, Bb, np.arange(len(rows)), np.arange(len(cols)))
        # the diagonal of the sampled block: output (rows[i], cols[i])
        assert_parity(gathered(D[b], rows, cols), want, K, f"batch entry {b}")
    del D
    free()


def test_splitk_partials_past_4gib():
    """16384 x 16384 x 4096 in 8 slices: the fp32 partial sums take 8 GiB
    (1 GiB a slice), so slices 4 to 7 start at or past 2^32 bytes of the
    workspace."""
    M, N, K, splits = 16384, 16384, 4096, 8
    P, Q = pattern(997, K, 74, 0), pattern(1009, K, 74, 1)
    need = g.splitk_workspace_bytes(M, N, K, splits)
    assert need == 2 * GIB4, need
    say(f"[gpu] split-K partials past 4 GiB: {M}x{N}x{K}, {splits} slices, workspace {need / 2**30:.2f} GiB")
    A, B = built(P, M, 3), built(Q, N, 5)
    D = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    g.gemm_f16_nt_splitk(A, B, D, splits=splits)
    torch.cuda.synchronize()
    assert all_written(D), "output elements left unwritten"
    rows, cols = sample(M, N, 3000, 4)
    want, _ = oracle.gemm_nt_sampled(P[inputs.periodic_index(M, len(P), 3)[rows]],
                                     Q[inputs.periodic_index(N, len(Q), 5)[cols]],
                                     np.arange(len(rows)), np.arange(len(cols)))
    assert_parity(gathered(D, rows, cols), want, K, "split-K past 4 GiB")
    del A, B, D
    free()
