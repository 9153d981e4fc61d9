"""GPU parity: every rung of the HIP ladder against the CPU oracle, through
the C-ABI, on seeded inputs (tolerance and exact pins as documented in
tests/parity.py and tests/test_oracle_pins.py).

All tests here need an MI355X; each prints the case it is about to run
before touching the GPU.
"""
import sys

import numpy as np
import pytest

import dense_fp16_gemm_nt_amd as g
import oracle
from dense_fp16_gemm_nt_amd import inputs, workloads
from tests.parity import as_f64, assert_parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"
ALL_RUNGS = [1, 2, 3, 4, 5, 8, 9, 10]
RING4_RUNGS = (8, 10)   # M, N >= 256, N a multiple of 8, K a multiple of 64, >= 2 k steps


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host_bits(t) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def run(rung, A, B, D=None):
    """rung 0 = gemm_f16_nt (the library's choice)."""
    if rung == 0:
        out = g.gemm_f16_nt(A, B, D)
    else:
        out = g.gemm_f16_nt_rung(rung, A, B, D)
    torch.cuda.synchronize()
    return out


def supported(rung, M, N, K):
    if rung == 1:
        return (M, N, K) == (128, 128, 64)
    if rung == 2:
        return (M, N) == (128, 128)
    if rung == 10:   # also a partial first step when K is not a multiple of 64, and any N
        return M >= 256 and N >= 256 and K % 8 == 0 and K > 64
    if rung in RING4_RUNGS:
        return M >= 256 and N >= 256 and N % 8 == 0 and K % 64 == 0 and K >= 128
    return True


def rand_case(M, N, K, seed, dist=workloads.U11):
    A, B = inputs.operands(M, N, K, seed, dist)
    return A, B


# ------------------------------------------------------------ small shapes

SMALL = [(w.M, w.N, w.K, w.seed, w.dist) for w in workloads.WORKLOADS[:2]] + [(128, 128, 512, 21, workloads.U11)]


@pytest.mark.parametrize("rung", [0] + ALL_RUNGS)
@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}")
def test_small_workloads(rung, case):
    M, N, K, seed, dist = case
    if not supported(rung, M, N, K):
        pytest.skip("rung does not implement this shape")
    A, B = rand_case(M, N, K, seed, dist)
    ref, _ = oracle.gemm_nt(A, B)
    say(f"[gpu] rung={rung} M={M} N={N} K={K} seed={seed}")
    D = run(rung, dev(A), dev(B))
    worst = assert_parity(host_bits(D), ref, K, f"rung {rung} {M}x{N}x{K}")
    say(f"      worst err/tol = {worst:.3f}")


RAGGED = [
    (1, 1, 8), (3, 5, 16), (33, 17, 24), (128, 4, 64), (130, 130, 72), (255, 257, 136),
    (256, 256, 8), (300, 260, 200), (257, 513, 520), (511, 129, 1000), (640, 384, 64 * 9 + 8),
    (64, 7, 40), (5, 3, 8),
]


@pytest.mark.parametrize("rung", [0, 3, 4, 5])
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_ragged_shapes(rung, shape):
    M, N, K = shape
    A, B = rand_case(M, N, K, 100 + M + N + K)
    ref, _ = oracle.gemm_nt(A, B)
    say(f"[gpu] ragged rung={rung} M={M} N={N} K={K}")
    D = run(rung, dev(A), dev(B))
    assert_parity(host_bits(D), ref, K, f"rung {rung} {M}x{N}x{K}")


# -------------------------------------------------------------- exact pins

@pytest.mark.parametrize("rung", [0] + ALL_RUNGS)
def test_selection_matrix_bitwise(rung):
    M, N, K = {1: (128, 128, 64), 2: (128, 128, 512), 6: (512, 256, 192), 7: (512, 256, 192), 8: (512, 256, 192), 10: (512, 256, 192)}.get(rung, (384, 320, 192))
    rng = np.random.default_rng(5)
    pick = rng.integers(0, K, M)
    A = np.zeros((M, K), np.float16)
    A[np.arange(M), pick] = 1
    B = (rng.uniform(-60000, 60000, (N, K))).astype(np.float16)
    say(f"[gpu] selection rung={rung} M={M} N={N} K={K}")
    D = run(rung, dev(A), dev(B))
    assert np.array_equal(host_bits(D), B[:, pick].T.view(np.uint16))


@pytest.mark.parametrize("rung", [0, 3, 4, 5, 8, 9, 10])
@pytest.mark.parametrize("K", [64, 512, 4096, 8192])
def test_all_ones_equals_k(rung, K):
    if not supported(rung, 256, 256, K):
        pytest.skip("rung does not implement this shape")
    A = np.ones((256, K), np.float16)
    B = np.ones((256, K), np.float16)
    say(f"[gpu] all-ones rung={rung} K={K}")
    D = run(rung, dev(A), dev(B))
    assert np.all(as_f64(host_bits(D)) == K)


@pytest.mark.parametrize("rung", [0, 3, 4, 5, 8, 9, 10])
def test_small_integers_bitwise(rung):
    rng = np.random.default_rng(14)
    shapes = [(256, 192, 8192, -4, 5), (264, 256, 768, 0, 5)]
    if rung in RING4_RUNGS:
        shapes = [(256, 256, 8192, -4, 5), (512, 256, 768, 0, 5)]
    for (M, N, K, lo, hi) in shapes:
        A = rng.integers(lo, hi, (M, K)).astype(np.float16)
        B = rng.integers(lo, hi, (N, K)).astype(np.float16)
        ref, _ = oracle.gemm_nt(A, B)
        say(f"[gpu] small-int rung={rung} M={M} N={N} K={K}")
        D = run(rung, dev(A), dev(B))
        got = host_bits(D)
        assert np.array_equal(got, ref), f"{np.sum(got != ref)} mismatches"


@pytest.mark.parametrize("rung", [0, 3, 4, 5, 8, 9, 10])
def test_designed_rows(rung):
    """Exact sums on a tie, on the overflow threshold and on the subnormal
    grid: round-half-even, +inf at 65520, gradual underflow."""
    K, R = (128, 256) if rung in RING4_RUNGS else (64, 128)
    A = np.zeros((R, K), np.float16)
    B = np.zeros((R, K), np.float16)
    A[0, :2] = [1, 1]
    A[1, 0] = 2.0 ** -12
    B[0, :2] = [2048, 1]
    B[1, :2] = [2048, 3]
    B[2, :2] = [65504, 16]
    B[3, 0] = 2.0 ** -12
    B[4, 0] = 2.0 ** -13
    B[5, :2] = [-65504, -16]
    say(f"[gpu] designed rows rung={rung}")
    D = host_bits(run(rung, dev(A), dev(B)))
    assert [int(x) for x in D[0, :3]] == [0x6800, 0x6802, 0x7C00]
    assert int(D[0, 5]) == 0xFC00
    assert int(D[1, 3]) == 0x0001, hex(int(D[1, 3]))   # 2^-24, smallest subnormal
    assert int(D[1, 4]) == 0x0000                       # 2^-25 ties to zero


# ------------------------------------------------------- degenerate shapes

@pytest.mark.parametrize("rung", [0, 3, 4, 5])
def test_k_zero_writes_zeros(rung):
    D = torch.full((70, 90), float("nan"), dtype=torch.float16, device=DEV)
    A = torch.empty((70, 0), dtype=torch.float16, device=DEV)
    B = torch.empty((90, 0), dtype=torch.float16, device=DEV)
    say(f"[gpu] K=0 rung={rung}")
    run(rung, A, B, D)
    assert torch.all(D == 0).item()


def test_empty_outputs_are_noops():
    A = torch.ones((0, 64), dtype=torch.float16, device=DEV)
    B = torch.ones((32, 64), dtype=torch.float16, device=DEV)
    say("[gpu] empty M")
    D = g.gemm_f16_nt(A, B)
    torch.cuda.synchronize()
    assert D.shape == (0, 32)


def test_error_paths_launch_nothing():
    A = torch.ones((128, 64), dtype=torch.float16, device=DEV)
    B = torch.ones((128, 64), dtype=torch.float16, device=DEV)
    D = torch.full((128, 128), 7.0, dtype=torch.float16, device=DEV)
    say("[gpu] error paths")
    with pytest.raises(g.GemmError) as e:
        g.gemm_f16_nt_rung(1, A[:, :56].contiguous(), B[:, :56].contiguous(), D)   # R1 needs K = 64
    assert e.value.status == g.UNSUPPORTED
    L = g.lib()
    st = L.gemm_f16_nt_rung(5, 128, 128, 60, A.data_ptr(), B.data_ptr(), D.data_ptr(), None)
    assert st == g.UNSUPPORTED          # rungs other than 3, 4 and 9 need K % 8 == 0
    st = L.gemm_f16_nt_rung(4, 128, 128, 4, A.data_ptr(), B.data_ptr(), D.data_ptr(), None)
    assert st == g.UNSUPPORTED          # rungs 4 and 9 stage such rows for K >= 8 only
    st = L.gemm_f16_nt(128, 128, 64, A.data_ptr() + 1, B.data_ptr(), D.data_ptr(), None)
    assert st == g.UNSUPPORTED          # odd address: not an fp16 array
    st = L.gemm_f16_nt(128, 128, 64, A.data_ptr(), B.data_ptr(), A.data_ptr() + 64, None)
    assert st == g.INVALID_ARG          # D overlaps A
    torch.cuda.synchronize()
    assert torch.all(D == 7.0).item()


# ----------------------------------------------- invariants of the schedule

@pytest.mark.parametrize("shape", [(520, 700, 256), (512, 768, 256)], ids=["ragged", "whole_tiles"])
def test_poisoned_output_is_fully_overwritten(shape):
    M, N, K = shape
    A, B = rand_case(M, N, K, 77)
    ref, _ = oracle.gemm_nt(A, B)
    for rung in (0, 3, 4, 5, 8, 9, 10):
        if not supported(rung, M, N, K):
            continue
        D = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        say(f"[gpu] poison rung={rung}")
        run(rung, dev(A), dev(B), D)
        assert_parity(host_bits(D), ref, K, f"poison rung {rung}")


def test_repeatable_and_grid_size_invariant():
    M, N, K = 1280, 1536, 1024
    A, B = rand_case(M, N, K, 78)
    dA, dB = dev(A), dev(B)
    say("[gpu] repeatability rung 4 / the four-wave rungs")
    first = host_bits(run(4, dA, dB))
    for _ in range(2):
        assert np.array_equal(host_bits(run(4, dA, dB)), first)
    for r in RING4_RUNGS:
        first4w = host_bits(run(r, dA, dB))
        for _ in range(2):
            assert np.array_equal(host_bits(run(r, dA, dB)), first4w)
    base = None
    for grid in (1, 7, 256, 512):
        say(f"[gpu] persistent grid={grid}")
        D = g.gemm_f16_nt_persistent(dA, dB, grid)
        torch.cuda.synchronize()
        bits = host_bits(D)
        if base is None:
            base = bits
            ref, _ = oracle.gemm_nt(A, B)
            assert_parity(bits, ref, K, "persistent")
        assert np.array_equal(bits, base), f"grid {grid} differs"


@pytest.mark.parametrize("rung", RING4_RUNGS)
@pytest.mark.parametrize("shape", [(4608, 4608, 256), (8192, 2304, 128), (256, 256, 128), (512, 768, 192)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ring4_persistent_rounds(rung, shape):
    """More tiles than compute units: workgroups of the four-wave ring walk
    several tiles each (the last round partial); every output compared."""
    M, N, K = shape
    A, B = rand_case(M, N, K, 80 + K)
    ref, _ = oracle.gemm_nt(A, B)
    D = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    say(f"[gpu] ring4 persistent rounds rung={rung} {M}x{N}x{K}")
    run(rung, dev(A), dev(B), D)
    assert_parity(host_bits(D), ref, K, f"rung {rung} {M}x{N}x{K}")


@pytest.mark.parametrize("shape", [(300, 264, 128), (520, 776, 256), (1000, 1032, 192), (4000, 4000, 1024),
                                   (300, 261, 128), (520, 777, 200), (1000, 1030, 1024)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ring4_ragged_tiles(shape):
    """M, N not multiples of 256 on the four-wave ring: the last tile row and
    column move back to end at M and N and overlap their neighbours.  Every
    output is compared with the oracle, repeated runs are bitwise equal (the
    shared rows are written twice with the same bits), and the padding
    columns of a pitched D are never written."""
    M, N, K = shape
    A, B = rand_case(M, N, K, 90 + K)
    ref, _ = oracle.gemm_nt(A, B)
    dA, dB = dev(A), dev(B)
    for rung in (0,) + RING4_RUNGS:
        if not supported(rung, M, N, K):
            assert N % 8 or K % 64, "only N % 8 != 0 or K % 64 != 0 leave out rungs 6-8"
            continue
        D = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        say(f"[gpu] ring4 ragged rung={rung} {M}x{N}x{K}")
        run(rung, dA, dB, D)
        first = host_bits(D)
        assert_parity(first, ref, K, f"rung {rung} {M}x{N}x{K}")
        for _ in range(2):
            assert np.array_equal(host_bits(run(rung, dA, dB, D)), first), f"rung {rung} not repeatable"
    Dfull = torch.full((1, M, N + 8), float("nan"), dtype=torch.float16, device=DEV)
    say(f"[gpu] ring4 ragged pitched D {M}x{N}x{K}")
    g.gemm_f16_nt_strided_batched(dA[None], dB[None], Dfull[:, :, :N])
    torch.cuda.synchronize()
    assert_parity(host_bits(Dfull[0, :, :N].contiguous()), ref, K, "pitched D")
    assert torch.isnan(Dfull[:, :, N:]).all().item()


@pytest.mark.parametrize("shape", [(256, 256, 72), (512, 256, 136), (520, 776, 200), (300, 264, 1000),
                                   (1024, 1024, 4040), (256, 512, 120)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ring4_partial_first_step(shape):
    """K not a multiple of 64 on the fourth form (rung 10 and the library's
    choice): the partial step goes first, its chunks before each row's first
    element read as zeros.  Every output against the oracle, and bitwise
    equal to the same product with each operand row padded in front with
    zeros to whole 64-wide steps (which runs the whole-step path): the
    padding only adds exact zero products."""
    M, N, K = shape
    A, B = rand_case(M, N, K, 140 + K)
    ref, _ = oracle.gemm_nt(A, B)
    hk = -K % 64
    Ap = np.concatenate([np.zeros((M, hk), np.float16), A], axis=1)
    Bp = np.concatenate([np.zeros((N, hk), np.float16), B], axis=1)
    say(f"[gpu] ring4 partial first step {M}x{N}x{K} (padded K {K + hk}) rung 10")
    padded = host_bits(run(10, dev(Ap), dev(Bp)))
    for rung in (0, 10):
        assert supported(rung, M, N, K)
        D = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        say(f"[gpu] ring4 partial first step {M}x{N}x{K} rung {rung}")
        got = host_bits(run(rung, dev(A), dev(B), D))
        assert_parity(got, ref, K, f"rung {rung} {M}x{N}x{K}")
        if rung == 0 and g.plan(M, N, K, torch.cuda.get_device_properties(0).multi_processor_count)[0] != 10:
            continue   # the library runs another kernel on this shape (its own summation order)
        same = (got == padded) | (((got | padded) & 0x7FFF) == 0)   # +0 and -0 alike
        assert same.all(), f"rung {rung}: {int((~same).sum())} outputs differ from the front-padded product"
    # operands inside larger rows (leading dimension > K) through the strided form
    lda, ldb = K + 24, K + 8
    Apad = torch.zeros((M, lda), dtype=torch.float16)
    Apad[:, :K] = torch.from_numpy(A)
    Bpad = torch.zeros((N, ldb), dtype=torch.float16)
    Bpad[:, :K] = torch.from_numpy(B)
    say(f"[gpu] ring4 partial first step {M}x{N}x{K} strided lda={lda} ldb={ldb}")
    Ds = g.gemm_f16_nt_strided_batched(Apad.to(DEV)[:, :K], Bpad.to(DEV)[:, :K])
    torch.cuda.synchronize()
    assert_parity(host_bits(Ds[0]), ref, K, f"strided {M}x{N}x{K}")


@pytest.mark.parametrize("shape", [(8192, 8192, 512), (32768, 4096, 128), (16384, 4096, 192), (8192, 4096, 2040),
                                   (8192, 4096, 200), (8192, 4096, 136), (16384, 4096, 1000)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ring4_consecutive_tiles_bitwise(shape):
    """Many tiles per workgroup on the fourth form, whose last step loads
    the next tile's first step when K has at most 16 steps (odd step counts
    swap the stages; K not a multiple of 64 makes that first step the
    masked partial one): every output is bitwise equal to the third form's
    (rung 8, one tile at a time, the same MFMA sequence per accumulator), on
    repeated runs."""
    M, N, K = shape
    rng = np.random.default_rng(M + N + K)
    A = torch.from_numpy(rng.uniform(-1, 1, (M, K)).astype(np.float16)).to(DEV)
    B = torch.from_numpy(rng.uniform(-1, 1, (N, K)).astype(np.float16)).to(DEV)
    say(f"[gpu] consecutive tiles {M}x{N}x{K}: rung 10 against rung 8")
    if K % 64 == 0:
        ref = host_bits(run(8, A, B))
    else:   # rung 8 needs whole steps: pad each row in front with zeros
        hk = -K % 64
        z = torch.zeros((1, hk), dtype=torch.float16, device=DEV)
        ref = host_bits(run(8, torch.cat([z.expand(M, hk), A], 1).contiguous(), torch.cat([z.expand(N, hk), B], 1).contiguous()))
    D = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    for rep in range(3):
        got = host_bits(run(10, A, B, D))
        same = (got == ref) | (((got | ref) & 0x7FFF) == 0)
        assert same.all(), f"run {rep}: {int((~same).sum())} outputs differ from rung 8"
    rows, cols = sample_positions(M, N, 500, K)
    want, _ = oracle.gemm_nt_sampled(A.cpu().numpy(), B.cpu().numpy(), rows, cols)
    assert_parity(got[rows, cols], want, K, f"{M}x{N}x{K}")


@pytest.mark.parametrize("shape", [(4352, 4352, 1024), (4500, 4352, 1024)], ids=lambda s: "x".join(map(str, s)))
def test_library_small_last_round(shape):
    """gemm_f16_nt with a small last round of 256x256 tiles: rows up to the
    whole rounds come from R10 and the rest from 128x128 tiles.  Each part
    is bitwise equal to that rung run on the whole product (a tile's result
    depends only on its own rows, columns and K), and sampled outputs,
    boundary rows among them, match the oracle."""
    M, N, K = shape
    rung_top, m_top, rung_rest = g.plan(M, N, K, torch.cuda.get_device_properties(0).multi_processor_count)
    assert (rung_top, rung_rest) == (10, 9) and 0 < m_top < M, (rung_top, m_top, rung_rest)
    A, B = rand_case(M, N, K, 700 + M)
    dA, dB = dev(A), dev(B)
    say(f"[gpu] small last round {M}x{N}x{K}: rows [0, {m_top}) on rung 10, the rest on rung 9")
    D = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    got = host_bits(run(0, dA, dB, D))
    top = host_bits(run(10, dA, dB))
    rest = host_bits(run(9, dA, dB))
    assert np.array_equal(got[:m_top], top[:m_top])
    assert np.array_equal(got[m_top:], rest[m_top:])
    rows, cols = sample_positions(M, N, 1500, M)
    rows = np.concatenate([rows, np.full(64, m_top - 1), np.full(64, m_top), np.full(64, M - 1)])
    cols = np.concatenate([cols, np.random.default_rng(6).integers(0, N, 192)])
    want, _ = oracle.gemm_nt_sampled(A, B, rows, cols)
    assert_parity(got[rows, cols], want, K, f"small last round {shape}")


@pytest.mark.parametrize("case", [
    ("plain", 4096, 4096, 1024),     # one launch of the four-wave ring
    ("plain", 4352, 4352, 1024),     # two launches: whole rounds, then 128x128 tiles
    ("plain", 256, 256, 512),        # 128x128 tiles only
    ("plain", 300, 264, 0),          # K = 0: the fill kernel
    ("splitk", 256, 256, 8192),      # split K: partial sums, then the reduction
    ("plain", 6144, 4096, 1088),     # 384 x 256 tiles on every row
    ("plain", 16384, 4096, 1088),    # two launches: 384 x 256 tiles on the top rows, then 256 x 256
], ids=lambda c: "{}_{}x{}x{}".format(*c))
def test_graph_capture_replays(case):
    """Every launch the library makes can be captured into a HIP graph (no
    memset, no allocation, no host synchronisation): replays of the graph,
    with eager work and synchronisation between them, reproduce the eager
    result bit for bit."""
    kind, M, N, K = case
    rng = np.random.default_rng(M + N + K)
    A = torch.from_numpy(rng.uniform(-1, 1, (M, K)).astype(np.float16)).to(DEV)
    B = torch.from_numpy(rng.uniform(-1, 1, (N, K)).astype(np.float16)).to(DEV)
    D = torch.empty((M, N), dtype=torch.float16, device=DEV)
    ws = None
    if kind == "splitk":
        ws = torch.empty(max(16, g.splitk_workspace_bytes(M, N, K, 0)), dtype=torch.uint8, device=DEV)

    def call():
        if kind == "splitk":
            g.gemm_f16_nt_splitk(A, B, D, workspace=ws)
        else:
            g.gemm_f16_nt(A, B, D)

    say(f"[gpu] graph capture {case}")
    call()
    torch.cuda.synchronize()
    ref = host_bits(D)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(3):
        D.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(D), ref), f"replay {rep} differs from the eager result"


def test_non_default_stream_and_interleaving():
    M, N, K = 512, 512, 512
    A, B = rand_case(M, N, K, 79)
    ref, _ = oracle.gemm_nt(A, B)
    s = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(s):
        dA, dB = dev(A), dev(B)
        say("[gpu] side stream")
        X = torch.randn(2048, 2048, device=DEV)
        for rung in (0, 4, 5, 8, 9, 10):
            D = g.gemm_f16_nt(dA, dB) if rung == 0 else g.gemm_f16_nt_rung(rung, dA, dB)
            X = X * 1.0001          # unrelated work queued on the same stream
            s.synchronize()
            assert_parity(host_bits(D), ref, K, f"stream rung {rung}")


# ------------------------------------------- full sizes, every output

def sample_positions(M, N, count, seed):
    rng = np.random.default_rng(seed)
    rows = [0, M - 1, 255, 256, M // 2, M - 256] + list(rng.integers(0, M, count))
    cols = [0, N - 1, 256, 255, N // 2, N - 257] + list(rng.integers(0, N, count))
    return np.clip(np.array(rows), 0, M - 1), np.clip(np.array(cols), 0, N - 1)


def poisoned(M, N):
    """A device output buffer filled with NaN: an output the kernel never
    writes stays NaN and fails the comparison."""
    return torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)


@pytest.mark.parametrize("name", ["square_4096", "square_8192", "tall_32768x1024x8192"])
def test_full_size_workloads(name):
    """The three large workloads at their full sizes, in the launch the
    bench times (the library's choice): every output element against the
    full oracle at the stated tolerance, into a NaN-poisoned D ("GEMM I",
    "Where Steps 1-3 leave us": a kernel that passes a numerical check on
    every output)."""
    w = workloads.BY_NAME[name]
    A, B = inputs.operands(w.M, w.N, w.K, w.seed, w.dist)
    say(f"[gpu] full size {w.describe()} (library choice, every output)")
    dA, dB = dev(A), dev(B)
    D = poisoned(w.M, w.N)
    run(0, dA, dB, D)
    got = host_bits(D)
    ref, threads = oracle.gemm_nt(A, B)
    say(f"      oracle on {threads} threads done")
    worst = assert_parity(got, ref, w.K, name)
    say(f"      every output: worst err/tol = {worst:.3f}")
    # extra assertions: the sampled oracle at the tile seams, finite output
    rows, cols = sample_positions(w.M, w.N, 3000, w.seed)
    ref_s, _ = oracle.gemm_nt_sampled(A, B, rows, cols)
    np.testing.assert_array_equal(ref_s, ref[rows, cols])
    assert torch.isfinite(D).all().item()
    if name == "square_4096":
        for rung in (4, 5, 8, 9, 10, 11):
            say(f"[gpu] full size square_4096 on rung {rung} (every output)")
            Dr = poisoned(w.M, w.N)
            run(rung, dA, dB, Dr)
            assert_parity(host_bits(Dr), ref, w.K, f"{name} rung {rung}")
            del Dr


# ------------------------------------------- rung 11: 384 x 256 tiles

WIDE = 11
WIDE_SHAPES = [(384, 256, 128), (768, 512, 192), (400, 300, 256), (1000, 1032, 512), (1536, 2048, 1024),
               (3456, 2560, 2048)]


@pytest.mark.parametrize("shape", WIDE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_wide_parity(shape):
    """Rung 11 (each staged B band feeds two waves of 192 A rows) against the
    oracle on every output: whole and ragged tiles (the last tile row and
    column move back and overlap), one and several tiles per workgroup,
    into a NaN-poisoned D."""
    M, N, K = shape
    A, B = rand_case(M, N, K, 1100 + M + N + K)
    ref, _ = oracle.gemm_nt(A, B)
    say(f"[gpu] rung 11 M={M} N={N} K={K}")
    D = poisoned(M, N)
    run(WIDE, dev(A), dev(B), D)
    assert_parity(host_bits(D), ref, K, f"rung 11 {M}x{N}x{K}")
    # repeatable bit for bit
    D2 = poisoned(M, N)
    run(WIDE, dev(A), dev(B), D2)
    assert torch.equal(D.view(torch.int16), D2.view(torch.int16))


def test_wide_exact_pins():
    """All-ones (D = K exactly), small integers (every fp32 partial sum
    exact, so the result is bitwise the oracle's) and designed rows
    (round-to-nearest-even ties, overflow to inf, subnormals) on rung 11."""
    M, N = 768, 512
    for K in (128, 4096):
        say(f"[gpu] rung 11 all-ones K={K}")
        D = run(WIDE, dev(np.ones((M, K), np.float16)), dev(np.ones((N, K), np.float16)))
        assert torch.all(D == float(K)).item()
    rng = np.random.default_rng(11)
    K = 2048
    A = rng.integers(-4, 5, (M, K)).astype(np.float16)
    B = rng.integers(-4, 5, (N, K)).astype(np.float16)
    ref, _ = oracle.gemm_nt(A, B)
    say("[gpu] rung 11 small integers")
    assert np.array_equal(host_bits(run(WIDE, dev(A), dev(B))), ref)
    K = 128
    A = np.zeros((M, K), np.float16)
    B = np.zeros((N, K), np.float16)
    A[5, :2] = [1, 1]
    B[7, :2] = [2048, 1]
    B[8, :2] = [2048, 3]
    B[9, :2] = [65504, 16]
    A[400, 0] = 2.0 ** -12
    B[300, 0] = 2.0 ** -12
    B[301, 0] = 2.0 ** -13
    ref, _ = oracle.gemm_nt(A, B)
    say("[gpu] rung 11 designed rows")
    got = host_bits(run(WIDE, dev(A), dev(B)))
    assert np.array_equal(got, ref)
    d = as_f64(got)
    assert d[5, 7] == 2048 and d[5, 8] == 2052 and np.isinf(d[5, 9]) and d[400, 300] == 2.0 ** -24 and d[400, 301] == 0


def test_library_picks_wide_tiles():
    """Where 384 x 256 tiles fill the rounds of compute units better
    (6144 x 4096 x 4096: one round against 1.5), the library runs rung 11:
    bitwise equal to that rung, and every output against the oracle."""
    M, N, K = 6144, 4096, 4096
    A, B = rand_case(M, N, K, 1201)
    dA, dB = dev(A), dev(B)
    say(f"[gpu] library choice M={M} N={N} K={K} (rung 11)")
    D = poisoned(M, N)
    run(0, dA, dB, D)
    Dr = poisoned(M, N)
    run(WIDE, dA, dB, Dr)
    assert torch.equal(D.view(torch.int16), Dr.view(torch.int16))
    ref, _ = oracle.gemm_nt(A, B)
    assert_parity(host_bits(D), ref, K, "library 6144x4096x4096")


@pytest.mark.parametrize("shape", [(16384, 4096, 1088), (8192, 8192, 1088)], ids=lambda s: "x".join(map(str, s)))
def test_library_wide_top_rows(shape):
    """Where 256 x 256 tiles fill whole rounds but 384 x 256 tiles do not,
    the library runs rung 11 on the top rows that fill whole rounds of
    384-row tiles and rung 10 on the rest (16384 x 4096: two rounds of
    384-row tiles and one of 256-row tiles against four).  Each part is
    bitwise equal to its rung on the whole product, so the whole equals
    rung 10's output bitwise (both accumulate each block's k steps in the
    same order); sampled outputs, the boundary rows among them, match the
    oracle."""
    M, N, K = shape
    rung_top, m_top, rung_rest = g.plan(M, N, K, torch.cuda.get_device_properties(0).multi_processor_count)
    assert (rung_top, rung_rest) == (WIDE, 10) and 0 < m_top < M and m_top % 384 == 0, (rung_top, m_top, rung_rest)
    A, B = rand_case(M, N, K, 1300 + M)
    dA, dB = dev(A), dev(B)
    say(f"[gpu] wide top rows {M}x{N}x{K}: rows [0, {m_top}) on rung 11, the rest on rung 10")
    got = host_bits(run(0, dA, dB, poisoned(M, N)))
    top = host_bits(run(WIDE, dA, dB, poisoned(M, N)))
    whole = host_bits(run(10, dA, dB, poisoned(M, N)))
    assert np.array_equal(got[:m_top], top[:m_top])
    assert np.array_equal(got, whole)
    rows, cols = sample_positions(M, N, 1500, M + 1)
    rows = np.concatenate([rows, np.full(64, m_top - 1), np.full(64, m_top), np.full(64, M - 1)])
    cols = np.concatenate([cols, np.random.default_rng(7).integers(0, N, 192)])
    want, _ = oracle.gemm_nt_sampled(A, B, rows, cols)
    assert_parity(got[rows, cols], want, K, f"wide top rows {shape}")


def test_wide_rejects_shapes_it_does_not_take():
    A, B = dev(np.ones((256, 128), np.float16)), dev(np.ones((256, 128), np.float16))
    with pytest.raises(g.GemmError) as e:
        g.gemm_f16_nt_rung(WIDE, A, B)           # M < 384
    assert e.value.status == g.UNSUPPORTED


# ------------------------------------------- general operands (any K, alignment)

GENERAL = [(1, 1, 1), (5, 3, 7), (64, 64, 13), (130, 70, 100), (257, 129, 1001), (300, 260, 9), (128, 128, 66)]


@pytest.mark.parametrize("rung", [0, 3, 4, 9])
@pytest.mark.parametrize("shape", GENERAL, ids=lambda s: "x".join(map(str, s)))
def test_general_k(rung, shape):
    """K % 8 != 0: rows are not 16-byte aligned.  The library runs the ring
    with register-staged loads (K >= 8) or R3's general form (K < 8); rung 3
    always runs the latter, rungs 4 and 9 the former (K >= 8 only)."""
    M, N, K = shape
    A, B = rand_case(M, N, K, 200 + M + N + K)
    if rung in (4, 9) and K < 8:
        with pytest.raises(g.GemmError) as e:
            g.gemm_f16_nt_rung(rung, dev(A), dev(B))
        assert e.value.status == g.UNSUPPORTED
        return
    ref, _ = oracle.gemm_nt(A, B)
    say(f"[gpu] general K rung={rung} M={M} N={N} K={K}")
    D = run(rung, dev(A), dev(B))
    assert_parity(host_bits(D), ref, K, f"general rung {rung} {M}x{N}x{K}")


def _offset_view(X: np.ndarray, off: int):
    """Contiguous device view of X starting `off` elements into a buffer
    (2-byte aligned, not 16-byte aligned for odd off)."""
    buf = torch.zeros(X.size + off + 8, dtype=torch.float16, device=DEV)
    v = buf[off: off + X.size].view(X.shape)
    v.copy_(torch.from_numpy(np.ascontiguousarray(X)).to(DEV))
    return v


@pytest.mark.parametrize("offs", [(1, 0, 0), (0, 3, 0), (0, 0, 5), (7, 1, 3)], ids=lambda o: "a{}b{}d{}".format(*o))
def test_misaligned_operands(offs):
    M, N, K = 200, 136, 96
    A, B = rand_case(M, N, K, 301)
    ref, _ = oracle.gemm_nt(A, B)
    dA, dB = _offset_view(A, offs[0]), _offset_view(B, offs[1])
    D = _offset_view(np.zeros((M, N), np.float16), offs[2])
    for rung in (0, 3, 4, 9):
        say(f"[gpu] misaligned offsets {offs} rung={rung}")
        D.fill_(float("nan"))
        run(rung, dA, dB, D)
        assert_parity(host_bits(D), ref, K, f"misaligned {offs} rung {rung}")
    with pytest.raises(g.GemmError) as e:     # the other rungs refuse them
        g.gemm_f16_nt_rung(5, dA, dB, D)
    assert e.value.status == g.UNSUPPORTED


@pytest.mark.parametrize("shape", [(128, 30000, 320), (100, 28000, 203)], ids=lambda s: "x".join(map(str, s)))
def test_library_thin_shapes(shape):
    """M well under 256 with enough tiles not to be tile-starved: the library
    takes 128 x 128 tiles (aligned rows, and register-staged ones for
    K % 8 != 0), which it checks against the oracle on every output."""
    M, N, K = shape
    A, B = rand_case(M, N, K, 40 + M)
    ref, _ = oracle.gemm_nt(A, B)
    assert g.plan(M, N, K, 256)[0] == 9
    say(f"[gpu] thin shape {M}x{N}x{K}")
    D = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    run(0, dev(A), dev(B), D)
    assert_parity(host_bits(D), ref, K, f"thin {M}x{N}x{K}")


# ------------------------ general operands on the pipelined ring (K >= 8)

# (M, N, K, element offsets of A, B and D).  Operands whose rows are off
# 16-byte boundaries run the ring with register-staged loads: on 128 x 128
# tiles when 256 x 256 ones would leave most compute units idle (up to 102
# tiles on 256 CUs), on 256 x 256 tiles otherwise.
STAGED = [
    (200, 136, 8, (0, 0, 0)),
    (300, 260, 63, (0, 0, 0)),
    (257, 385, 65, (1, 0, 0)),
    (1000, 1000, 1001, (0, 0, 0)),
    (2816, 2816, 9, (0, 0, 0)),
    (3072, 2816, 133, (0, 0, 0)),
    (2600, 2900, 517, (1, 3, 5)),
    (2816, 3072, 1000, (0, 1, 0)),
    (2944, 2816, 255, (7, 0, 2)),
]


def _staged_operands(A, B, M, N, offs):
    dA, dB = _offset_view(A, offs[0]), _offset_view(B, offs[1])
    D = _offset_view(np.full((M, N), np.nan, np.float16), offs[2])
    return dA, dB, D


@pytest.mark.parametrize("shape", STAGED, ids=lambda s: "{}x{}x{}_a{}b{}d{}".format(*s[:3], *s[3]))
def test_staged_ring_general_operands(shape):
    M, N, K, offs = shape
    A, B = rand_case(M, N, K, 700 + K)
    ref, _ = oracle.gemm_nt(A, B)
    dA, dB, D = _staged_operands(A, B, M, N, offs)
    say(f"[gpu] staged ring M={M} N={N} K={K} offsets={offs}")
    run(0, dA, dB, D)
    assert_parity(host_bits(D), ref, K, f"staged {M}x{N}x{K} {offs}")


@pytest.mark.parametrize("shape", [(384, 320, 75, (3, 1, 0)), (2816, 2816, 203, (1, 0, 3))],
                         ids=lambda s: "{}x{}x{}".format(*s[:3]))
def test_staged_ring_selection_bitwise(shape):
    """A selects one element of each B row per output: D = B[:, pick]^T
    exactly.  Picks at both ends of K land in the chunk that crosses K and
    in the first one."""
    M, N, K, offs = shape
    rng = np.random.default_rng(K)
    pick = rng.integers(0, K, M)
    pick[:10] = [K - 1, K - 2, K - 3, K - 7, K - 8, K - 9, 0, 1, 7, 8]
    A = np.zeros((M, K), np.float16)
    A[np.arange(M), pick] = 1
    B = rng.uniform(-60000, 60000, (N, K)).astype(np.float16)
    dA, dB, D = _staged_operands(A, B, M, N, offs)
    say(f"[gpu] staged selection M={M} N={N} K={K} offsets={offs}")
    run(0, dA, dB, D)
    assert np.array_equal(host_bits(D), B[:, pick].T.view(np.uint16))


@pytest.mark.parametrize("shape", [(264, 256, 1001, (0, 0, 0)), (2816, 2816, 777, (5, 2, 1))],
                         ids=lambda s: "{}x{}x{}".format(*s[:3]))
def test_staged_ring_small_integers_bitwise(shape):
    """Integer sums below 2^24 are exact in any fp32 order: bitwise parity."""
    M, N, K, offs = shape
    rng = np.random.default_rng(M + K)
    A = rng.integers(-4, 5, (M, K)).astype(np.float16)
    B = rng.integers(-4, 5, (N, K)).astype(np.float16)
    ref, _ = oracle.gemm_nt(A, B)
    dA, dB, D = _staged_operands(A, B, M, N, offs)
    say(f"[gpu] staged small-int M={M} N={N} K={K} offsets={offs}")
    run(0, dA, dB, D)
    got = host_bits(D)
    assert np.array_equal(got, ref), f"{np.sum(got != ref)} mismatches"


# ------------------------------------------------- strided / batched form

def _padded3(Xs, ld: int):
    """Device (batch, rows, cols) view of the matrices Xs in one buffer with
    row pitch ld (ld >= cols) and batch stride rows * ld."""
    rows, cols = Xs[0].shape
    buf = torch.zeros((len(Xs), rows, ld), dtype=torch.float16)
    for i, X in enumerate(Xs):
        buf[i, :, :cols] = torch.from_numpy(X)
    return buf.to(DEV)[:, :, :cols]


def _padded(X: np.ndarray, ld: int):
    """Device tensor holding X (rows x cols) with row pitch ld (ld >= cols)."""
    rows, cols = X.shape
    buf = torch.zeros((rows, ld), dtype=torch.float16)
    buf[:, :cols] = torch.from_numpy(X)
    return buf.to(DEV)[:, :cols]


@pytest.mark.parametrize("case", [
    # batch, M, N, K, pad_a, pad_b, pad_d, broadcast_b
    (3, 300, 260, 136, 8, 24, 4, False),
    (2, 512, 512, 256, 0, 0, 0, False),      # whole tiles: the fast variant
    (2, 256, 256, 64, 64, 0, 0, False),      # whole tiles with padded A rows
    (4, 130, 70, 40, 16, 8, 12, True),       # B shared by every batch entry
    (1, 1, 1, 8, 0, 0, 0, False),
    (3, 97, 45, 21, 3, 5, 1, False),         # K % 8 != 0, odd pitches: register-staged loads
    (2, 256, 256, 128, 4, 0, 0, True),       # whole tiles but lda % 8 != 0: register-staged loads
    (4, 1536, 1536, 200, 3, 0, 2, False),    # odd pitches on 256 x 256 tiles (144 of them)
], ids=lambda c: "b{}_{}x{}x{}".format(*c[:4]))
def test_strided_batched(case):
    batch, M, N, K, pa, pb, pd, bcast = case
    rng = np.random.default_rng(batch * 1000 + M + N + K)
    As = [rng.uniform(-1, 1, (M, K)).astype(np.float16) for _ in range(batch)]
    Bs = [rng.uniform(-1, 1, (N, K)).astype(np.float16) for _ in range(1 if bcast else batch)]
    A = _padded3(As, K + pa)
    B = _padded3(Bs, K + pb)
    assert A.stride(1) == K + pa and B.stride(1) == K + pb   # row pitches really padded
    if bcast:
        B = B[0]
    Dfull = torch.full((batch, M, N + pd), float("nan"), dtype=torch.float16, device=DEV)
    D = Dfull[:, :, :N]
    say(f"[gpu] strided batch={batch} M={M} N={N} K={K} pads=({pa},{pb},{pd}) bcast={bcast}")
    g.gemm_f16_nt_strided_batched(A, B, D)
    torch.cuda.synchronize()
    for b in range(batch):
        ref, _ = oracle.gemm_nt(As[b], Bs[0 if bcast else b])
        assert_parity(host_bits(D[b].contiguous()), ref, K, f"batch {b}")
    if pd:  # the padding columns of D are never written
        assert torch.isnan(Dfull[:, :, N:]).all().item()


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
def test_attention_scores(layout):
    B_, H, Sq, Sk, d = 2, 3, 200, 264, 64
    rng = np.random.default_rng(7 if layout == "bhsd" else 8)
    q = rng.uniform(-1, 1, (B_, H, Sq, d)).astype(np.float16)
    k = rng.uniform(-1, 1, (B_, H, Sk, d)).astype(np.float16)
    if layout == "bhsd":
        Q, Kt = dev(q), dev(k)
    else:  # heads interleaved in the rows: (B, S, H, d) storage viewed as (B, H, S, d)
        Q = dev(np.ascontiguousarray(q.transpose(0, 2, 1, 3))).transpose(1, 2)
        Kt = dev(np.ascontiguousarray(k.transpose(0, 2, 1, 3))).transpose(1, 2)
    say(f"[gpu] attention scores layout={layout}")
    S = g.attention_scores(Q, Kt)
    torch.cuda.synchronize()
    assert S.shape == (B_, H, Sq, Sk)
    for b in range(B_):
        for h in range(H):
            ref, _ = oracle.gemm_nt(q[b, h], k[b, h])
            assert_parity(host_bits(S[b, h].contiguous()), ref, d, f"b{b} h{h}")


@pytest.mark.parametrize("K", [64, 128, 200])
def test_strided_unaligned_output_rows(K):
    """Row pitch and batch stride of D that leave rows 2-byte aligned only
    (K = 64 on R4's edge tiles, longer K on the four-wave ring)."""
    batch, M, N = 2, 260, 257
    rng = np.random.default_rng(31)
    As = [rng.uniform(-1, 1, (M, K)).astype(np.float16) for _ in range(batch)]
    Bs = [rng.uniform(-1, 1, (N, K)).astype(np.float16) for _ in range(batch)]
    ldd, sd = N + 3, (M - 1) * (N + 3) + N + 5
    flat = torch.full((sd * batch + 16,), float("nan"), dtype=torch.float16, device=DEV)
    D = flat.as_strided((batch, M, N), (sd, ldd, 1))
    say(f"[gpu] strided unaligned D ldd={ldd} sd={sd}")
    g.gemm_f16_nt_strided_batched(torch.stack([dev(a) for a in As]), torch.stack([dev(b) for b in Bs]), D)
    torch.cuda.synchronize()
    for b in range(batch):
        ref, _ = oracle.gemm_nt(As[b], Bs[b])
        assert_parity(host_bits(D[b].contiguous()), ref, K, f"batch {b}")


# ------------------------------------------------------------ split-K form

@pytest.mark.parametrize("case", [
    (256, 256, 512, 0), (256, 256, 512, 2), (256, 256, 512, 4), (256, 256, 512, 8),
    (300, 260, 520, 3), (200, 130, 200, 2), (128, 64, 64, 4), (512, 256, 2048, 16), (1, 1, 8, 2),
    (256, 256, 65536, 0), (256, 256, 8192, 64),
], ids=lambda c: "{}x{}x{}_s{}".format(*c))
def test_splitk(case):
    M, N, K, splits = case
    A, B = rand_case(M, N, K, 500 + M + N + K + splits)
    ref, _ = oracle.gemm_nt(A, B)
    dA, dB = dev(A), dev(B)
    D = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    say(f"[gpu] split-K M={M} N={N} K={K} splits={splits}")
    g.gemm_f16_nt_splitk(dA, dB, D, splits=splits)
    torch.cuda.synchronize()
    assert_parity(host_bits(D), ref, K, f"split-K {case}")
    first = host_bits(D)
    g.gemm_f16_nt_splitk(dA, dB, D, splits=splits)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(D), first)        # fixed slice order: repeatable


@pytest.mark.parametrize("shape", [(6144, 6144, 6144), (6280, 5888, 4096)], ids=lambda s: "x".join(map(str, s)))
def test_splitk_whole_rounds_plus_split_rows(shape):
    """The library's split for a small last round of tiles: the top rows
    run unsplit, the rest split K (ragged M included).  Sampled outputs
    (rows on both sides of the boundary among them) against the oracle;
    every output written; repeatable."""
    M, N, K = shape
    m_top, splits = g.splitk_plan(M, N, K, torch.cuda.get_device_properties(0).multi_processor_count)
    assert m_top > 0 and splits > 1, (m_top, splits)
    A, B = rand_case(M, N, K, 600 + M)
    dA, dB = dev(A), dev(B)
    D = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    say(f"[gpu] split-K whole rounds {M}x{N}x{K}: {m_top} rows unsplit, {splits} slices")
    g.gemm_f16_nt_splitk(dA, dB, D)
    torch.cuda.synchronize()
    assert not torch.isnan(D).any().item()
    rows, cols = sample_positions(M, N, 2000, M + K)
    rows = np.concatenate([rows, np.full(64, m_top - 1), np.full(64, m_top), np.full(64, M - 1)])
    cols = np.concatenate([cols, np.random.default_rng(5).integers(0, N, 192)])
    want, _ = oracle.gemm_nt_sampled(A, B, rows, cols)
    got = host_bits(D)
    assert_parity(got[rows, cols], want, K, f"split rows {shape}")
    g.gemm_f16_nt_splitk(dA, dB, D)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(D), got)


def test_splitk_exact_pins():
    """Small integers: every fp32 partial and their sum are exact, so the
    split result equals the oracle bit for bit; all-ones gives K."""
    rng = np.random.default_rng(44)
    M, N, K = 256, 192, 4096
    A = rng.integers(-4, 5, (M, K)).astype(np.float16)
    B = rng.integers(-4, 5, (N, K)).astype(np.float16)
    ref, _ = oracle.gemm_nt(A, B)
    say("[gpu] split-K small integers")
    D = g.gemm_f16_nt_splitk(dev(A), dev(B), splits=8)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(D), ref)
    ones = torch.ones((256, 8192), dtype=torch.float16, device=DEV)
    D = g.gemm_f16_nt_splitk(ones, ones, splits=16)
    torch.cuda.synchronize()
    assert torch.all(D.float() == 8192).item()


def test_splitk_rejects_small_workspace():
    A = torch.ones((256, 512), dtype=torch.float16, device=DEV)
    ws = torch.empty(1024, dtype=torch.uint8, device=DEV)
    D = torch.full((256, 256), 7.0, dtype=torch.float16, device=DEV)
    say("[gpu] split-K small workspace")
    with pytest.raises(g.GemmError) as e:
        g.gemm_f16_nt_splitk(A, A, D, splits=4, workspace=ws)
    assert e.value.status == g.INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(D == 7.0).item()


# ------------------------------- products beyond the five fixed workloads

@pytest.mark.parametrize("name", [w.name for w in workloads.EXTRA_WORKLOADS])
def test_extra_workloads_sampled(name):
    """The general-shape, batched and attention-score products that
    `bench.py --suite` times, at full size and in the same layouts, on
    sampled outputs of every batch entry; every output element is written
    (D starts as NaN)."""
    w = workloads.EXTRA_BY_NAME[name]
    A3, B3 = inputs.batched_operands(w.batch, w.M, w.N, w.K, w.seed, w.dist)
    say(f"[gpu] extra product {w.describe()}")
    D = torch.full((w.batch, w.M, w.N), float("nan"), dtype=torch.float16, device=DEV)
    if w.kind == "gemm":
        g.gemm_f16_nt(dev(A3[0]), dev(B3[0]), D[0])
    elif w.kind == "splitk":
        g.gemm_f16_nt_splitk(dev(A3[0]), dev(B3[0]), D[0])
    elif w.kind == "heads_rows":
        # (S, H, d) storage read as H products: leading dimension H*d, batch stride d
        A = dev(A3.transpose(1, 0, 2)).transpose(0, 1)
        B = dev(B3.transpose(1, 0, 2)).transpose(0, 1)
        assert A.stride() == (w.K, w.batch * w.K, 1)
        g.gemm_f16_nt_strided_batched(A, B, D)
    else:
        g.gemm_f16_nt_strided_batched(dev(A3), dev(B3), D)
    torch.cuda.synchronize()
    assert not torch.isnan(D).any().item(), "output elements left unwritten"
    per = 3000 if w.batch == 1 else 200
    worst = 0.0
    for b in range(w.batch):
        rows, cols = sample_positions(w.M, w.N, per, w.seed * 100 + b)
        ref, _ = oracle.gemm_nt_sampled(A3[b], B3[b], rows, cols)
        got = host_bits(D[b][torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)])
        worst = max(worst, assert_parity(got, ref, w.K, f"{name} entry {b}"))
    say(f"      worst err/tol = {worst:.3f}")


# ----------------------------------------- random shapes through every path

def _random_shapes(count, seed):
    """Shapes that reach every branch of the library's choice: tiny and
    tile-starved (128 x 128 tiles), thin, ragged M and N on the four-wave
    ring, K not a multiple of 64 (partial first step), K not a multiple of
    8 (register-staged rows), K < 8 (element copies), one k step."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        kind = i % 6
        if kind == 0:
            M, N, K = rng.integers(1, 300, 3)
        elif kind == 1:
            M, N = rng.integers(256, 2600, 2)
            K = 8 * int(rng.integers(9, 200))
        elif kind == 2:
            M, N = rng.integers(256, 1800, 2)
            K = 64 * int(rng.integers(2, 20))
        elif kind == 3:
            M, N = rng.integers(1, 1500, 2)
            K = int(rng.integers(8, 700)) | 1          # odd K: rows off 16-byte boundaries
        elif kind == 4:
            M, N, K = rng.integers(1, 40, 3)
            K = int(K) % 7 + 1                           # K < 8
        else:
            M = int(rng.integers(1, 200))
            N = int(rng.integers(2000, 9000))
            K = int(rng.choice([64, 8 * int(rng.integers(1, 64))]))
        out.append((int(M), int(N), int(K)))
    return out


@pytest.mark.parametrize("shape", _random_shapes(36, 2024), ids=lambda s: "x".join(map(str, s)))
def test_random_shapes_library_choice(shape):
    """The library's choice on random shapes: every output written (D
    starts as NaN) and sampled outputs, the last row and column among them,
    within the tolerance of the oracle; the result repeats bitwise."""
    M, N, K = shape
    A, B = rand_case(M, N, K, 3000 + M * 7 + N * 3 + K)
    dA, dB = dev(A), dev(B)
    say(f"[gpu] random shape M={M} N={N} K={K} plan={g.plan(M, N, K, torch.cuda.get_device_properties(0).multi_processor_count)}")
    D = run(0, dA, dB, poisoned(M, N))
    got = host_bits(D)
    assert not np.isnan(as_f64(got)).any(), "output elements left unwritten"
    rows, cols = sample_positions(M, N, 600, M + N + K)
    want, _ = oracle.gemm_nt_sampled(A, B, rows, cols)
    assert_parity(got[rows, cols], want, K, f"random {shape}")
    again = host_bits(run(0, dA, dB, poisoned(M, N)))
    assert np.array_equal(got, again)


def _random_strided(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        batch = int(rng.integers(1, 5))
        M, N = (int(x) for x in rng.integers(1, 700, 2))
        K = int(rng.choice([int(rng.integers(1, 600)), 8 * int(rng.integers(1, 80))]))
        pad_a, pad_b, pad_d = (int(x) for x in rng.integers(0, 24, 3))
        bcast = int(rng.integers(0, 3))     # 0: none, 1: A shared by the batch, 2: B shared
        out.append((batch, M, N, K, pad_a, pad_b, pad_d, bcast))
    return out


@pytest.mark.parametrize("case", _random_strided(24, 77), ids=lambda c: "b{}_{}x{}x{}_pad{}-{}-{}_bc{}".format(*c))
def test_random_strided_batched(case):
    """The strided-batched entry on random batches, shapes and padded row
    pitches (any 2-byte alignment), with A or B broadcast over the batch:
    every output written and every batch entry's sampled outputs within the
    oracle's tolerance."""
    batch, M, N, K, pad_a, pad_b, pad_d, bcast = case
    rng = np.random.default_rng(M + N + K + batch)
    ba = 1 if bcast == 1 else batch
    bb = 1 if bcast == 2 else batch
    A3 = rng.uniform(-1, 1, (ba, M, K)).astype(np.float16)
    B3 = rng.uniform(-1, 1, (bb, N, K)).astype(np.float16)
    Af = torch.zeros((ba, M, K + pad_a), dtype=torch.float16, device=DEV)
    Bf = torch.zeros((bb, N, K + pad_b), dtype=torch.float16, device=DEV)
    Af[:, :, :K] = dev(A3)
    Bf[:, :, :K] = dev(B3)
    A = Af[:, :, :K] if bcast != 1 else Af[0, :, :K]
    B = Bf[:, :, :K] if bcast != 2 else Bf[0, :, :K]
    Df = torch.full((batch, M, N + pad_d), float("nan"), dtype=torch.float16, device=DEV)
    D = Df[:, :, :N]
    say(f"[gpu] random strided {case}")
    g.gemm_f16_nt_strided_batched(A, B, D)
    torch.cuda.synchronize()
    got = D.cpu().view(torch.int16).numpy().view(np.uint16)
    assert not np.isnan(as_f64(got)).any(), "output elements left unwritten"
    assert torch.isnan(Df[:, :, N:]).all().item(), "the row padding of D was written"
    for b in range(batch):
        rows, cols = sample_positions(M, N, 150, b + 1)
        want, _ = oracle.gemm_nt_sampled(A3[0 if ba == 1 else b], B3[0 if bb == 1 else b], rows, cols)
        assert_parity(got[b][rows, cols], want, K, f"strided {case} entry {b}")


def _random_splitk(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        M, N = (int(x) for x in rng.integers(1, 700, 2))
        form = i % 3        # whole 64-wide steps, a ragged last step, any K
        K = [64 * int(rng.integers(2, 129)), 8 * int(rng.integers(9, 1025)), int(rng.integers(1, 3000))][form]
        splits = 0 if rng.random() < 0.3 else int(rng.integers(2, 65))     # 0: the library's count
        out.append((M, N, K, splits))
    return out


@pytest.mark.parametrize("case", _random_splitk(18, 91), ids=lambda c: "{}x{}x{}_s{}".format(*c))
def test_random_splitk(case):
    """The split-K entry on random shapes and slice counts (more slices than
    64-wide steps among them, K with a ragged last step, K the fast path
    does not take): every output written (D starts as NaN), sampled outputs
    within the oracle's tolerance, and the fixed slice order repeats the
    result bitwise."""
    M, N, K, splits = case
    A, B = rand_case(M, N, K, 4000 + M * 5 + N * 11 + K + splits)
    dA, dB = dev(A), dev(B)
    say(f"[gpu] random split-K M={M} N={N} K={K} splits={splits} "
        f"workspace={g.splitk_workspace_bytes(M, N, K, splits)}")
    D = poisoned(M, N)
    g.gemm_f16_nt_splitk(dA, dB, D, splits=splits)
    torch.cuda.synchronize()
    got = host_bits(D)
    assert not np.isnan(as_f64(got)).any(), "output elements left unwritten"
    rows, cols = sample_positions(M, N, 600, M * 3 + N + K)
    want, _ = oracle.gemm_nt_sampled(A, B, rows, cols)
    assert_parity(got[rows, cols], want, K, f"random split-K {case}")
    D = poisoned(M, N)
    g.gemm_f16_nt_splitk(dA, dB, D, splits=splits)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(D), got)


# ------------------------------------- rung 12: one side of at most 96 rows

SKINNY = [(1, 1, 8), (5, 300, 100), (16, 4096, 4096), (64, 1000, 777), (33, 17, 1030), (300, 40, 515),
          (50, 5000, 4095), (4000, 7, 333), (64, 64, 64), (16, 200, 14336), (64, 2048, 2047), (2, 70000, 64),
          (48, 3000, 40), (64, 65, 9), (7, 9000, 2048), (80, 3000, 1000), (96, 5000, 4095), (4000, 90, 333),
          (72, 2048, 64), (96, 96, 4096)]


@pytest.mark.parametrize("shape", SKINNY, ids=lambda s: "x".join(map(str, s)))
def test_skinny_parity(shape):
    """Rung 12 (and the library's choice where it picks rung 12) against the
    full oracle, output by output, into a NaN-poisoned D: either side
    small, ragged row counts, K with a crossing chunk (K % 32 != 0) and K
    % 8 != 0 (rows on 2-byte boundaries), more waves than k chunks."""
    M, N, K = shape
    A, B = rand_case(M, N, K, 7000 + M + 3 * N + K)
    ref, _ = oracle.gemm_nt(A, B)
    dA, dB = dev(A), dev(B)
    say(f"[gpu] rung 12 M={M} N={N} K={K} plan={g.plan(M, N, K, 256)}")
    D = run(12, dA, dB, poisoned(M, N))
    assert_parity(host_bits(D), ref, K, f"rung 12 {shape}")
    if g.plan(M, N, K, 256)[0] == 12:
        D0 = run(0, dA, dB, poisoned(M, N))
        assert np.array_equal(host_bits(D0), host_bits(D))


@pytest.mark.parametrize("shape", [(16, 4096, 8192), (4096, 40, 2040), (64, 512, 1000)], ids=lambda s: "x".join(map(str, s)))
def test_skinny_exact_pins(shape):
    """Small integers: every fp32 partial sum and the waves' total are
    exact, so rung 12 equals the oracle bit for bit; all-ones gives K."""
    M, N, K = shape
    rng = np.random.default_rng(M + N + K)
    A = rng.integers(-4, 5, (M, K)).astype(np.float16)
    B = rng.integers(-4, 5, (N, K)).astype(np.float16)
    ref, _ = oracle.gemm_nt(A, B)
    say(f"[gpu] rung 12 small integers {shape}")
    D = run(12, dev(A), dev(B), poisoned(M, N))
    assert np.array_equal(host_bits(D), ref)
    ones = torch.ones((M, K), dtype=torch.float16, device=DEV)
    onesb = torch.ones((N, K), dtype=torch.float16, device=DEV)
    D = run(12, ones, onesb, poisoned(M, N))
    assert torch.all(D.float() == float(K)).item()


@pytest.mark.parametrize("offs", [(1, 0, 0), (0, 3, 5), (7, 1, 3)], ids=lambda o: "a{}b{}d{}".format(*o))
def test_skinny_misaligned_and_pitched(offs):
    """Rung 12 on operands at 2-byte offsets (through the library's choice)
    and on padded row pitches with batch 1 (through the strided entry),
    against the full oracle; the padding of D stays unwritten."""
    M, N, K = 24, 3000, 1001
    A, B = rand_case(M, N, K, 7100 + sum(offs))
    ref, _ = oracle.gemm_nt(A, B)
    assert g.plan(M, N, K, 256)[0] == 12
    say(f"[gpu] rung 12 offsets {offs}")
    dA, dB = _offset_view(A, offs[0]), _offset_view(B, offs[1])
    D = _offset_view(np.full((M, N), np.nan, np.float16), offs[2])
    g.gemm_f16_nt(dA, dB, D)
    torch.cuda.synchronize()
    assert_parity(host_bits(D), ref, K, f"rung 12 offsets {offs}")
    pa, pb, pd = 3 + offs[0], 5 + offs[1], 7 + offs[2]
    Af = torch.zeros((1, M, K + pa), dtype=torch.float16, device=DEV)
    Bf = torch.zeros((1, N, K + pb), dtype=torch.float16, device=DEV)
    Af[0, :, :K] = dev(A)
    Bf[0, :, :K] = dev(B)
    Df = torch.full((1, M, N + pd), float("nan"), dtype=torch.float16, device=DEV)
    g.gemm_f16_nt_strided_batched(Af[:, :, :K], Bf[:, :, :K], Df[:, :, :N])
    torch.cuda.synchronize()
    assert_parity(host_bits(Df[0, :, :N]), ref, K, f"rung 12 pitched {offs}")
    assert torch.isnan(Df[:, :, N:]).all().item()


def test_skinny_repeatable_and_split_k_entry():
    """Rung 12's fixed summation order repeats bitwise; the split-K entry
    with one slice runs the library's choice (rung 12 here) and equals it."""
    M, N, K = 32, 8192, 8192
    A, B = rand_case(M, N, K, 7200)
    dA, dB = dev(A), dev(B)
    say("[gpu] rung 12 repeatable")
    first = host_bits(run(0, dA, dB, poisoned(M, N)))
    for _ in range(3):
        assert np.array_equal(host_bits(run(0, dA, dB, poisoned(M, N))), first)
    D = poisoned(M, N)
    g.gemm_f16_nt_splitk(dA, dB, D, splits=1)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(D), first)
    rows, cols = sample_positions(M, N, 800, 7)
    want, _ = oracle.gemm_nt_sampled(A, B, rows, cols)
    assert_parity(first[rows, cols], want, K, "rung 12 32x8192x8192")



# ---------------- rung 13: K split among the waves of small tiles of both sides

def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


# one shape per tile of rung 13 (16*mt rows of the side with fewer rows by
# 16*nf of the other), both sides over 96 rows, either orientation, ragged
# tile rows and columns, K with a crossing chunk and K % 8 != 0
KSPLIT = [((100, 100, 1001), (1, 1, 2, 8)), ((260, 250, 1001), (1, 2, 2, 8)), ((1000, 130, 1001), (2, 2, 1, 8)),
          ((130, 2100, 2056), (2, 4, 1, 8)), ((333, 1500, 1001), (3, 4, 1, 8)), ((2100, 130, 4095), (2, 4, 1, 8)),
          ((300, 2000, 3000), (3, 4, 1, 8)), ((97, 97, 8), (1, 1, 2, 8)), ((140, 700, 40), None),
          ((130, 6000, 1001), (2, 4, 1, 4)), ((6000, 130, 1001), (2, 4, 1, 4)), ((260, 3000, 1001), (4, 4, 1, 4)),
          ((3000, 260, 1001), (4, 4, 1, 4)), ((200, 4096, 4096), (4, 4, 1, 4))]


@pytest.mark.parametrize("shape,tile", KSPLIT, ids=lambda s: "x".join(map(str, s)) if s else "any")
def test_ksplit_parity(shape, tile):
    """Rung 13 against the full oracle, output by output, into a
    NaN-poisoned D, on every tile it launches; where the library's choice
    is rung 13 it returns the same bits."""
    M, N, K = shape
    if tile is not None:
        assert g.ksplit_plan(13, M, N, K, 256) == tile
    A, B = rand_case(M, N, K, 7300 + M + 3 * N + K)
    ref, _ = oracle.gemm_nt(A, B)
    dA, dB = dev(A), dev(B)
    say(f"[gpu] rung 13 M={M} N={N} K={K} tile={g.ksplit_plan(13, M, N, K, _cus())} plan={g.plan(M, N, K, _cus())}")
    D = run(13, dA, dB, poisoned(M, N))
    assert_parity(host_bits(D), ref, K, f"rung 13 {shape}")
    if g.plan(M, N, K, _cus())[0] == 13:
        D0 = run(0, dA, dB, poisoned(M, N))
        assert np.array_equal(host_bits(D0), host_bits(D))


@pytest.mark.parametrize("shape", [(256, 1024, 8192), (4096, 130, 2040), (300, 2000, 1000), (130, 6000, 1001),
                                   (3000, 260, 1001)], ids=lambda s: "x".join(map(str, s)))
def test_ksplit_exact_pins(shape):
    """Small integers: every fp32 partial sum and the waves' total are
    exact, so rung 13 equals the oracle bit for bit; all-ones gives K."""
    M, N, K = shape
    rng = np.random.default_rng(M + N + K + 13)
    A = rng.integers(-4, 5, (M, K)).astype(np.float16)
    B = rng.integers(-4, 5, (N, K)).astype(np.float16)
    ref, _ = oracle.gemm_nt(A, B)
    say(f"[gpu] rung 13 small integers {shape}")
    D = run(13, dev(A), dev(B), poisoned(M, N))
    assert np.array_equal(host_bits(D), ref)
    ones = torch.ones((M, K), dtype=torch.float16, device=DEV)
    onesb = torch.ones((N, K), dtype=torch.float16, device=DEV)
    D = run(13, ones, onesb, poisoned(M, N))
    assert torch.all(D.float() == float(K)).item()


@pytest.mark.parametrize("offs", [(1, 0, 0), (0, 3, 5), (7, 1, 3)], ids=lambda o: "a{}b{}d{}".format(*o))
def test_ksplit_misaligned_and_pitched(offs):
    """Rung 13 on operands at 2-byte offsets (through the library's choice)
    and on padded row pitches with batch 1 (through the strided entry),
    against the full oracle; the padding of D stays unwritten."""
    M, N, K = 200, 1500, 2001
    A, B = rand_case(M, N, K, 7400 + sum(offs))
    ref, _ = oracle.gemm_nt(A, B)
    assert g.plan(M, N, K, 256)[0] == 13
    say(f"[gpu] rung 13 offsets {offs}")
    dA, dB = _offset_view(A, offs[0]), _offset_view(B, offs[1])
    D = _offset_view(np.full((M, N), np.nan, np.float16), offs[2])
    g.gemm_f16_nt(dA, dB, D)
    torch.cuda.synchronize()
    assert_parity(host_bits(D), ref, K, f"rung 13 offsets {offs}")
    pa, pb, pd = 3 + offs[0], 5 + offs[1], 7 + offs[2]
    Af = torch.zeros((1, M, K + pa), dtype=torch.float16, device=DEV)
    Bf = torch.zeros((1, N, K + pb), dtype=torch.float16, device=DEV)
    Af[0, :, :K] = dev(A)
    Bf[0, :, :K] = dev(B)
    Df = torch.full((1, M, N + pd), float("nan"), dtype=torch.float16, device=DEV)
    g.gemm_f16_nt_strided_batched(Af[:, :, :K], Bf[:, :, :K], Df[:, :, :N])
    torch.cuda.synchronize()
    assert_parity(host_bits(Df[0, :, :N]), ref, K, f"rung 13 pitched {offs}")
    assert torch.isnan(Df[:, :, N:]).all().item()


def test_splitk_entry_takes_rung13_or_one_launch_where_modeled_faster():
    """The split-K entry with splits = 0 runs rung 13 unsplit where its model
    beats the slices' and the ring's (256 x 4096 x 4096): bitwise equal to
    rung 13, no workspace needed; and one launch where the ring is modeled
    faster (128 x 14336 x 4096): bitwise equal to the plain entry."""
    cus = _cus()
    for (M, N, K, other) in [(256, 4096, 4096, 13), (128, 14336, 4096, 0)]:
        assert g.splitk_plan(M, N, K, cus) == (0, 1) and g.splitk_workspace_bytes(M, N, K) == 0
        A, B = rand_case(M, N, K, 7600 + M)
        dA, dB = dev(A), dev(B)
        say(f"[gpu] split-K entry one launch {M}x{N}x{K} (against rung {other})")
        D = poisoned(M, N)
        g.gemm_f16_nt_splitk(dA, dB, D)
        torch.cuda.synchronize()
        got = host_bits(D)
        assert np.array_equal(got, host_bits(run(other, dA, dB, poisoned(M, N))))
        rows, cols = sample_positions(M, N, 600, M + N + K)
        want, _ = oracle.gemm_nt_sampled(A, B, rows, cols)
        assert_parity(got[rows, cols], want, K, f"split-K entry {M}x{N}x{K}")


@pytest.mark.parametrize("shape", [(130, 17000, 1001), (17000, 130, 1001), (130, 6000, 3000), (6000, 130, 3000)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ksplit_s_major_parity(shape):
    """Rung 13 in its S-major tile order (64-row L tiles, an L side over 32
    MiB, more than one round of workgroups): every output against the
    oracle into NaN-poisoned D, either operand as S, bitwise repeatable."""
    M, N, K = shape
    mt, nf, db, nw = g.ksplit_plan(13, M, N, K, _cus())
    s_rows, l_rows = min(M, N), max(M, N)
    wgs = -(-l_rows // (16 * nf)) * -(-s_rows // (16 * mt))
    assert nf == 4 and mt <= 3 and l_rows * K * 2 > 32 << 20 and wgs > _cus() and g.plan(M, N, K, _cus())[0] == 13
    A, B = rand_case(M, N, K, 7700 + M)
    ref, _ = oracle.gemm_nt(A, B)
    dA, dB = dev(A), dev(B)
    say(f"[gpu] rung 13 S-major {M}x{N}x{K} tile={(mt, nf, db, nw)} workgroups={wgs}")
    got = host_bits(run(13, dA, dB, poisoned(M, N)))
    assert_parity(got, ref, K, f"rung 13 S-major {shape}")
    assert np.array_equal(host_bits(run(0, dA, dB, poisoned(M, N))), got)


@pytest.mark.parametrize("shape", [(128, 4096, 14336), (4096, 128, 4096), (256, 1024, 8192), (96, 16384, 8192),
                                   (128, 8192, 8192)], ids=lambda s: "x".join(map(str, s)))
def test_ksplit_full_size_repeatable_and_split_k_entry(shape):
    """Full-size products the library runs on rung 13: sampled outputs
    against the oracle, no output left unwritten, bitwise repeats, and the
    split-K entry, where it runs them unsplit, equal to the plain one."""
    M, N, K = shape
    assert g.plan(M, N, K, _cus())[0] == 13
    A, B = rand_case(M, N, K, 7500 + M + N)
    dA, dB = dev(A), dev(B)
    say(f"[gpu] rung 13 full size {shape} tile={g.ksplit_plan(13, M, N, K, _cus())}")
    first = host_bits(run(0, dA, dB, poisoned(M, N)))
    assert not np.isnan(as_f64(first)).any(), "output elements left unwritten"
    for _ in range(2):
        assert np.array_equal(host_bits(run(0, dA, dB, poisoned(M, N))), first)
    if g.splitk_plan(M, N, K, _cus()) == (0, 1):
        D = poisoned(M, N)
        g.gemm_f16_nt_splitk(dA, dB, D)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(D), first)
    rows, cols = sample_positions(M, N, 800, M + K)
    want, _ = oracle.gemm_nt_sampled(A, B, rows, cols)
    assert_parity(first[rows, cols], want, K, f"rung 13 {shape}")