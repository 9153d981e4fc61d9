"""Pins for the CPU oracle, each against something other than the oracle:
numpy's float16 conversion (a library routine), exact rational arithmetic on
tiny shapes with a brute-force rounding, closed forms (identity, selection,
all-ones, small integers through exact integer matmul) and hand-built rows
whose exact sums land on ties, the overflow threshold and the subnormal grid.

The definition being pinned is D = round_fp16(A B^T) with B stored N x K
("GEMM I - the tiled baseline", problem statement; "TIRx GEMM detailed
technical notes", V3 and V8): fp16 operands, wide accumulation, one
rounding at writeback.
"""
import bisect
from fractions import Fraction

import numpy as np
import pytest

import oracle

ALL16 = np.arange(65536, dtype=np.uint16)


def f16(values):
    return np.asarray(values, dtype=np.float16)


# ---------------------------------------------------------------- codec (P1)

def test_decode_all_patterns_match_numpy():
    got = oracle.f16_to_f64(ALL16)
    ref = ALL16.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros and infinities decode with their sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0x0000])
    assert got[0x7C00] == np.inf and got[0xFC00] == -np.inf


def _finite_positive():
    v = ALL16[:0x7C00].view(np.float16).astype(np.float64)  # 0 .. 65504
    return v


def test_encode_midpoints_and_neighbours_match_numpy():
    v = _finite_positive()
    mid = (v[:-1] + v[1:]) / 2.0                     # exact in fp64
    probes = np.concatenate([
        v, mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf),
        [65504.0, 65519.99, 65520.0, np.nextafter(65520.0, 0.0), 65536.0, 1e6],
    ])
    probes = np.concatenate([probes, -probes])
    got = oracle.f64_to_f16(probes)
    with np.errstate(over="ignore"):
        ref = probes.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(probes[i], hex(got[i]), hex(ref[i])) for i in bad[:8]]


@pytest.mark.parametrize("x,bits", [
    (2049.0, 0x6800),             # tie between 2048 and 2050 -> even (2048)
    (2051.0, 0x6802),             # tie between 2050 and 2052 -> even (2052)
    (2049.0 + 2.0 ** -20, 0x6801),  # just above the tie: 2050 (a route through fp32 gives 2048)
    (65519.0, 0x7BFF),
    (65520.0, 0x7C00),            # the overflow threshold rounds to +inf
    (-65520.0, 0xFC00),
    (2.0 ** -25, 0x0000),         # half the smallest subnormal: tie to even (0)
    (0.75 * 2.0 ** -24, 0x0001),
    (1.5 * 2.0 ** -24, 0x0002),   # tie between 1 and 2 subnormal steps -> 2
    (2.0 ** -14 - 2.0 ** -26, 0x0400),  # rounds up into the first normal binade
    (0.0, 0x0000),
])
def test_encode_closed_forms(x, bits):
    assert int(oracle.f64_to_f16([x])[0]) == bits


def test_encode_nan_and_negative_zero():
    assert np.isnan(np.uint16(oracle.f64_to_f16([np.nan])[0]).view(np.float16))
    assert int(oracle.f64_to_f16([-0.0])[0]) == 0x8000


def test_oracle_rounds_once_not_through_fp32():
    # exact sum 2049 + 2^-20: a fp64 -> fp32 -> fp16 path lands on the tie
    # 2049 and then on 2048; the single rounding must give 2050.
    A = f16([[1.0, 1.0, 2.0 ** -10]])
    B = f16([[2048.0, 1.0, 2.0 ** -10]])    # 2048 + 1 + 2^-20
    D, _ = oracle.gemm_nt(A, B)
    assert int(D[0, 0]) == 0x6801


# ------------------------------------------- brute force on tiny shapes (P2)

_POS16 = [Fraction(float(x)) for x in ALL16[:0x7C00].view(np.float16)]


def _round_bruteforce(q: Fraction) -> int:
    """Nearest fp16 by search over the sorted list of all finite values;
    ties to the even bit pattern; |q| >= 65520 -> inf."""
    sign = 0x8000 if q < 0 else 0
    a = -q if q < 0 else q
    if a >= 65520:
        return sign | 0x7C00
    i = bisect.bisect_left(_POS16, a)
    if i < len(_POS16) and _POS16[i] == a:
        return sign | i
    lo, hi = i - 1, i                       # _POS16[lo] < a < _POS16[hi]
    dl, dh = a - _POS16[lo], _POS16[hi] - a
    if dl < dh:
        return sign | lo
    if dh < dl:
        return sign | hi
    return sign | (lo if lo % 2 == 0 else hi)


def _exact_nt(A, B):
    M, K = A.shape
    N = B.shape[0]
    Af = [[Fraction(float(x)) for x in row] for row in A]
    Bf = [[Fraction(float(x)) for x in row] for row in B]
    out = np.empty((M, N), dtype=np.uint16)
    for m in range(M):
        for n in range(N):
            out[m, n] = _round_bruteforce(sum((Af[m][k] * Bf[n][k] for k in range(K)), Fraction(0)))
    return out


@pytest.mark.parametrize("K", [1, 2, 3, 7, 8, 15, 16, 17, 63, 64, 65])
def test_bruteforce_tiny(K):
    rng = np.random.default_rng(1000 + K)
    for M, N in [(1, 1), (3, 5), (8, 2)]:
        # mixed magnitudes so outputs span subnormal .. large binades
        A = (rng.uniform(-1, 1, (M, K)) * 2.0 ** rng.integers(-12, 6, (M, K))).astype(np.float16)
        B = (rng.uniform(-1, 1, (N, K)) * 2.0 ** rng.integers(-12, 6, (N, K))).astype(np.float16)
        D, _ = oracle.gemm_nt(A, B)
        ref = _exact_nt(A, B)
        assert np.array_equal(D, ref), (M, N, K)


def test_bruteforce_catches_operand_roles():
    # B is N x K: D[m, n] pairs row m of A with row n of B.  A transposed
    # reading (B as K x N) would be a different matrix here.
    A = f16([[1, 2, 3], [4, 5, 6]])            # M=2, K=3
    B = f16([[1, 0, 0], [0, 1, 0], [0, 0, 1], [1, 1, 1]])  # N=4, K=3
    D, _ = oracle.gemm_nt(A, B)
    assert np.array_equal(D.view(np.float16).astype(np.float64),
                          np.array([[1, 2, 3, 6], [4, 5, 6, 15]], dtype=np.float64))


# ----------------------------------------------------- algebraic pins (P3-P8)

def _rand16(rng, shape, scale=1.0):
    return (rng.uniform(-scale, scale, shape)).astype(np.float16)


def test_transpose_identity_bitwise():
    rng = np.random.default_rng(7)
    A = _rand16(rng, (37, 96))
    B = _rand16(rng, (53, 96))
    D1, _ = oracle.gemm_nt(A, B)
    D2, _ = oracle.gemm_nt(B, A)
    assert np.array_equal(D1, D2.T)


def test_identity_operands():
    rng = np.random.default_rng(8)
    K = 64
    B = _rand16(rng, (40, K))
    I = np.eye(K, dtype=np.float16)
    D, _ = oracle.gemm_nt(I, B)                 # A = I  ->  D = B^T
    assert np.array_equal(D.view(np.float16), B.T)
    A = _rand16(rng, (24, K))
    D, _ = oracle.gemm_nt(A, I)                 # B = I  ->  D = A
    assert np.array_equal(D.view(np.float16), A)


def test_selection_matrix():
    rng = np.random.default_rng(9)
    M, N, K = 50, 33, 24
    perm = rng.integers(0, K, M)
    A = np.zeros((M, K), dtype=np.float16)
    A[np.arange(M), perm] = 1
    B = _rand16(rng, (N, K), 100.0)
    D, _ = oracle.gemm_nt(A, B)
    assert np.array_equal(D.view(np.float16), B[:, perm].T)


@pytest.mark.parametrize("K", [64, 512, 4096, 8192])
def test_all_ones_equals_k(K):
    A = np.ones((3, K), dtype=np.float16)
    B = np.ones((2, K), dtype=np.float16)
    D, _ = oracle.gemm_nt(A, B)
    assert np.all(D.view(np.float16).astype(np.float64) == K)


def test_small_integers_exact():
    rng = np.random.default_rng(10)
    M, N, K = 20, 30, 8192
    Ai = rng.integers(-4, 5, (M, K))
    Bi = rng.integers(-4, 5, (N, K))
    exact = Ai @ Bi.T                            # int64, exact
    ref = exact.astype(np.float64).astype(np.float16).view(np.uint16)
    D, _ = oracle.gemm_nt(Ai.astype(np.float16), Bi.astype(np.float16))
    assert np.array_equal(D, ref)


def test_small_integers_on_ties():
    # non-negative entries put the sums near 3072, where the fp16 step is 2:
    # every odd sum is an exact tie and must round to the even neighbour
    rng = np.random.default_rng(13)
    M, N, K = 24, 40, 768
    Ai = rng.integers(0, 5, (M, K))
    Bi = rng.integers(0, 5, (N, K))
    exact = Ai @ Bi.T
    ties = (exact >= 2048) & (exact < 4096) & (exact % 2 == 1)
    assert ties.sum() > 100
    ref = exact.astype(np.float64).astype(np.float16).view(np.uint16)
    D, _ = oracle.gemm_nt(Ai.astype(np.float16), Bi.astype(np.float16))
    assert np.array_equal(D, ref)
    # round-half-even, not half-up: every tie lands on a multiple of 4
    vals = D.view(np.float16).astype(np.int64)
    assert np.all(vals[ties] % 4 == 0)


def test_designed_rows_ties_overflow_subnormals():
    K = 8
    A = np.zeros((2, K), dtype=np.float16)
    A[0, :2] = [1, 1]
    A[1, 0] = 2.0 ** -12
    B = np.zeros((5, K), dtype=np.float16)
    B[0, :2] = [2048, 1]        # 2049 -> 2048
    B[1, :2] = [2048, 3]        # 2051 -> 2052
    B[2, :2] = [65504, 16]      # 65520 -> +inf
    B[3, 0] = 2.0 ** -12        # 2^-24: smallest subnormal
    B[4, 0] = 2.0 ** -13        # 2^-25: tie -> 0
    D, _ = oracle.gemm_nt(A, B)
    assert [int(x) for x in D[0, :3]] == [0x6800, 0x6802, 0x7C00]
    assert [int(x) for x in D[1, 3:]] == [0x0001, 0x0000]


def test_k_zero_and_empty():
    D, _ = oracle.gemm_nt(np.zeros((3, 0), np.float16), np.zeros((4, 0), np.float16))
    assert D.shape == (3, 4) and np.all(D == 0)
    D, _ = oracle.gemm_nt(np.zeros((0, 8), np.float16), np.zeros((4, 8), np.float16))
    assert D.shape == (0, 4)


def test_sampled_equals_full():
    rng = np.random.default_rng(11)
    A = _rand16(rng, (70, 136))
    B = _rand16(rng, (45, 136))
    D, _ = oracle.gemm_nt(A, B, nthreads=3)
    r = rng.integers(0, 70, 500)
    c = rng.integers(0, 45, 500)
    s, _ = oracle.gemm_nt_sampled(A, B, r, c, nthreads=2)
    assert np.array_equal(s, D[r, c])
    with pytest.raises(IndexError):
        oracle.gemm_nt_sampled(A, B, [70], [0])


def test_thread_count_does_not_change_result():
    rng = np.random.default_rng(12)
    A = _rand16(rng, (33, 200))
    B = _rand16(rng, (17, 200))
    D1, t1 = oracle.gemm_nt(A, B, nthreads=1)
    D8, t8 = oracle.gemm_nt(A, B, nthreads=8)
    assert t1 == 1 and t8 == 8
    assert np.array_equal(D1, D8)
