"""C-ABI library on the CPU: it loads, exports every declared symbol,
validates before any HIP call, and its host-side schedule / ring logic
matches the pages' printed tables and is a bijection over tiles."""
import ctypes
import os
import re

import numpy as np
import pytest

import dense_fp16_gemm_nt_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_f16_nt.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return np.array(rows, dtype=np.int64)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_f16_nt\w*)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "gemm_f16_nt" in names and len(names) >= 7
    L = ctypes.CDLL(g.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    assert g.status_string(0) == "ok"
    for s in (g.INVALID_ARG, g.UNSUPPORTED, g.LAUNCH, g.DEVICE, 12345):
        assert isinstance(g.status_string(s), str) and g.status_string(s)


A0, B0, D0 = 0x10000, 0x20000000, 0x40000000   # fake, 16-byte aligned, disjoint


@pytest.mark.parametrize("args,want", [
    ((0, 64, 64, 64, A0, B0, D0), g.OK),
    ((0, -1, 64, 64, A0, B0, D0), g.INVALID_ARG),
    ((0, 64, -1, 64, A0, B0, D0), g.INVALID_ARG),
    ((0, 64, 64, -8, A0, B0, D0), g.INVALID_ARG),
    ((0, 64, 64, 64, 0, B0, D0), g.INVALID_ARG),
    ((0, 64, 64, 64, A0, 0, D0), g.INVALID_ARG),
    ((0, 64, 64, 64, A0, B0, 0), g.INVALID_ARG),
    ((0, 64, 64, 12, A0, B0, D0), g.OK),                   # K % 8 != 0: register-staged loads
    ((0, 64, 64, 64, A0 + 2, B0, D0), g.OK),               # A rows not 16-byte aligned: the same
    ((0, 64, 64, 64, A0, B0 + 8, D0), g.OK),
    ((0, 64, 64, 64, A0, B0, D0 + 4), g.OK),
    ((3, 64, 64, 13, A0, B0, D0), g.OK),                   # R3 takes general operands too
    ((4, 64, 64, 12, A0, B0, D0), g.OK),                   # R4 and R9 stage general rows through registers
    ((9, 64, 64, 64, A0 + 2, B0, D0), g.OK),
    ((4, 64, 64, 4, A0, B0, D0), g.UNSUPPORTED),           # ... for K >= 8
    ((9, 64, 64, 6, A0, B0, D0), g.UNSUPPORTED),
    ((5, 64, 64, 12, A0, B0, D0), g.UNSUPPORTED),          # the other rungs need 16-byte rows
    ((5, 64, 64, 64, A0 + 2, B0, D0), g.UNSUPPORTED),
    ((8, 256, 256, 128, A0, B0, D0 + 8), g.UNSUPPORTED),
    ((1, 128, 128, 64, A0, B0 + 2, D0), g.UNSUPPORTED),
    ((0, 64, 64, 64, A0 + 1, B0, D0), g.UNSUPPORTED),      # odd address: not an fp16 array
    ((0, 64, 64, 64, A0, B0, D0 + 1), g.UNSUPPORTED),
    ((0, 64, 10_000_000, 4, A0, B0, D0), g.UNSUPPORTED),   # K < 8 runs on R3's grid: N/128 > 65535
    ((3, 64, 10_000_000, 12, A0, B0, D0), g.UNSUPPORTED),  # so does rung 3
    ((0, 64, 10_000_000, 12, A0, B0, D0), g.OK),           # the staged ring's grid is one-dimensional
    ((0, 64, 64, 64, A0, B0, A0 + 4096), g.INVALID_ARG),   # D overlaps A
    ((0, 64, 64, 64, A0, B0, B0), g.INVALID_ARG),          # D overlaps B
    ((14, 64, 64, 64, A0, B0, D0), g.INVALID_ARG),         # unknown rung
    ((13, 64, 64, 64, A0, B0, D0), g.OK),                   # rung 13: any M, N >= 1 ...
    ((13, 5000, 3000, 4096, A0, B0, D0), g.OK),
    ((13, 1, 1, 8, A0, B0, D0), g.OK),
    ((13, 16, 4096, 7, A0, B0, D0), g.UNSUPPORTED),         # ... and K >= 8
    ((13, 300, 4096, 4095, A0 + 2, B0 + 6, D0 + 2), g.OK),  # ... rows on any 2-byte boundary
    ((13, 1 << 31, 1 << 31, 64, A0, 1 << 40, 1 << 44), g.UNSUPPORTED),  # 2^46 tiles of 16 x 16
    ((12, 64, 4096, 4096, A0, B0, D0), g.OK),               # rung 12: one side of at most 64 rows
    ((12, 4096, 64, 4096, A0, B0, D0), g.OK),
    ((12, 96, 4096, 4096, A0, B0, D0), g.OK),               # ... up to 96 rows
    ((12, 97, 97, 4096, A0, B0, D0), g.UNSUPPORTED),        # ... neither side small
    ((12, 16, 4096, 7, A0, B0, D0), g.UNSUPPORTED),         # ... K >= 8
    ((12, 16, 4096, 4095, A0 + 2, B0 + 6, D0 + 2), g.OK),   # ... rows on any 2-byte boundary
    ((11, 384, 256, 128, A0, B0, D0), g.OK),                # rung 11: 384 x 256 tiles
    ((11, 383, 256, 128, A0, B0, D0), g.UNSUPPORTED),       # ... at least one tile row
    ((11, 384, 255, 128, A0, B0, D0), g.UNSUPPORTED),       # ... and column
    ((11, 384, 256, 136, A0, B0, D0), g.UNSUPPORTED),       # ... whole 64-wide k steps
    ((11, 384, 256, 64, A0, B0, D0), g.UNSUPPORTED),        # ... at least two
    ((11, 400, 300, 192, A0, B0, D0), g.OK),                # ragged M, N
    ((11, 384, 1 << 23, 128, A0, 1 << 34, 1 << 36), g.UNSUPPORTED),   # output blocks span 384 * N bytes
    ((11, 384, (1 << 23) - 8, 128, A0, 1 << 34, 1 << 36), g.OK),
    ((10, 64, 64, 64, A0, B0, D0), g.UNSUPPORTED),         # rung 10: M, N >= 256
    ((10, 512, 256, 192, A0, B0, D0), g.OK),
    ((10, 256, 260, 128, A0, B0, D0), g.OK),              # rung 10 takes any N >= 256
    ((8, 256, 260, 128, A0, B0, D0), g.UNSUPPORTED),      # rung 8 keeps N % 8 == 0
    ((10, 256, 256, 136, A0, B0, D0), g.OK),               # rung 10: K % 64 != 0, partial first step
    ((10, 256, 264, 72, A0, B0, D0), g.OK),
    ((10, 256, 256, 64, A0, B0, D0), g.UNSUPPORTED),       # ... but at least two k steps
    ((10, 256, 256, 40, A0, B0, D0), g.UNSUPPORTED),
    ((10, 256, 256, (1 << 21) + 8, A0, B0, D0), g.UNSUPPORTED),  # ... and rows under 2^21 elements
    ((10, 256, 256, 1 << 21, A0, 1 << 32, 1 << 33), g.OK),  # whole steps: any row length
    ((8, 256, 256, 136, A0, B0, D0), g.UNSUPPORTED),       # rungs 6-8: whole 64-wide steps only
    ((9, 64, 64, 64, A0, B0, D0), g.OK),                   # rung 9: any shape
    ((8, 64, 64, 64, A0, B0, D0), g.UNSUPPORTED),          # rung 8: M, N >= 256
    ((-1, 64, 64, 64, A0, B0, D0), g.INVALID_ARG),
    ((1, 128, 128, 64, A0, B0, D0), g.OK),
    ((1, 128, 128, 128, A0, B0, D0), g.UNSUPPORTED),       # R1 is one 128x128x64 tile
    ((2, 128, 128, 4096, A0, B0, D0), g.OK),
    ((2, 256, 128, 64, A0, B0, D0), g.UNSUPPORTED),        # R2 is one tile
    ((3, 1000, 333, 72, A0, B0, D0), g.OK),
    ((4, 1, 1, 8, A0, B0, D0), g.OK),
    ((5, 5000, 7, 8, A0, B0, D0), g.OK),
    ((8, 256, 512, 128, A0, B0, D0), g.OK),
    ((8, 64, 64, 64, A0, B0, D0), g.UNSUPPORTED),          # R8 needs M, N >= 256
    ((8, 256, 256, 64, A0, B0, D0), g.UNSUPPORTED),        # ... and at least two k steps
    ((8, 256, 256, 200, A0, B0, D0), g.UNSUPPORTED),       # ... of 64
    ((8, 256, 300, 128, A0, B0, D0), g.UNSUPPORTED),       # ... N a multiple of 8
    ((8, 300, 264, 128, A0, B0, D0), g.OK),                # ragged M, N: the last tiles move back
    ((8, 255, 264, 128, A0, B0, D0), g.UNSUPPORTED),       # ... but not below one tile
    ((6, 512, 256, 192, A0, B0, D0), g.INVALID_ARG),       # rungs 6 and 7 were removed
    ((7, 512, 256, 192, A0, B0, D0), g.INVALID_ARG),
    ((0, 0, 64, 64, 0, 0, 0), g.OK),                       # empty output: nothing needed
    ((0, 64, 64, 0, 0, 0, D0), g.OK),                      # K = 0: D only
    ((0, 64, 64, 1 << 23, A0, B0, D0), g.UNSUPPORTED),     # beyond the kernels' index range
    # the four-wave ring's output blocks span 256 * N bytes in a 32-bit size: N < 2^24
    ((8, 256, 1 << 24, 128, A0, 1 << 34, 1 << 36), g.UNSUPPORTED),
    ((10, 256, 1 << 24, 128, A0, 1 << 34, 1 << 36), g.UNSUPPORTED),
    ((8, 256, (1 << 24) + 8, 128, A0, 1 << 34, 1 << 36), g.UNSUPPORTED),
    ((10, 256, (1 << 24) - 8, 128, A0, 1 << 34, 1 << 36), g.OK),
    ((8, 256, (1 << 24) - 8, 128, A0, 1 << 34, 1 << 36), g.OK),
    ((0, 256, 1 << 24, 128, A0, 1 << 34, 1 << 36), g.OK),   # the library's choice takes another kernel
])
def test_validation(args, want):
    assert g.check(*args) == want


def test_invalid_call_returns_before_any_device_work():
    L = g.lib()
    assert L.gemm_f16_nt(-1, 4, 8, A0, B0, D0, None) == g.INVALID_ARG
    assert L.gemm_f16_nt_rung(0, 4, 4, 8, A0, B0, D0, None) == g.INVALID_ARG
    assert L.gemm_f16_nt_persistent(4, 4, 8, A0, B0, D0, 0, None) == g.INVALID_ARG
    assert L.gemm_f16_nt(0, 4, 8, 0, 0, 0, None) == g.OK     # empty: no-op


@pytest.mark.skipif(os.environ.get("HIP_VISIBLE_DEVICES") is None and os.path.exists("/dev/kfd"),
                    reason="a GPU may be present")
def test_valid_call_without_gpu_fails_loudly():
    # no device here: a well-formed call must report DEVICE, not pretend
    assert g.lib().gemm_f16_nt(64, 64, 64, A0, B0, D0, None) == g.DEVICE


def test_ring_plan_matches_printed_phase_table():
    gold = _golden("ring_schedule_depth2.txt")
    stage, lap, _ = g.ring_plan(2, len(gold))
    assert np.array_equal(stage, gold[:, 1])
    assert np.array_equal(lap & 1, gold[:, 2])


def test_ring_plan_refill_schedule_ktiles5():
    gold = _golden("ring_refill_ktiles5.txt")
    stage, _, refill = g.ring_plan(2, 5)
    assert np.array_equal(stage, gold[:, 1])
    assert np.array_equal(refill, gold[:, 2])


@pytest.mark.parametrize("depth,steps", [(1, 7), (2, 64), (3, 10), (4, 129)])
def test_ring_plan_invariants(depth, steps):
    stage, lap, refill = g.ring_plan(depth, steps)
    for k in range(steps):
        assert stage[k] == k % depth and lap[k] == k // depth
        if refill[k] >= 0:
            # a refill reuses the stage just consumed, one lap later
            assert stage[refill[k]] == stage[k] and lap[refill[k]] == lap[k] + 1
    # every step except the prologue's is loaded by exactly one refill
    loaded = sorted(int(r) for r in refill if r >= 0)
    assert loaded == list(range(min(depth, steps), steps))


@pytest.mark.parametrize("M,N,grid", [
    (4096, 4096, 256), (8192, 8192, 256), (32768, 1024, 256), (256, 256, 256),
    (4096, 4096, 1), (4096, 4096, 7), (4096, 4096, 512), (1000, 3000, 37), (1, 1, 3),
    (8192, 8192, 148),
])
def test_schedule_is_a_bijection(M, N, grid):
    wg, tm, tn = g.schedule(M, N, grid)
    T_m, T_n = -(-M // 256), -(-N // 256)
    assert len(wg) == T_m * T_n
    assert np.all((tm >= 0) & (tm < T_m) & (tn >= 0) & (tn < T_n))
    ids = tm * T_n + tn
    assert len(np.unique(ids)) == T_m * T_n
    counts = np.bincount(wg)
    assert counts.max() - counts.min() <= 1          # balanced to one tile


def test_schedule_matches_printed_persistent_arithmetic():
    M, N, tile, tiles, grid, mean_x10 = _golden("persistent_grid_4096.txt")[0]
    # same tile count with the library's 256 x 256 tiles at twice the size
    scale = 256 // tile
    wg, _, _ = g.schedule(M * scale, N * scale, grid)
    assert len(wg) == tiles
    counts = np.bincount(wg, minlength=grid)
    assert round(10 * counts.mean()) == mean_x10
    assert set(counts.tolist()) == {tiles // grid, tiles // grid + 1}


def test_schedule_xcd_locality():
    # one tile per workgroup at 4096^2: the 32 workgroups of one XCD
    # (w mod 8 equal) own a compact block of tiles (8 tile rows x 4 columns)
    wg, tm, tn = g.schedule(4096, 4096, 256)
    for x in range(8):
        sel = (wg % 8) == x
        assert sel.sum() == 32
        assert len(np.unique(tm[sel])) == 8 and len(np.unique(tn[sel])) == 4


@pytest.mark.parametrize("rung,M,N,cus", [
    (10, 4096, 4096, 256), (10, 8192, 8192, 256), (10, 32768, 1024, 256), (10, 4000, 4000, 256),
    (10, 300, 264, 256), (10, 256, 256, 256), (10, 6144, 6144, 256), (10, 1000, 3000, 37), (8, 4608, 4608, 304),
    (5, 4096, 4096, 256), (5, 1000, 3000, 37), (4, 4096, 4096, 256), (4, 1000, 3000, 256), (9, 4096, 4096, 256),
    (9, 200, 32768, 256), (11, 6144, 4096, 256), (11, 8192, 8192, 256), (11, 400, 300, 256), (11, 4000, 1000, 37),
])
def test_tile_walk_covers_every_output_once(rung, M, N, cus):
    """Every rung's tile walk covers every output element: exactly once
    where the tiles divide M and N; the four-wave ring's moved-back last
    row and column of tiles overlap only their neighbours, and every other
    rung masks its edge tiles (its origins are whole multiples of the tile).
    Every workgroup of a persistent walk gets its share to within one tile."""
    wg, r0, c0 = g.tile_walk(rung, M, N, cus)
    tile = 128 if rung == 9 else 256
    tile_m = 384 if rung == 11 else tile
    tm, tn = -(-M // tile_m), -(-N // tile)
    assert len(wg) == tm * tn
    cover = np.zeros((M, N), np.int16)
    for r, c in zip(r0.tolist(), c0.tolist()):
        cover[r: r + tile_m, c: c + tile] += 1
    assert cover.min() >= 1
    if rung in (8, 10, 11):
        assert np.all((r0 >= 0) & (r0 + tile_m <= M) & (c0 >= 0) & (c0 + tile <= N))   # whole tiles, in range
        # outputs computed twice: exactly the band where the moved-back last
        # tile row (column) overlaps its neighbour
        band_r = np.zeros(M, bool)
        band_c = np.zeros(N, bool)
        if M % tile_m:
            band_r[M - tile_m: (M // tile_m) * tile_m] = True
        if N % tile:
            band_c[N - tile: (N // tile) * tile] = True
        twice = band_r[:, None] | band_c[None, :]
        assert np.array_equal(cover > 1, twice)
        assert cover.max() <= 4
    else:
        assert np.all(r0 % tile_m == 0) and np.all(c0 % tile == 0)
        assert cover.max() == 1
    counts = np.bincount(wg)
    assert counts.max() - counts.min() <= 1


@pytest.mark.parametrize("M,N,rounds", [(4096, 4096, 1), (8192, 8192, 4), (32768, 1024, 2)])
def test_tile_walk_four_wave_xcd_blocks(M, N, rounds):
    """The library's kernel at the three large workloads: in every round of
    tiles, the 32 workgroups of one XCD (w mod 8 equal) work on one block of
    4 tile rows x 8 tile columns (24 MiB of operand bands at 4096^3, the
    least for 32 tiles), so the bands they share stay in that XCD's L2
    ("TIRx GEMM detailed technical notes", V6 "Better L2 Locality")."""
    wg, r0, c0 = g.tile_walk(10, M, N, 256)
    visit = np.zeros_like(wg)
    for w in range(256):
        sel = np.nonzero(wg == w)[0]
        visit[sel] = np.arange(len(sel))
    assert visit.max() + 1 == rounds
    for i in range(rounds):
        for x in range(8):
            sel = (wg % 8 == x) & (visit == i)
            assert sel.sum() == 32
            rows, cols = np.unique(r0[sel]), np.unique(c0[sel])
            assert (len(rows), len(cols)) == ((4, 8) if N >= 2048 else (8, 4))
            assert rows.max() - rows.min() == 256 * (len(rows) - 1)
            assert cols.max() - cols.min() == 256 * (len(cols) - 1)


def test_tile_walk_argument_errors():
    L = g.lib()
    assert L.gemm_f16_nt_tile_walk(3, 256, 256, 256, None, None, None, 0) == g.INVALID_ARG   # no tile walk
    assert L.gemm_f16_nt_tile_walk(10, 200, 4096, 256, None, None, None, 0) == g.UNSUPPORTED
    assert L.gemm_f16_nt_tile_walk(10, 256, 256, 0, None, None, None, 0) == g.INVALID_ARG
    assert L.gemm_f16_nt_tile_walk(10, 256, 256, 256, None, None, None, 1) == g.INVALID_ARG
    assert L.gemm_f16_nt_tile_walk(10, 0, 256, 256, None, None, None, 0) == 0


@pytest.mark.parametrize("args,want", [
    # M, N, K, A, lda, sa, B, ldb, sb, D, ldd, sd, batch
    ((64, 64, 64, A0, 64, 4096, B0, 64, 4096, D0, 64, 4096, 3), g.OK),
    ((64, 64, 64, A0, 72, 0, B0, 64, 0, D0, 64, 4096, 3), g.OK),           # broadcast A and B
    ((64, 64, 64, A0, 56, 0, B0, 64, 0, D0, 64, 4096, 1), g.INVALID_ARG),  # lda < K
    ((64, 64, 64, A0, 64, 0, B0, 64, 0, D0, 60, 4096, 1), g.INVALID_ARG),  # ldd < N
    ((64, 64, 64, A0, 68, 0, B0, 64, 0, D0, 64, 4096, 1), g.OK),           # lda % 8 != 0: register-staged loads
    ((64, 64, 64, A0, 64, 4, B0, 64, 0, D0, 64, 4096, 2), g.OK),           # stride_a % 8 != 0: the same
    ((64, 64, 13, A0, 13, 832, B0, 13, 0, D0, 64, 4096, 2), g.OK),         # K % 8 != 0
    ((64, 64, 64, A0 + 1, 64, 0, B0, 64, 0, D0, 64, 4096, 1), g.UNSUPPORTED),  # odd address
    ((64, 64, 4, A0, 68, 0, B0, 64, 0, D0, 64, 4096, 70000), g.UNSUPPORTED),   # K < 8 on R3's grid: batch > 65535
    ((64, 64, 64, A0, 68, 0, B0, 64, 0, D0, 64, 4096, 70000), g.OK),           # the staged ring takes it
    ((64, 64, 64, A0, 64, 0, B0, 64, 0, D0, 66, 8192, 2), g.OK),           # odd row pitch of D
    ((64, 64, 64, A0, 64, 0, B0, 64, 0, D0, 64, 4097, 2), g.OK),           # odd batch stride of D
    ((64, 64, 64, A0, 64, 0, B0, 64, 0, D0, 64, 4000, 2), g.INVALID_ARG),  # outputs overlap
    ((64, 64, 64, A0, 64, 0, B0, 64, 0, D0, 64, 0, 2), g.INVALID_ARG),     # all batches on one D
    ((64, 64, 64, A0, 64, 0, B0, 64, 0, D0, 64, 4096, 0), g.OK),           # empty batch
    ((64, 64, 64, A0, 64, 0, B0, 64, 0, D0, 64, 4096, -1), g.INVALID_ARG),
    ((64, 64, 64, A0, 64, 0, B0, 64, 0, A0 + 64, 64, 4096, 1), g.INVALID_ARG),  # D overlaps A
])
def test_strided_validation(args, want):
    assert g.check_strided(*args) == want


def test_splitk_workspace_sizes():
    L = g.lib()
    # K = 512 is 8 steps of 64; 4 slices of 2 steps; fp32 partials
    assert L.gemm_f16_nt_splitk_workspace(256, 256, 512, 4) == 4 * 256 * 256 * 4
    # 3 requested slices of 8 steps -> 3 steps each -> slices of 192, 192, 128
    assert L.gemm_f16_nt_splitk_workspace(256, 256, 512, 3) == 3 * 256 * 256 * 4
    # more slices than steps: one step per slice
    assert L.gemm_f16_nt_splitk_workspace(100, 60, 136, 16) == 3 * 100 * 60 * 4
    # K % 8 != 0 runs unsplit (register-staged loads)
    assert L.gemm_f16_nt_splitk_workspace(100, 60, 130, 16) == 0
    assert L.gemm_f16_nt_splitk_workspace(256, 256, 512, 1) == 0
    assert L.gemm_f16_nt_splitk_workspace(256, 256, 0, 4) == 0
    assert L.gemm_f16_nt_splitk_workspace(256, 256, 512, 65) == g.INVALID_ARG
    assert L.gemm_f16_nt_splitk_workspace(-1, 256, 512, 2) == g.INVALID_ARG


@pytest.mark.parametrize("shape,want", [
    ((6144, 6144, 6144), (10, 5376, 9)),      # 2.25 rounds: 21 tile rows on R10, 768 rows on 128x128 tiles
    ((6144, 6144, 1024), (10, 5376, 9)),
    ((6144, 6144, 512), (10, 6144, 0)),       # short K: one launch
    ((4352, 4352, 4096), (10, 3840, 9)),
    ((7168, 7168, 4096), (10, 6912, 9)),
    ((5120, 5120, 4096), (10, 5120, 0)),      # more than a third of a round left
    ((4096, 4096, 4096), (10, 4096, 0)),      # whole rounds
    ((8192, 8192, 8192), (11, 6144, 10)),     # 2 rounds of 384-row tiles on the top rows + 1 of 256-row ones, against 4
    ((32768, 1024, 8192), (10, 32768, 0)),
    ((256, 256, 512), (13, 256, 0)),          # tile-starved: K split among the waves of 16 x 16 tiles
    ((2560, 2560, 4096), (9, 2560, 0)),
    ((4000, 4000, 4000), (10, 4000, 0)),
    ((200, 4096, 1024), (13, 200, 0)),        # 64 tiles of 128^2 in their bounds-checked form: rung 13
    ((4096, 4092, 1024), (10, 4096, 0)),      # N % 8 != 0: the fourth form stores unaligned rows
    ((4096, 4096, 64), (4, 4096, 0)),         # one k step: not the four-wave ring
    ((128, 32768, 4096), (9, 128, 0)),        # M = 128: half of every 256-row tile would be padding
    ((200, 32768, 4096), (9, 200, 0)),        # M = 200: 128 tiles of 256^2 fill half the device
    ((384, 65536, 64), (4, 384, 0)),          # 512 tiles of 256^2 against 1536 of 128^2
    ((128, 32768, 4095), (9, 128, 0)),        # ... also for register-staged rows
    ((100, 100, 5), (3, 100, 0)),             # K < 8 off 16-byte rows: R3's general form
    ((100, 100, 100), (13, 100, 0)),          # K % 8 != 0 with one tile: rung 13 takes any 2-byte rows
    ((3000, 1000, 999), (9, 3000, 0)),        # K % 8 != 0: R9's register-staged form
    ((4096, 4096, 4095), (4, 4096, 0)),       # ... R4's when 256 x 256 tiles fill the device
    ((6144, 4096, 4096), (11, 6144, 0)),      # one round of 384 x 256 tiles against 1.5 of 256 x 256
    ((12288, 4096, 4096), (11, 12288, 0)),    # both fill whole rounds: the wider tile's fewer bytes per FLOP
    ((12288, 2048, 2048), (11, 12288, 0)),
    ((16384, 4096, 1088), (11, 12288, 10)),   # the top rows that fill whole rounds of 384-row tiles
    ((12288, 12288, 4096), (11, 12288, 0)),
    ((8192, 4096, 4096), (10, 8192, 0)),      # 2 rounds of 256-row tiles: no split beats it
    ((6144, 4096, 4000), (10, 6144, 0)),      # K not whole 64-wide steps: the four-wave ring
    ((6144, 4096, 1024), (10, 6144, 0)),      # short K: the four-wave ring carries its ring across tiles
    ((16, 4096, 14336), (12, 16, 0)),         # one small side: rung 12 splits K inside each workgroup
    ((4096, 16, 14336), (12, 4096, 0)),       # ... either side
    ((64, 8192, 8192), (12, 64, 0)),
    ((32, 28672, 8192), (12, 32, 0)),         # at most 32 rows: any large side
    ((64, 28672, 8192), (9, 64, 0)),          # 64 rows and a large side over 16384: 128 x 128 tiles
    ((80, 8192, 8192), (12, 80, 0)),          # up to 96 rows with a large side up to 12288
    ((96, 16384, 8192), (13, 96, 0)),         # ... beyond it, rung 13's 48 x 64 tiles in S-major order
    ((97, 4096, 4096), (13, 97, 0)),          # neither side small: 32 x 64 tiles, K split among waves
    ((128, 1024, 8192), (13, 128, 0)),        # 8 tiles of 128^2 for 128 steps: rung 13
    ((4096, 128, 4096), (13, 4096, 0)),       # ... either side
    ((300, 2000, 3000), (13, 300, 0)),
    ((128, 8192, 8192), (13, 128, 0)),        # rung 13's model at most 0.87 of the ring's
    ((256, 4096, 14336), (13, 256, 0)),
    ((1024, 1024, 8192), (13, 1024, 0)),
    ((1024, 1024, 2048), (13, 1024, 0)),      # 4-wave 64 x 64 tiles (14.2 us against 15.9 on 128 x 128 tiles)
    ((640, 4096, 4096), (9, 640, 0)),         # above 0.87: the ring
    ((384, 4096, 1024), (9, 384, 0)),
    ((384, 4096, 4096), (9, 384, 0)),         # rung 13 would take 3 rounds of workgroups
    ((64, 28672, 8192), (9, 64, 0)),          # ... and a large side re-read from HBM per round
    ((256, 2048, 65536), (13, 256, 0)),       # one round: the tile rows share the large side's blocks
    ((16, 4096, 4095), (12, 16, 0)),          # any K >= 8 ...
    ((16, 4096, 7), (3, 16, 0)),              # ... below that, R3's general form
])
def test_library_plan(shape, want):
    assert g.plan(*shape, 256) == want


@pytest.mark.parametrize("M,N,K", [(8192, 8192, 8192), (16384, 4096, 1088), (20480, 4096, 4096), (16384, 16384, 4096),
                                   (10240, 8192, 4096), (12288, 4096, 4096), (6144, 4096, 4096)])
@pytest.mark.parametrize("cus", [80, 256, 304])
def test_wide_top_rows_plan_invariants(M, N, K, cus):
    """When rung 11 takes only the top rows, they are whole 384-row tile
    rows and the rest is at least one 256-row tile row on rung 10; the plan
    never costs more rounds of tiles than rung 10 alone (a 384-row tile
    counted as 1.5/1.025 of a 256-row one, a second launch as 0.02 of a
    round)."""
    rung_top, m_top, rung_rest = g.plan(M, N, K, cus)
    tn = (N + 255) // 256

    def rounds(rows, tile):
        return -(-(-(-rows // tile) * tn) // cus)

    base = rounds(M, 256)
    if rung_top != 11:
        return
    if m_top == M:
        assert rung_rest == 0 and rounds(M, 384) * 1.5 / 1.025 < base
    else:
        assert rung_rest == 10 and m_top % 384 == 0 and M - m_top >= 256
        assert rounds(m_top, 384) * 1.5 / 1.025 + rounds(M - m_top, 256) + 0.02 < base


@pytest.mark.parametrize("shape,cus,want", [
    ((6144, 6144, 6144), 256, (5376, 3)),     # 2.25 rounds: 21 tile rows whole, 768 rows split 3 ways
    ((6280, 5888, 4096), 256, (5632, 3)),     # ragged M
    ((4352, 4352, 4096), 256, (0, 1)),        # the unsplit call's 128x128 tiles fit in one round: no split
    ((4096, 4096, 4096), 256, (0, 1)),        # whole rounds: no split
    ((8192, 8192, 8192), 256, (0, 1)),
    ((6144, 6144, 2048), 256, (0, 1)),        # short K: the split costs more than the last round
    ((256, 256, 65536), 256, (0, 64)),        # tile-starved: every row splits
    ((256, 1024, 8192), 256, (0, 1)),         # rung 13's model beats 32 slices: unsplit, rung 13
    ((128, 1024, 8192), 256, (0, 1)),
    ((256, 2048, 65536), 256, (0, 32)),       # at most 4 tiles and a long K: slices of 4 steps
    ((256, 256, 65536), 256, (0, 64)),        # ... where rung 13's per-workgroup K costs more
    ((256, 4096, 4096), 256, (0, 1)),         # rung 13 modeled faster than 8 slices (the plain entry keeps R9)
    ((128, 14336, 4096), 256, (0, 1)),        # R9's 112 tiles unsplit modeled faster than 4 slices
    ((128, 8192, 8192), 256, (0, 1)),         # rung 13's 4-wave 64 x 64 tiles modeled faster than 8 slices
    ((64, 1024, 8192), 256, (0, 1)),          # one small side: rung 12, unsplit
    ((16, 4096, 14336), 256, (0, 1)),
    ((1024, 1024, 8192), 256, (0, 16)),       # 16 tiles: slices of at least 8 steps
    ((256, 256, 512), 256, (0, 1)),           # 8 steps on one tile: unsplit
])
def test_splitk_plan(shape, cus, want):
    assert g.splitk_plan(*shape, cus) == want


@pytest.mark.parametrize("rung,shape,cus,want", [
    (12, (16, 4096, 14336), 256, (1, 1, 2, 8)),      # 16 rows of S: one L block, two groups in flight
    (12, (16, 14336, 8192), 256, (1, 1, 2, 8)),      # ... also with 32-row L tiles on every CU, below K = 12288
    (12, (16, 8192, 28672), 256, (1, 2, 1, 8)),      # 32 L rows for every compute unit and a long K
    (12, (4096, 32, 4096), 256, (2, 1, 1, 8)),
    (12, (32, 14336, 14336), 256, (2, 2, 1, 8)),
    (12, (64, 8192, 8192), 256, (4, 2, 1, 8)),       # from 48 rows of S, 32 L rows whenever every CU gets them
    (12, (64, 4096, 4096), 256, (4, 1, 1, 8)),       # ... here they would not
    (12, (96, 16384, 8192), 80, (6, 2, 1, 8)),
    (13, (256, 1024, 8192), 256, (2, 2, 1, 8)),      # 512 workgroups of 32 x 32: 2 rounds of 4 blocks
    (13, (128, 1024, 8192), 256, (1, 2, 2, 8)),      # 256 of 16 x 32: one round of 3 blocks
    (13, (128, 4096, 4096), 256, (2, 4, 1, 8)),      # 256 of 32 x 64
    (13, (300, 2000, 3000), 256, (3, 4, 1, 8)),      # 224 of 48 x 64
    (13, (100, 100, 1001), 256, (1, 1, 2, 8)),
    (13, (4096, 128, 4096), 256, (2, 4, 1, 8)),      # S is the side with fewer rows, here B
    (13, (256, 4096, 4096), 256, (4, 4, 1, 4)),      # 256 of 64 x 64 on 4 waves: 8 blocks at ~65 GB/s
    (13, (128, 8192, 28672), 256, (4, 4, 1, 4)),
    (13, (130, 6000, 1001), 256, (2, 4, 1, 4)),      # 1,125 of 32 x 64: 4 waves pay with several rounds
    (13, (6000, 130, 3000), 256, (2, 4, 1, 4)),
    (13, (128, 4096, 4096), 64, (4, 4, 1, 4)),       # fewer compute units: larger tiles (4 waves)
])
def test_ksplit_plan(rung, shape, cus, want):
    """The workgroup tile of rungs 12 and 13, as the host evaluates it."""
    assert g.ksplit_plan(rung, *shape, cus) == want


def test_ksplit_plan_model_choice():
    """Rung 13's tile is the one with the smallest model, the first of the
    list on ties: rounds of workgroups times the bytes each streams ((mt +
    nf) 16-row blocks of K), over the tile's rate, plus 3 us; the 4-wave
    32 x 64 tile only with more workgroups than compute units."""
    tiles = [((1, 1, 2, 8), 75e3, False), ((1, 2, 2, 8), 75e3, False), ((2, 2, 1, 8), 75e3, False),
             ((2, 4, 1, 8), 75e3, False), ((3, 4, 1, 8), 75e3, False), ((2, 4, 1, 4), 90e3, True),
             ((4, 4, 1, 4), 65e3, False)]
    for (M, N, K) in [(256, 1024, 8192), (97, 4096, 4096), (1000, 1000, 1001), (300, 2000, 3000), (700, 130, 1001),
                      (5000, 5000, 64), (129, 129, 129), (256, 4096, 4096), (1024, 1024, 8192), (130, 6000, 1001),
                      (512, 4096, 14336), (128, 8192, 8192)]:
        for cus in (64, 256, 304):
            s, l = min(M, N), max(M, N)
            best, bt = None, None
            for t, rate, multi in tiles:
                wgs = -(-l // (16 * t[1])) * -(-s // (16 * t[0]))
                if multi and wgs <= cus:
                    continue
                v = float(-(-wgs // cus)) * float(t[0] + t[1]) * 32.0 * float(K) / rate + 3.0
                if bt is None or v < bt:
                    best, bt = t, v
            assert g.ksplit_plan(13, M, N, K, cus) == best, (M, N, K, cus)


def test_ksplit_plan_errors():
    L = g.lib()
    x = ctypes.c_int()
    p = ctypes.byref(x)
    assert L.gemm_f16_nt_ksplit_plan(11, 64, 64, 64, 256, p, p, p, p) == g.INVALID_ARG
    assert L.gemm_f16_nt_ksplit_plan(13, 0, 64, 64, 256, p, p, p, p) == g.INVALID_ARG
    assert L.gemm_f16_nt_ksplit_plan(13, 64, 64, 64, 0, p, p, p, p) == g.INVALID_ARG
    assert L.gemm_f16_nt_ksplit_plan(13, 64, 64, 64, 256, None, p, p, p) == g.INVALID_ARG
    assert L.gemm_f16_nt_ksplit_plan(13, 64, 64, 64, 256, p, p, p, None) == g.INVALID_ARG
    assert L.gemm_f16_nt_ksplit_plan(12, 97, 97, 4096, 256, p, p, p, p) == g.UNSUPPORTED
    assert L.gemm_f16_nt_ksplit_plan(13, 64, 64, 7, 256, p, p, p, p) == g.UNSUPPORTED


@pytest.mark.parametrize("M,N,K", [(6144, 6144, 6144), (4352, 4352, 4096), (4500, 4352, 4096), (7168, 7168, 4096),
                                   (10000, 3000, 8192), (3000, 10000, 1024)])
@pytest.mark.parametrize("cus", [80, 256, 304])
def test_splitk_plan_invariants(M, N, K, cus):
    """Unsplit rows are whole 256-row tile rows that fit in whole rounds of
    the compute units; the split rows take at least two slices."""
    m_top, splits = g.splitk_plan(M, N, K, cus)
    tn = (N + 255) // 256
    tiles = (M + 255) // 256 * tn
    assert m_top % 256 == 0 and 0 <= m_top < M
    if m_top:
        assert m_top // 256 * tn <= tiles // cus * cus and splits >= 2
        assert tiles % cus != 0


def test_splitk_noalloc_rejects_beyond_its_scratch():
    """With an explicit slice count the no-allocation entry point sizes its
    partial sums before any HIP call: beyond the 64 MiB scratch array it
    returns GEMM_F16_NT_SCRATCH and launches nothing."""
    L = g.lib()
    A, B, D = 0x10000, 0x20000000, 0x40000000
    # 64 slices of 1024 x 1024 fp32 partial sums: 256 MiB
    assert L.gemm_f16_nt_splitk_noalloc(1024, 1024, 65536, A, B, D, 64, None) == g.SCRATCH
    assert L.gemm_f16_nt_splitk_workspace(1024, 1024, 65536, 64) == 256 << 20
    # 17 slices of 1024 x 1024 (68 MiB): over; 16 slices (64 MiB): fits, so
    # the call goes on to the device query, which fails here without a GPU
    assert L.gemm_f16_nt_splitk_noalloc(1024, 1024, 65536, A, B, D, 17, None) == g.SCRATCH
    assert L.gemm_f16_nt_splitk_noalloc(1024, 1024, 65536, A, B, D, 16, None) == g.DEVICE
    assert L.gemm_f16_nt_splitk_noalloc(1024, 1024, 65536, A, B, D, 65, None) == g.INVALID_ARG
    assert L.gemm_f16_nt_splitk_noalloc(1024, 1024, 65536, A + 1, B, D, 64, None) == g.UNSUPPORTED
    assert L.gemm_f16_nt_splitk_noalloc(0, 1024, 65536, A, B, D, 64, None) == g.OK
    assert g.status_string(g.SCRATCH) != g.status_string(12345)


def test_splitk_argument_errors_before_any_device_work():
    L = g.lib()
    assert L.gemm_f16_nt_splitk(256, 256, 512, A0, B0, D0, -1, None, 0, None) == g.INVALID_ARG
    assert L.gemm_f16_nt_splitk(256, 256, 512, A0, B0, D0, 65, None, 0, None) == g.INVALID_ARG
    assert L.gemm_f16_nt_splitk(256, 256, 512, A0 + 1, B0, D0, 2, None, 0, None) == g.UNSUPPORTED
    assert L.gemm_f16_nt_splitk(0, 256, 512, A0, B0, D0, 2, None, 0, None) == g.OK


from hypothesis import given, settings, strategies as st


@settings(max_examples=300, deadline=None)
@given(M=st.integers(1, 20000), N=st.integers(1, 20000), K8=st.integers(1, 2048),
       cus=st.sampled_from([80, 256, 304]))
def test_library_plan_picks_rungs_that_take_their_rows(M, N, K8, cus):
    """Whatever the library chooses for a shape, each launch of the plan is
    one its rung accepts: rows [0, m_top) on rung_top, the rest on rung_rest
    at the row offset the library launches them with."""
    K = 8 * K8
    A, B, D = 1 << 36, 2 << 36, 3 << 36          # fake, aligned, far apart
    rt, mt, rr = g.plan(M, N, K, cus)
    assert 0 < mt <= M
    assert g.check(rt, mt, N, K, A, B, D) == g.OK, (rt, mt)
    if mt == M:
        assert rr == 0
    else:
        assert rr != 0 and g.check(rr, M - mt, N, K, A + 2 * mt * K, B, D + 2 * mt * N) == g.OK, (rr, M - mt)


def test_rung13_only_where_tiles_are_few():
    """The library takes rung 13 only for single products whose 256 x 256
    tiles number fewer than the compute units (its model never beats the
    ring's by a fifth once the tiles fill them), and never where rung 12
    applies; its tile always keeps every workgroup's blocks within the
    instantiated set.  (The split-K entry may still prefer slices there:
    with a workspace, long K on a tiny output splits better.)"""
    tiles13 = {(1, 1, 2, 8), (1, 2, 2, 8), (2, 2, 1, 8), (2, 4, 1, 8), (3, 4, 1, 8), (2, 4, 1, 4), (4, 4, 1, 4)}
    for cus in (80, 256, 304):
        for M in (97, 128, 200, 256, 384, 512, 768, 1024, 1536, 2048, 4096, 8192):
            for N in (128, 1024, 2048, 4096, 8192, 14336, 28672):
                for K in (64, 1000, 2048, 4096, 8192, 14336, 28672):
                    top = g.plan(M, N, K, cus)[0]
                    if top != 13:
                        continue
                    tiles = -(-M // 256) * -(-N // 256)
                    assert tiles < cus, (M, N, K, cus)
                    assert g.ksplit_plan(13, M, N, K, cus) in tiles13
