// Rungs 12 and 13: K split among a workgroup's waves on small output tiles.
//
// Rung 12 takes products with one side of at most 96 rows (M <= 96 or
// N <= 96), the tile-starved shapes of small-batch inference (e.g. 16 x
// 4096 x 14336); rung 13 takes products whose 128- and 256-row tiles would
// leave most compute units idle for a long K (e.g. 256 x 1024 x 8192).
// Tiles of 128 or 256 rows leave most of such a tile empty or, with few
// tiles, most compute units idle, each of the few busy ones walking all of
// K.  Here every workgroup owns a small tile of the output: 16 * MT rows
// of the smaller side ("S") and 16 * NF rows of the larger side ("L"), all
// of S on rung 12 (MT <= 6), a 2-D grid of tiles on rung 13.  Its 8 waves
// split K between them: wave w contracts a contiguous range of 32-wide k
// chunks, and the waves' fp32 partial sums are added through LDS in wave
// order before the one fp16 rounding ("GEMM I - the tiled baseline", the
// problem statement; K split inside one workgroup, so no workspace and no
// second launch, in the spirit of the persistent scheduler of "TIRx GEMM
// detailed technical notes", V6, that keeps every compute unit on work).
//
// Loads: each 32-wide k chunk of a 16-row block is one MFMA fragment per
// lane (lane l: row l % 16, k elements 8 * (l / 16) .. + 7 of the chunk:
// the v_mfma_f32_16x16x32_f16 operand layout), but a load instruction in
// that layout touches 16 rows x 64 bytes.  Measured on MI355X such loads
// stream at ~35 GB/s per compute unit, so each wave instead loads four
// chunks (128 k) of a block at a time as 4 instructions of 4 rows x 256
// bytes (lane l: row 4u + l / 16, k elements 8 * (l % 16) .. + 7 of the
// 128), writes them into its own 4 KiB of LDS (16-byte slots XOR-swizzled
// by row, so neither the writes nor the reads conflict) and reads them back
// as fragments.  No barrier: only the wave itself reads its buffer.  The
// loads are latency-bound (each wave waits for its group before using it),
// so with DB = 2 a wave keeps two groups in flight: the next group's loads
// go out before the current group is used (registers allow it for up to 4
// blocks).  Rows on any 2-byte boundary (gfx950's global loads take
// unaligned addresses).  The rest of a wave's range after its whole
// 4-chunk groups, including the chunk that crosses K, is read as fragments
// directly: the crossing chunk as the row's last 8 elements, shifted
// (load_row_chunk, chunk_shift); this needs K >= 8.  Rows past the operand
// are read as its last row and their outputs are not stored.  The output
// block layout: lane l holds (S row 4 * (l / 16) + r, L row l % 16), r =
// 0..3.  Each output's sum runs in a fixed order (k chunks in order within
// a wave, then waves 0..7), so results repeat bit for bit, whatever DB.
#pragma once

#include "common.hpp"
#include "ring.hpp"
#include "sched.hpp"

namespace g16 {
namespace skinny {

constexpr int kWaves = 8;
constexpr int kMaxSmall = 96;   // rung 12: all of S in one workgroup, 16 * MT rows, MT <= 6 (more spills registers)

struct Args {
    const f16* S;   // smaller side: s_rows x K, row pitch ld_s
    const f16* L;   // larger side: l_rows x K, row pitch ld_l
    f16* D;
    int64_t ld_s, s_rows, ld_l, l_rows, K, ldd;
    uint32_t l_tiles, s_tiles;   // workgroups along L and along S
};

// Tile order.  L-major: workgroup b takes L tile b % l_tiles and S tile
// b / l_tiles, so the workgroups of a round (dealt to the XCDs in turn)
// cover whole rows of L tiles.  When L is large and takes more than one
// round, that reads it from HBM once per round; S-major instead gives each
// XCD a contiguous run of workgroups (xcd_slot) over groups of kSGroup S
// tiles by all L tiles, so the S tiles of one L tile run together on one
// XCD and L is read once.  Measured on MI355X (interleaved, the same bits):
// 128 x 8192 x 8192 59.5 -> 41.2 us, 4096 x 256 x 8192 44.8 -> 41.3,
// 256 x 4096 x 14336 66.3 -> 63.3; with one round or a small L it lost
// (512 x 2048 x 4096 22.4 -> 23.4), so it is taken only for L over
// kSMajorMinBytes and more than one round, and only on the tiles of 64 L
// rows (32 x 32 tiles ran 2x slower with the mapping's code in the kernel,
// 256 x 1024 x 8192 14.2 -> 30.6, whatever the order).
constexpr int64_t kSGroup = 8;
constexpr int64_t kSMajorMinBytes = int64_t(32) << 20;

// LDS of one workgroup: the waves' 4 KiB transposition buffers during the
// k loop, then (after a barrier) the waves' partial sums.
template <int MT, int NF, int NW = kWaves>
constexpr int lds_bytes()
{
    constexpr int red = NW * MT * NF * 64 * 16, tb = NW * 4096;
    return red > tb ? red : tb;
}

// TRANS = false: S is A (D[s][l]); TRANS = true: S is B (D[l][s]).
// DB: 4-chunk groups in flight per wave (1 or 2).  SMAJ: the S-major tile
// order (a template parameter: with the L-major order the kernel is the
// same code as without the option; measured on MI355X, a run-time choice
// made the 32 x 32 tile's loop twice as slow, 15.5 -> 30.8 us on 256 x
// 1024 x 8192).
template <int MT, int NF, int DB, bool TRANS, bool SMAJ = false, int NW = kWaves>
__global__ __launch_bounds__(64 * NW) void skinny_kernel(const Args g)
{
    static_assert(DB == 1 || DB == 2, "one or two groups in flight");
    constexpr int NB = MT + NF;   // 16-row blocks: MT of S, then NF of L
    __shared__ __attribute__((aligned(16))) char smem[lds_bytes<MT, NF, NW>()];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, kq = lane >> 4;
    int64_t i0, j0;
    if constexpr (SMAJ) {
        int64_t ty, tx;
        grouped_tile_in<int64_t>(xcd_slot(blockIdx.x, (int64_t)g.l_tiles * g.s_tiles), g.s_tiles, g.l_tiles, kSGroup,
                                 &ty, &tx);
        i0 = ty * 16 * MT;
        j0 = tx * 16 * NF;
    } else {
        const uint32_t ty = blockIdx.x / g.l_tiles, tx = blockIdx.x - ty * g.l_tiles;
        i0 = (int64_t)ty * 16 * MT;
        j0 = (int64_t)tx * 16 * NF;
    }
    auto row_ptr = [&](int b, int r) -> const char* {
        if (b < MT) {
            const int64_t rr = i0 + 16 * b + r;
            return reinterpret_cast<const char*>(g.S + (rr < g.s_rows ? rr : g.s_rows - 1) * g.ld_s);
        }
        const int64_t rr = j0 + 16 * (b - MT) + r;
        return reinterpret_cast<const char*>(g.L + (rr < g.l_rows ? rr : g.l_rows - 1) * g.ld_l);
    };
    const char* gptr[NB][4];   // group loads: row 4u + kq of block b
    const char* fptr[NB];      // fragment loads: row r16 of block b
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int u = 0; u < 4; ++u) gptr[b][u] = row_ptr(b, 4 * u + kq);
        fptr[b] = row_ptr(b, r16);
    }
    // this wave's chunks [c0, c1): whole groups of 4 chunks inside K, then the rest
    const int64_t K = g.K, chunks = (K + 31) / 32;
    const int64_t per = ((chunks + NW - 1) / NW + 3) / 4 * 4;
    const int64_t c0 = w * per, c1 = c0 + per < chunks ? c0 + per : chunks;
    const int64_t cw = c1 < K / 32 ? c1 : K / 32;
    const int64_t groups = cw > c0 ? (cw - c0) / 4 : 0;
    f32x4 acc[MT][NF];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[t][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mma = [&](const u32x4 (&sv)[NB]) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int f = 0; f < NF; ++f)
                acc[t][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, sv[t]),
                                                                   __builtin_bit_cast(f16x8, sv[MT + f]), acc[t][f], 0, 0, 0);
    };
    // LDS slots: the write of (row 4u + kq, 8-element group r16) and the
    // read of (row r16, group 4u + kq), 16-byte slots XOR-swizzled by row
    char* tb = smem + w * 4096;
    uint32_t wo[4], ro[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int row = 4 * u + kq, kg = 4 * u + kq;
        wo[u] = (uint32_t)(row * 256 + ((r16 ^ row) & 15) * 16);
        ro[u] = (uint32_t)(r16 * 256 + ((kg ^ r16) & 15) * 16);
    }
    typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
    auto load_group = [&](u32x4 (&v)[NB][4], int64_t c) {
        const int64_t kb = (c * 32 + 8 * r16) * 2;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int u = 0; u < 4; ++u) v[b][u] = *(const G16_GLOBAL u32x4_a2*)(gptr[b][u] + kb);
    };
    auto use_group = [&](const u32x4 (&v)[NB][4]) {
        u32x4 fr[4][NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4*>(tb + wo[u]) = v[b][u];
#pragma unroll
            for (int u = 0; u < 4; ++u) fr[u][b] = *reinterpret_cast<const u32x4*>(tb + ro[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) mma(fr[u]);
    };
    int64_t c = c0;
    if constexpr (DB == 1) {
        for (int64_t gi = 0; gi < groups; ++gi, c += 4) {
            u32x4 v[NB][4];
            load_group(v, c);
            use_group(v);
        }
    } else {
        // two register sets; the steady loop has no branch inside, so the
        // wait before each use covers only the group being used
        u32x4 v0[NB][4], v1[NB][4];
        int64_t gi = 0;
        if (groups > 0) load_group(v0, c);
        for (; gi + 2 < groups; gi += 2, c += 8) {
            load_group(v1, c + 4);
            use_group(v0);
            load_group(v0, c + 8);
            use_group(v1);
        }
        if (gi + 1 < groups) {
            load_group(v1, c + 4);
            use_group(v0);
            use_group(v1);
            c += 8;
        } else if (gi < groups) {
            use_group(v0);
            c += 4;
        }
    }
    for (; c < c1; ++c) {
        const int kk = (int)(c * 32 + 8 * kq);
        u32x4 fv[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) fv[b] = chunk_shift(load_row_chunk(fptr[b], kk, (int)K, true), kk, (int)K);
        mma(fv);
    }
    // the waves' partial sums (in the LDS the buffers used, once every wave
    // is done with its buffer), added in wave order, rounded once
    f32x4* red = reinterpret_cast<f32x4*>(smem);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int f = 0; f < NF; ++f) red[(w * MT * NF + t * NF + f) * 64 + lane] = acc[t][f];
    __syncthreads();
    for (int b = w; b < MT * NF; b += NW) {
        f32x4 sum = red[b * 64 + lane];
#pragma unroll
        for (int v = 1; v < NW; ++v) sum += red[(v * MT * NF + b) * 64 + lane];
        const int t = b / NF, f = b % NF;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t si = i0 + 16 * t + 4 * kq + r, lj = j0 + 16 * f + r16;
            if (si < g.s_rows && lj < g.l_rows) {
                if (TRANS)
                    g.D[lj * g.ldd + si] = (f16)sum[r];
                else
                    g.D[si * g.ldd + lj] = (f16)sum[r];
            }
        }
    }
}

// A workgroup tile: 16 * mt rows of S and 16 * nf rows of L, db groups in
// flight, nw waves splitting K.
struct Tile {
    int mt, nf, db, nw = kWaves;
};

// The tiles of 64 L rows that run in the S-major order (when L is large
// and takes more than one round).  Rung 13's 4-wave 64 x 64 tile keeps the
// L-major order: measured on MI355X it ran 3-30% slower in the S-major one
// (256 x 8192 x 8192 69.4 -> 77.2 us, 128 x 8192 x 8192 36.7 -> 42.5).
inline bool smajor_tile(const Tile& t) { return t.nf == 4 && t.mt <= 3; }

// Rung 12's tile: all of S (mt = ceil(S / 16)) and 16 or 32 rows of L.
// 32 L rows ("wide") need every compute unit to get a workgroup; measured
// on MI355X (16 or 32 rows of S, L of 4096-28672 rows, K of 4096-28672)
// they pay from K = 14336 for up to 32 rows of S (16 x 8192 x 28672: 79.9
// us against 87.3 with 16 rows, 32 x 14336 x 14336: 87.7 against 103.3)
// and lose below it (16 x 14336 x 8192: 38.1 against 34.9), and from 48
// rows of S they pay at any K (64 x 8192 x 8192 28.5 against 35.4).  With
// 16 rows of S and one L block a wave keeps two groups in flight (16 x
// 4096 x 14336 24.3 -> 19.1 us, 16 x 14336 x 4096 22.9 -> 18.8); other
// tiles gain nothing from it.
constexpr int64_t kWideMinK = 12288;

inline Tile skinny_tile(int64_t s_rows, int64_t l_rows, int64_t K, int cus)
{
    const int mt = (int)((s_rows + 15) / 16);
    const bool wide = (l_rows + 31) / 32 >= (int64_t)cus;
    if (mt <= 2) {
        if (wide && K >= kWideMinK) return Tile{mt, 2, 1};
        return Tile{mt, 1, mt == 1 ? 2 : 1};
    }
    return Tile{mt, wide ? 2 : 1, 1};
}

// Rung 13's tiles, and a model of their time in microseconds: a workgroup
// streams (mt + nf) 16-row blocks of K elements at a rate of its own (one
// workgroup per compute unit, latency-bound loads), rounds of workgroups
// over the compute units, plus ~3 us of launch and reduction.  The 8-wave
// tiles' ~75 GB/s was fitted on MI355X over 75 shapes of 128-2048 x
// 1024-14336 x 1024-14336 rows: on the 29 of them where these tiles beat
// the ring kernels, the tile the model picks runs within 2.3% of the best
// of 16 tiles on average (16% at worst).  (6 x 2 blocks, best on a few
// shapes, never has the smallest model: 3 x 4 has the same workgroup count
// with fewer blocks.)
//
// Two tiles split K among 4 waves, each with a SIMD's whole register file:
// 32 x 64 (~90 GB/s, taken only with more than one round of workgroups:
// two of them fit on a compute unit, and in a single round the 8-wave form
// splits each tile's K finer, 128 x 4096 x 4096 13.1 against 15.2 us), and
// 64 x 64 (~65 GB/s: its 8 blocks per wave spill registers with 8 waves).
// Measured on MI355X over 20 shapes of 128-1024 x 1024-8192 x 4096-28672
// (interleaved, bitwise equal on integer operands) they make the model's
// pick 1.067x faster (geometric mean) and within 1.2% of the best of the
// seven tiles: 256 x 4096 x 4096 23.7 -> 21.1 us, 256 x 8192 x 8192 96.8 ->
// 65.5, 128 x 8192 x 28672 171.3 -> 147.6, 1024 x 1024 x 8192 39.4 -> 37.3.
struct Tile13 {
    Tile t;
    double bytes_per_us;
    bool multi_round;   // only with more workgroups than compute units
};
constexpr Tile13 kTiles13[] = {{{1, 1, 2}, 75e3, false}, {{1, 2, 2}, 75e3, false}, {{2, 2, 1}, 75e3, false},
                               {{2, 4, 1}, 75e3, false}, {{3, 4, 1}, 75e3, false}, {{2, 4, 1, 4}, 90e3, true},
                               {{4, 4, 1, 4}, 65e3, false}};
constexpr double kFixedUs = 3.0;

inline int64_t tile_workgroups(int64_t s_rows, int64_t l_rows, const Tile& t)
{
    return ((l_rows + 16 * t.nf - 1) / (16 * t.nf)) * ((s_rows + 16 * t.mt - 1) / (16 * t.mt));
}

inline double tile_model_us(int64_t s_rows, int64_t l_rows, int64_t K, int cus, const Tile13& c)
{
    const int64_t rounds = (tile_workgroups(s_rows, l_rows, c.t) + cus - 1) / cus;
    return (double)rounds * (double)(c.t.mt + c.t.nf) * 32.0 * (double)K / c.bytes_per_us + kFixedUs;
}

// The tile with the smallest model (the first of the list on ties).
inline Tile ksplit_tile(int64_t s_rows, int64_t l_rows, int64_t K, int cus, double* model_us)
{
    Tile best = kTiles13[0].t;
    double bt = tile_model_us(s_rows, l_rows, K, cus, kTiles13[0]);
    for (const Tile13& c : kTiles13) {
        if (c.multi_round && tile_workgroups(s_rows, l_rows, c.t) <= (int64_t)cus) continue;
        const double v = tile_model_us(s_rows, l_rows, K, cus, c);
        if (v < bt) {
            bt = v;
            best = c.t;
        }
    }
    if (model_us) *model_us = bt;
    return best;
}

}  // namespace skinny
}  // namespace g16
