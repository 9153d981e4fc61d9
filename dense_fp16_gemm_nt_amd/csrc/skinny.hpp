// Rung 12: products with one side of at most 96 rows (M <= 96 or N <= 96),
// the tile-starved shapes of small-batch inference (e.g. 16 x 4096 x 14336).
//
// Tiles of 128 or 256 rows leave most of such a tile empty and, with few
// tiles, most compute units idle, each of the few busy ones walking all of
// K.  Here every workgroup owns 16 * NF rows of the large side ("L") and
// all rows of the small side ("S", 16 * MT rows, MT <= 6), so the large
// side alone sets the workgroup count, and its 8 waves split K between
// them: wave w contracts a contiguous range of 32-wide k chunks, and the
// waves' fp32 partial sums are added through LDS in wave order before the
// one fp16 rounding ("GEMM I - the tiled baseline", the problem statement;
// K split inside one workgroup, so no workspace and no second launch, in
// the spirit of the persistent scheduler of "TIRx GEMM detailed technical
// notes", V6, that keeps every compute unit on work).
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
// as fragments.  No barrier: only the wave itself reads its buffer.  Rows
// on any 2-byte boundary (gfx950's global loads take unaligned addresses).
// The rest of a wave's range after its whole 4-chunk groups, including the
// chunk that crosses K, is read as fragments directly: the crossing chunk
// as the row's last 8 elements, shifted (load_row_chunk, chunk_shift);
// this needs K >= 8.  Rows past the operand are read as its last row and
// their outputs are not stored.  The output block layout: lane l holds
// (small row 4 * (l / 16) + r, large row l % 16), r = 0..3.  Each output's
// sum runs in a fixed order (k chunks in order within a wave, then waves
// 0..7), so results repeat bit for bit.
#pragma once

#include "common.hpp"
#include "ring.hpp"

namespace g16 {
namespace skinny {

constexpr int kWaves = 8;
constexpr int kMaxSmall = 96;   // rows of the small side: 16 * MT, MT <= 6 (more spills registers)

struct Args {
    const f16* S;   // small side: s_rows x K, row pitch ld_s
    const f16* L;   // large side: l_rows x K, row pitch ld_l
    f16* D;
    int64_t ld_s, s_rows, ld_l, l_rows, K, ldd;
};

// TRANS = false: S is A (D[s][l]); TRANS = true: S is B (D[l][s]).
template <int MT, int NF, bool TRANS>
__global__ __launch_bounds__(64 * kWaves) void skinny_kernel(const Args g)
{
    constexpr int NB = MT + NF;   // 16-row blocks: MT of S, then NF of L
    __shared__ f32x4 red[kWaves][MT * NF][64];
    __shared__ __attribute__((aligned(16))) char tbuf[kWaves][4096];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, kq = lane >> 4;
    const int64_t j0 = (int64_t)blockIdx.x * 16 * NF;
    auto row_ptr = [&](int b, int r) -> const char* {
        if (b < MT) {
            const int64_t rr = 16 * b + r;
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
    const int64_t per = ((chunks + kWaves - 1) / kWaves + 3) / 4 * 4;
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
    char* tb = tbuf[w];
    uint32_t wo[4], ro[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int row = 4 * u + kq, kg = 4 * u + kq;
        wo[u] = (uint32_t)(row * 256 + ((r16 ^ row) & 15) * 16);
        ro[u] = (uint32_t)(r16 * 256 + ((kg ^ r16) & 15) * 16);
    }
    typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
    int64_t c = c0;
    for (int64_t gi = 0; gi < groups; ++gi, c += 4) {
        const int64_t kb = (c * 32 + 8 * r16) * 2;
        u32x4 v[NB][4];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int u = 0; u < 4; ++u) v[b][u] = *(const G16_GLOBAL u32x4_a2*)(gptr[b][u] + kb);
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
    }
    for (; c < c1; ++c) {
        const int kk = (int)(c * 32 + 8 * kq);
        u32x4 fv[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) fv[b] = chunk_shift(load_row_chunk(fptr[b], kk, (int)K, true), kk, (int)K);
        mma(fv);
    }
    // the waves' partial sums, added in wave order, rounded once
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int f = 0; f < NF; ++f) red[w][t * NF + f][lane] = acc[t][f];
    __syncthreads();
    for (int b = w; b < MT * NF; b += kWaves) {
        f32x4 sum = red[0][b][lane];
#pragma unroll
        for (int v = 1; v < kWaves; ++v) sum += red[v][b][lane];
        const int t = b / NF, f = b % NF;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t si = 16 * t + 4 * kq + r, lj = j0 + 16 * f + r16;
            if (si < g.s_rows && lj < g.l_rows) {
                if (TRANS)
                    g.D[lj * g.ldd + si] = (f16)sum[r];
                else
                    g.D[si * g.ldd + lj] = (f16)sum[r];
            }
        }
    }
}

// Large-side rows per workgroup: 32 when that still gives every compute
// unit a workgroup, else 16 (measured on MI355X: 64 x 8192 x 8192 28.5 us
// with 32 rows against 35.4 with 16; 64 x 4096 x 4096 13.2 against 11.9).
inline int choose_nf(int64_t l_rows, int cus)
{
    return (l_rows + 31) / 32 >= (int64_t)cus ? 2 : 1;
}

}  // namespace skinny
}  // namespace g16
