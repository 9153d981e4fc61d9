// Rung 12: products with one side of at most 64 rows (M <= 64 or N <= 64),
// the tile-starved shapes of small-batch inference (e.g. 16 x 4096 x 14336).
//
// Tiles of 128 or 256 rows leave most of such a tile empty and, with few
// tiles, most compute units idle, each of the few busy ones walking all of
// K.  Here every workgroup owns 16 * NF rows of the large side ("L") and
// all rows of the small side ("S", 16 * MT rows, MT <= 4), so the large
// side alone sets the workgroup count, and its 8 waves split K between
// them: wave w contracts a contiguous range of 32-wide k chunks, and the
// waves' fp32 partial sums are added through LDS in wave order before the
// one fp16 rounding ("GEMM I - the tiled baseline", the problem statement;
// K split inside one workgroup, so no workspace and no second launch, in
// the spirit of the persistent scheduler of "TIRx GEMM detailed technical
// notes", V6, that keeps every compute unit on work).
//
// Operands go straight from global memory into MFMA operand registers, one
// 16-byte load per lane per fragment (no LDS staging: the large side is
// read once, so only the memory-level parallelism of the waves' loads
// matters).  v_mfma_f32_16x16x32_f16 lane layout: lane l supplies row
// l % 16 of a 16-row block at k elements 8 * (l / 16) .. + 7 of the chunk,
// for both operands, and holds the outputs (row 4 * (l / 16) + r, column
// l % 16), r = 0..3, of the 16 x 16 block (S rows by L rows).
//
// Any 2-byte alignment of rows (gfx950's global loads take unaligned
// addresses) and any K >= 8: the chunk that crosses K is read as the
// row's last 8 elements and shifted (load_row_chunk, chunk_shift).  Rows
// past the operand are read as its last row and their outputs are not
// stored.  Each output's sum runs in a fixed order (k chunks in order
// within a wave, then waves 0..7), so results repeat bit for bit.
#pragma once

#include "common.hpp"
#include "ring.hpp"

namespace g16 {
namespace skinny {

constexpr int kWaves = 8;
constexpr int kMaxSmall = 64;   // rows of the small side: 16 * MT, MT <= 4

struct Args {
    const f16* S;   // small side: s_rows x K, row pitch ld_s
    const f16* L;   // large side: l_rows x K, row pitch ld_l
    f16* D;
    int64_t ld_s, s_rows, ld_l, l_rows, K, ldd;
};

// TRANS = false: S is A (D[s][l]); TRANS = true: S is B (D[l][s]).
template <int MT, int NF, int U, bool TRANS>
__global__ __launch_bounds__(64 * kWaves) void skinny_kernel(const Args g)
{
    __shared__ f32x4 red[kWaves][MT * NF][64];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, kq = lane >> 4;
    const int64_t j0 = (int64_t)blockIdx.x * 16 * NF;
    const char* lrow[NF];
    const char* srow[MT];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int64_t r = j0 + 16 * f + r16;
        lrow[f] = reinterpret_cast<const char*>(g.L + (r < g.l_rows ? r : g.l_rows - 1) * g.ld_l);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int64_t r = 16 * t + r16;
        srow[t] = reinterpret_cast<const char*>(g.S + (r < g.s_rows ? r : g.s_rows - 1) * g.ld_s);
    }
    // this wave's chunks [c0, c1); [c0, cf) lie wholly inside K (at most
    // one chunk, the last of K, crosses it)
    const int64_t K = g.K, chunks = (K + 31) / 32, per = (chunks + kWaves - 1) / kWaves;
    const int64_t c0 = w * per, c1 = c0 + per < chunks ? c0 + per : chunks;
    const int64_t whole = K / 32, cf = c1 < whole ? c1 : (whole > c0 ? whole : c0);
    f32x4 acc[MT][NF];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[t][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mma = [&](const u32x4 (&sv)[MT], const u32x4 (&lv)[NF]) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int f = 0; f < NF; ++f)
                acc[t][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, sv[t]),
                                                                   __builtin_bit_cast(f16x8, lv[f]), acc[t][f], 0, 0, 0);
    };
    typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
    int64_t c = c0;
    for (; c + U <= cf; c += U) {
        // U chunks' loads first, then their MFMAs
        u32x4 lv[U][NF], sv[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t kb = ((c + u) * 32 + 8 * kq) * 2;
#pragma unroll
            for (int f = 0; f < NF; ++f) lv[u][f] = *(const G16_GLOBAL u32x4_a2*)(lrow[f] + kb);
#pragma unroll
            for (int t = 0; t < MT; ++t) sv[u][t] = *(const G16_GLOBAL u32x4_a2*)(srow[t] + kb);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) mma(sv[u], lv[u]);
    }
    for (; c < c1; ++c) {
        const int kk = (int)(c * 32 + 8 * kq);
        u32x4 lv[NF], sv[MT];
#pragma unroll
        for (int f = 0; f < NF; ++f) lv[f] = chunk_shift(load_row_chunk(lrow[f], kk, (int)K, true), kk, (int)K);
#pragma unroll
        for (int t = 0; t < MT; ++t) sv[t] = chunk_shift(load_row_chunk(srow[t], kk, (int)K, true), kk, (int)K);
        mma(sv, lv);
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

// Large-side rows per workgroup: the largest 16 * NF (NF in 4, 2, 1) that
// still gives at least three workgroups per four compute units (more rows
// per workgroup re-read the small side less often; measured on MI355X,
// 16 x 28672 x 8192: 106.6 / 111.1 / 124.4 us for NF = 4 / 2 / 1).
inline int choose_nf(int64_t l_rows, int cus)
{
    for (int nf = 4; nf > 1; nf /= 2)
        if ((l_rows + 16 * nf - 1) / (16 * nf) * 4 >= (int64_t)cus * 3) return nf;
    return 1;
}

}  // namespace skinny
}  // namespace g16
