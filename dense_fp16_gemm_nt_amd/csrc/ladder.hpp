// Rungs 1-3 of the ladder: synchronous, all-waves cooperative copy into
// swizzled LDS, then MFMA.  128 x 128 output tile per workgroup of 4 waves
// (256 threads); each wave owns a 64 x 64 quadrant = 2 x 2 blocks of the
// 32x32x16 MFMA.  BK = 64 (128-byte LDS rows, 8 chunks).
//
//  R1  one tile, K = 64, grid 1 x 1       ("GEMM I", Step 1)
//  R2  one tile, K-loop over 64-wide steps ("GEMM I", Step 2)
//  R3  2D grid, one workgroup per tile     ("GEMM I", Step 3); r3_any is
//      its general-operand form (any K, strides, 2-byte alignment)
#pragma once

#include "common.hpp"

namespace g16 {
namespace ladder {

constexpr int BM = 128, BN = 128, BK = 64, CH = BK / 8, SWZ = 1;
constexpr int THREADS = 256;

// Copy rows [r0, r0+128) x k-chunks [k0, k0+64) of a row-major (rows x K)
// operand into a swizzled LDS tile.  Rows >= rows and k >= K read as zero,
// so edge tiles and a K tail contribute nothing.
template <bool CHECK>
__device__ __forceinline__ void copy_tile(const f16* __restrict__ src, int64_t rows, int64_t K,
                                          int64_t r0, int64_t k0, char* lds, int t)
{
#pragma unroll
    for (int j = 0; j < (BM * CH) / THREADS; ++j) {
        const int q = t + THREADS * j;
        const int r = q / CH, c = q % CH;
        const int64_t gr = r0 + r, gk = k0 + 8 * c;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (!CHECK || (gr < rows && gk < K))
            v = *reinterpret_cast<const u32x4*>(src + gr * K + gk);
        *reinterpret_cast<u32x4*>(lds + lds_chunk_offset<CH, SWZ>(r, c)) = v;
    }
}

__device__ __forceinline__ f16x8 frag(const char* lds, int row, int chunk)
{
    return *reinterpret_cast<const f16x8*>(lds + lds_chunk_offset<CH, SWZ>(row, chunk));
}

// One 64-wide k step on the staged tiles: wave quadrant (wm, wn).
__device__ __forceinline__ void mma_step(const char* As, const char* Bs, int wm, int wn, int lane,
                                         f32x16 (&acc)[2][2])
{
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
        const int chunk = 2 * kk + (lane >> 5);
        f16x8 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = frag(As, wm + 32 * i + (lane & 31), chunk);
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = frag(Bs, wn + 32 * j + (lane & 31), chunk);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma_32x32x16(b[j], a[i], acc[i][j]);
    }
}

// R1: the smallest correct tile.  M = N = 128, K = 64, one workgroup.
__global__ __launch_bounds__(THREADS) void r1_single_tile(const f16* __restrict__ A,
                                                          const f16* __restrict__ B,
                                                          f16* __restrict__ D)
{
    __shared__ __attribute__((aligned(128))) char As[BM * BK * 2];
    __shared__ __attribute__((aligned(128))) char Bs[BN * BK * 2];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    // (1) all threads copy, then publish
    copy_tile<false>(A, BM, BK, 0, 0, As, t);
    copy_tile<false>(B, BN, BK, 0, 0, Bs, t);
    __syncthreads();
    // (2) every wave multiplies its quadrant; the first (only) step
    //     overwrites the accumulator (starts from zero)
    const int wm = 64 * (w >> 1), wn = 64 * (w & 1);
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    mma_step(As, Bs, wm, wn, lane, acc);
    // (3) round once and write back
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) store_block<true>(D, BN, BM, BN, wm + 32 * i, wn + 32 * j, acc[i][j], lane);
}

// R2 / R3: K-loop over 64-wide steps into one accumulator; the grid covers
// ceil(M/128) x ceil(N/128) tiles (R2 launches 1 x 1 on a 128 x 128
// problem).  blockIdx.x selects the tile row (m), blockIdx.y the tile
// column (n), as in the pages' 2D grid.  Two barriers per step: one
// publishes the copy, one keeps the next copy from overwriting a tile that
// a slower wave is still reading.
__global__ __launch_bounds__(THREADS) void r23_kloop_grid(const f16* __restrict__ A,
                                                          const f16* __restrict__ B,
                                                          f16* __restrict__ D, int64_t M, int64_t N,
                                                          int64_t K)
{
    __shared__ __attribute__((aligned(128))) char As[BM * BK * 2];
    __shared__ __attribute__((aligned(128))) char Bs[BN * BK * 2];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t m_st = (int64_t)blockIdx.x * BM;
    const int64_t n_st = (int64_t)blockIdx.y * BN;
    const int wm = 64 * (w >> 1), wn = 64 * (w & 1);
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    const bool inner = (m_st + BM <= M) && (n_st + BN <= N);
    for (int64_t k0 = 0; k0 < K; k0 += BK) {
        if (inner && k0 + BK <= K) {
            copy_tile<false>(A + m_st * K, BM, K, 0, k0, As, t);
            copy_tile<false>(B + n_st * K, BN, K, 0, k0, Bs, t);
        } else {
            copy_tile<true>(A + m_st * K, M - m_st, K, 0, k0, As, t);
            copy_tile<true>(B + n_st * K, N - n_st, K, 0, k0, Bs, t);
        }
        __syncthreads();
        mma_step(As, Bs, wm, wn, lane, acc);
        __syncthreads();
    }
    const bool full = inner && (N % 4 == 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (full)
                store_block<true>(D, N, M, N, m_st + wm + 32 * i, n_st + wn + 32 * j, acc[i][j], lane);
            else
                store_block<false>(D, N, M, N, m_st + wm + 32 * i, n_st + wn + 32 * j, acc[i][j], lane, N % 4 == 0);
        }
}


// General operands on R3's structure: any K, any leading dimensions and
// batch strides, any 2-byte alignment ("GEMM I" claims any M, N, K; the
// fast rungs need 16-byte rows).  Each thread fills its 16-byte LDS chunks
// element by element (zero outside M, N, K), then the R3 K-loop runs on the
// swizzled tile; D is written element by element unless every row start of
// every batch entry is 8-byte aligned.  Grid (tiles_m, tiles_n, batch).
__device__ __forceinline__ void copy_tile_any(const f16* __restrict__ src, int64_t ld, int64_t rows, int64_t K,
                                              int64_t k0, char* lds, int t)
{
#pragma unroll
    for (int j = 0; j < (BM * CH) / THREADS; ++j) {
        const int q = t + THREADS * j;
        const int r = q / CH, c = q % CH;
        const int64_t gk = k0 + 8 * c;
        f16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (r < rows && gk + e < K) ? src[r * ld + gk + e] : (f16)0;
        *reinterpret_cast<f16x8*>(lds + lds_chunk_offset<CH, SWZ>(r, c)) = v;
    }
}

__global__ __launch_bounds__(THREADS) void r3_any(const GemmArgs g)
{
    __shared__ __attribute__((aligned(128))) char As[BM * BK * 2];
    __shared__ __attribute__((aligned(128))) char Bs[BN * BK * 2];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t m_st = (int64_t)blockIdx.x * BM, n_st = (int64_t)blockIdx.y * BN, b = blockIdx.z;
    const f16* __restrict__ A = g.A + b * g.sa + m_st * g.lda;
    const f16* __restrict__ B = g.B + b * g.sb + n_st * g.ldb;
    f16* __restrict__ D = g.D + b * g.sd;
    const int wm = 64 * (w >> 1), wn = 64 * (w & 1);
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    for (int64_t k0 = 0; k0 < g.K; k0 += BK) {
        copy_tile_any(A, g.lda, g.M - m_st, g.K, k0, As, t);
        copy_tile_any(B, g.ldb, g.N - n_st, g.K, k0, Bs, t);
        __syncthreads();
        mma_step(As, Bs, wm, wn, lane, acc);
        __syncthreads();
    }
    const bool vec = ((uintptr_t)g.D & 7) == 0 && g.ldd % 4 == 0 && g.sd % 4 == 0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            store_block<false>(D, g.ldd, g.M, g.N, m_st + wm + 32 * i, n_st + wn + 32 * j, acc[i][j], lane, vec);
}

}  // namespace ladder
}  // namespace g16
