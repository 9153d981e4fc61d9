// Rung 5: wave-specialized persistent kernel.
//
// The pages' step 7 gives the load engine and the math engine their own
// warps, joined by producer/consumer rings, inside a persistent kernel that
// walks a grouped tile order ("GEMM III - warp specialization & clusters to
// SOTA", Step 7; "TIRx GEMM detailed technical notes", V6 "Persistent Kernel
// and Tile Scheduler" and V7 "Warp Specialization and Pipelining").
//
// gfx950 form:
//  * 12 waves: waves 0-7 are consumers (two per SIMD), waves 8-11 are
//    producers (one per SIMD).  A gfx950 wave's register allocation is fixed
//    for the whole kernel (no per-role reallocation), so every wave gets
//    512/3 registers; a consumer holds a 128 x 64 fp32 accumulator (128
//    registers), the producers hold only addresses.
//  * Producers issue direct-to-LDS loads (no data registers), wait on their
//    own vmcnt, and arrive at the workgroup barrier; consumers only read LDS
//    and issue MFMA.  One s_barrier per k step, reached by all 12 waves,
//    carries both handoffs of the operand ring: "step k is in LDS"
//    (producer -> consumer) and "stage of step k-1 is free" (consumer ->
//    producer).  The producer starts with STAGES-1 free stages filled before
//    the first barrier; the consumers start blocked at that barrier -- the
//    pages' opposite initial phases.
//  * The step counter runs across tiles and never resets, so a refill can
//    prefetch the next tile's first k steps while the consumers finish the
//    current tile and write it back (the accumulator handoff of the pages'
//    second ring is the consumers' own registers here).
//  * Grid = number of CUs; workgroup w visits tiles xcd_slot(w) + i*grid of
//    the grouped order.
#pragma once

#include "common.hpp"
#include "ring.hpp"
#include "sched.hpp"

namespace g16 {
namespace ws {

template <int BK_, int STAGES_, int SWZ_>
struct Cfg {
    static constexpr int BM = 256, BN = 256, BK = BK_, STAGES = STAGES_, SWZ = SWZ_;
    static constexpr int CONSUMERS = 8, PRODUCERS = 4, WAVES = 12, THREADS = 64 * WAVES;
    static constexpr int CH = BK / 8;
    static constexpr int ROW_BYTES = BK * 2;
    static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;
    static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int A_LOADS = A_BYTES / 1024 / PRODUCERS;
    static constexpr int B_LOADS = B_BYTES / 1024 / PRODUCERS;
    static constexpr int LPW = A_LOADS + B_LOADS;
    static constexpr int WTM = 128, WTN = 64;  // consumer tile: 2 x 4 consumers
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int KSUB = BK / 16;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert((STAGES - 2) * LPW < 64, "vmcnt range");
};

template <class C>
__device__ __forceinline__ void consume_stage(const char* As, const char* Bs, int wm, int wn, int lane,
                                              f32x16 (&acc)[C::FM][C::FN])
{
#pragma unroll
    for (int kk = 0; kk < C::KSUB; ++kk) {
        const int chunk = 2 * kk + (lane >> 5);
        f16x8 a[C::FM], b[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
            a[i] = *reinterpret_cast<const f16x8*>(
                As + lds_chunk_offset<C::CH, C::SWZ>(wm + 32 * i + (lane & 31), chunk));
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            b[j] = *reinterpret_cast<const f16x8*>(
                Bs + lds_chunk_offset<C::CH, C::SWZ>(wn + 32 * j + (lane & 31), chunk));
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma_32x32x16(b[j], a[i], acc[i][j]);
    }
}

template <class C, bool EDGE>
__global__ __launch_bounds__(768, 1) void ws_kernel(const f16* __restrict__ A, const f16* __restrict__ B,
                                                    f16* __restrict__ D, int64_t M, int64_t N, int64_t K,
                                                    int64_t tiles_m, int64_t tiles_n)
{
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t total = tiles_m * tiles_n;
    const int64_t grid = gridDim.x, wg = blockIdx.x;
    const int64_t slot = xcd_slot(wg, grid);
    const int64_t my_tiles = slot < total ? (total - slot + grid - 1) / grid : 0;
    const int64_t KT = (K + C::BK - 1) / C::BK;
    const int64_t S = my_tiles * KT;  // k steps this workgroup runs, over all its tiles
    const int64_t ldb = K * 2;

    if (wave >= C::CONSUMERS) {
        // ------------------------------------------------------ producer
        const int p = wave - C::CONSUMERS;
        uint32_t a_off[C::A_LOADS], b_off[C::B_LOADS];
        int a_row[C::A_LOADS], b_row[C::B_LOADS], a_kc[C::A_LOADS], b_kc[C::B_LOADS];
        ring::lane_offsets<C, C::A_LOADS>(p, lane, ldb, a_off, a_row, a_kc);
        ring::lane_offsets<C, C::B_LOADS>(p, lane, ldb, b_off, b_row, b_kc);
        auto issue = [&](int64_t step) {
            const int64_t i = step / KT, kt = step - i * KT;
            const TileCoord tc = grouped_tile(persistent_tile(wg, i, grid), tiles_m, tiles_n);
            const int64_t m0 = tc.m_idx * C::BM, n0 = tc.n_idx * C::BN;
            char* st = smem + (int)(step % C::STAGES) * C::STAGE_BYTES;
            const int64_t k0 = kt * C::BK;
            ring::issue_loads<C, C::A_LOADS, EDGE>(reinterpret_cast<const char*>(A) + m0 * ldb, a_off, a_row,
                                                   a_kc, M - m0, K, k0, st, p);
            ring::issue_loads<C, C::B_LOADS, EDGE>(reinterpret_cast<const char*>(B) + n0 * ldb, b_off, b_row,
                                                   b_kc, N - n0, K, k0, st + C::A_BYTES, p);
        };
#pragma unroll
        for (int s = 0; s < C::STAGES - 1; ++s)
            if (s < S) issue(s);
        for (int64_t g = 0; g < S; ++g) {
            if (g + C::STAGES - 2 < S)
                wait_vmcnt<(C::STAGES - 2) * C::LPW>();
            else
                wait_vmcnt<0>();
            wg_barrier();
            const int64_t nk = ring_refill_after(g - 1, C::STAGES, S);
            if (nk >= 0) issue(nk);
        }
        return;
    }

    // ---------------------------------------------------------- consumer
    const int c = wave;
    const int wm = (c >> 2) * C::WTM, wn = (c & 3) * C::WTN;
    int64_t g = 0;
    for (int64_t i = 0; i < my_tiles; ++i) {
        const TileCoord tc = grouped_tile(persistent_tile(wg, i, grid), tiles_m, tiles_n);
        const int64_t m0 = tc.m_idx * C::BM, n0 = tc.n_idx * C::BN;
        f32x16 acc[C::FM][C::FN];
#pragma unroll
        for (int a = 0; a < C::FM; ++a)
#pragma unroll
            for (int b = 0; b < C::FN; ++b) acc[a][b] = f32x16{};
        for (int64_t kt = 0; kt < KT; ++kt, ++g) {
            wg_barrier();
            const char* st = smem + (int)(g % C::STAGES) * C::STAGE_BYTES;
            consume_stage<C>(st, st + C::A_BYTES, wm, wn, lane, acc);
        }
        const bool full = !EDGE || (m0 + C::BM <= M && n0 + C::BN <= N && N % 4 == 0);
#pragma unroll
        for (int a = 0; a < C::FM; ++a)
#pragma unroll
            for (int b = 0; b < C::FN; ++b) {
                const int64_t mb = m0 + wm + 32 * a, nb = n0 + wn + 32 * b;
                if (full)
                    store_block<true>(D, N, M, N, mb, nb, acc[a][b], lane);
                else
                    store_block<false>(D, N, M, N, mb, nb, acc[a][b], lane, N % 4 == 0);
            }
    }
}

}  // namespace ws
}  // namespace g16
