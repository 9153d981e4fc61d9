// Rung 4: pipelined LDS ring fed by direct-to-LDS loads.
//
// The pages' step 4/5 replace the threads' copy with an asynchronous copy
// engine and then double-buffer the operand tiles so the next K tile
// streams in while the current one is multiplied ("TIRx GEMM detailed
// technical notes", V4 "TMA Async Load and Store" and V5 "Software Pipeline
// with Double-Buffered SMEM").  On gfx950 the copy engine is the
// direct-to-LDS form of the vector memory load (global_load_lds_dwordx4):
// each lane names a 16-byte global source and the data lands in LDS without
// passing through registers; completion is the issuing wave's vmcnt.
//
// Workgroup tile BM x BN (256 x 256), BK-wide k steps, STAGES-deep ring.
// 4 waves (one per SIMD), 2 x 2, each owning a (BM/2) x (BN/2) = 128 x 128
// accumulator (16 blocks of 32x32, 256 fp32 per lane).  Every wave issues
// its share of the loads and then multiplies; one workgroup barrier per k
// step both publishes step k and releases the stage of step k-1.
#pragma once

#include "common.hpp"
#include "sched.hpp"

namespace g16 {

// 16 zero bytes: the source of every out-of-range lane of an edge tile.
__device__ __attribute__((aligned(64))) uint32_t g_zero_line[16] = {0};

namespace ring {

template <int BM_, int BN_, int BK_, int STAGES_, int SWZ_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, SWZ = SWZ_;
    static constexpr int WAVES = 4, THREADS = 256;
    static constexpr int CH = BK / 8;                 // 16-byte chunks per LDS row
    static constexpr int ROW_BYTES = BK * 2;
    static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;  // one wave load = 1 KiB
    static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int A_LOADS = A_BYTES / 1024 / WAVES;  // per wave per step
    static constexpr int B_LOADS = B_BYTES / 1024 / WAVES;
    static constexpr int LPW = A_LOADS + B_LOADS;
    static constexpr int WTM = BM / 2, WTN = BN / 2;  // wave tile
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int KSUB = BK / 16;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert((STAGES - 2) * LPW < 64, "vmcnt range");
    static_assert(A_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0, "load split");
};

// Per-lane source offsets (bytes, relative to the tile's first row at k=0)
// for this wave's loads of one operand.  Load j of wave w covers tile rows
// [(w*NL + j)*RPL, +RPL); lane l lands at row l / CH of that group and
// physical chunk l % CH, so it fetches logical chunk (l % CH) ^ swz(row).
template <class C, int NL>
__device__ __forceinline__ void lane_offsets(int w, int lane, int64_t ld_bytes, uint32_t (&off)[NL],
                                             int (&row)[NL], int (&kc)[NL])
{
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int r = (w * NL + j) * C::ROWS_PER_LOAD + lane / C::CH;
        const int c = (lane % C::CH) ^ swz_of_row<C::CH, C::SWZ>(r);
        row[j] = r;
        kc[j] = c * 8;
        off[j] = (uint32_t)(r * ld_bytes + c * 16);
    }
}

// Issue this wave's NL direct-to-LDS loads of one operand for k offset k0
// into LDS region `dst` (wave-uniform).
template <class C, int NL, bool EDGE>
__device__ __forceinline__ void issue_loads(const char* base, const uint32_t (&off)[NL], const int (&row)[NL],
                                            const int (&kc)[NL], int64_t rows_valid, int64_t K, int64_t k0,
                                            char* dst, int w)
{
    const char* kbase = base + k0 * 2;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        char* d = dst + (w * NL + j) * 1024;
        if (EDGE) {
            const bool ok = row[j] < rows_valid && k0 + kc[j] < K;
            const void* src = ok ? (const void*)(kbase + off[j]) : (const void*)g_zero_line;
            load_lds_16(src, d);
        } else {
            load_lds_16(kbase + off[j], d);
        }
    }
}

template <class C>
__device__ __forceinline__ f16x8 frag(const char* tile, int row, int chunk)
{
    return *reinterpret_cast<const f16x8*>(tile + lds_chunk_offset<C::CH, C::SWZ>(row, chunk));
}

// Multiply one staged k step into the wave's accumulators.
template <class C>
__device__ __forceinline__ void mma_stage(const char* As, const char* Bs, int wm, int wn, int lane,
                                          f32x16 (&acc)[C::FM][C::FN])
{
#pragma unroll
    for (int kk = 0; kk < C::KSUB; ++kk) {
        const int chunk = 2 * kk + (lane >> 5);
        f16x8 a[C::FM], b[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) a[i] = frag<C>(As, wm + 32 * i + (lane & 31), chunk);
#pragma unroll
        for (int j = 0; j < C::FN; ++j) b[j] = frag<C>(Bs, wn + 32 * j + (lane & 31), chunk);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma_32x32x16(b[j], a[i], acc[i][j]);
    }
}

template <class C, bool EDGE>
__global__ __launch_bounds__(256, 1) void ring_kernel(const f16* __restrict__ A, const f16* __restrict__ B,
                                                      f16* __restrict__ D, int64_t M, int64_t N, int64_t K,
                                                      int64_t tiles_m, int64_t tiles_n)
{
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);

    const int64_t total = tiles_m * tiles_n;
    const TileCoord tc = grouped_tile(xcd_slot(blockIdx.x, total), tiles_m, tiles_n);
    const int64_t m0 = tc.m_idx * C::BM, n0 = tc.n_idx * C::BN;

    const int64_t ldb = K * 2;
    const char* a_base = reinterpret_cast<const char*>(A) + m0 * ldb;
    const char* b_base = reinterpret_cast<const char*>(B) + n0 * ldb;
    uint32_t a_off[C::A_LOADS], b_off[C::B_LOADS];
    int a_row[C::A_LOADS], b_row[C::B_LOADS], a_kc[C::A_LOADS], b_kc[C::B_LOADS];
    lane_offsets<C, C::A_LOADS>(w, lane, ldb, a_off, a_row, a_kc);
    lane_offsets<C, C::B_LOADS>(w, lane, ldb, b_off, b_row, b_kc);
    const int64_t a_rows = M - m0, b_rows = N - n0;

    const int64_t KT = (K + C::BK - 1) / C::BK;
    auto issue = [&](int64_t step) {
        char* st = smem + (int)(step % C::STAGES) * C::STAGE_BYTES;
        const int64_t k0 = step * C::BK;
        issue_loads<C, C::A_LOADS, EDGE>(a_base, a_off, a_row, a_kc, a_rows, K, k0, st, w);
        issue_loads<C, C::B_LOADS, EDGE>(b_base, b_off, b_row, b_kc, b_rows, K, k0, st + C::A_BYTES, w);
    };

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16{};

    // prologue: steps 0 .. STAGES-2
#pragma unroll
    for (int s = 0; s < C::STAGES - 1; ++s)
        if (s < KT) issue(s);

    const int wm = (w >> 1) * C::WTM, wn = (w & 1) * C::WTN;
    for (int64_t kt = 0; kt < KT; ++kt) {
        // this wave's loads of step kt have landed
        if (kt + C::STAGES - 2 < KT)
            wait_vmcnt<(C::STAGES - 2) * C::LPW>();
        else
            wait_vmcnt<0>();
        // every wave's loads of step kt are visible, and every wave has
        // finished reading the stage of step kt-1
        wg_barrier();
        const int64_t nk = ring_refill_after(kt - 1, C::STAGES, KT);
        if (nk >= 0) issue(nk);
        const char* st = smem + (int)(kt % C::STAGES) * C::STAGE_BYTES;
        mma_stage<C>(st, st + C::A_BYTES, wm, wn, lane, acc);
    }

    const bool full = !EDGE || (m0 + C::BM <= M && n0 + C::BN <= N && N % 4 == 0);
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            const int64_t mb = m0 + wm + 32 * i, nb = n0 + wn + 32 * j;
            if (full)
                store_block<true>(D, N, M, N, mb, nb, acc[i][j], lane);
            else
                store_block<false>(D, N, M, N, mb, nb, acc[i][j], lane);
        }
}

}  // namespace ring
}  // namespace g16
