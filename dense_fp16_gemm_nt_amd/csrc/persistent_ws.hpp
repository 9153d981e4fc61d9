// Rung 5: wave-specialized persistent kernel.
//
// The pages' step 7 gives the load engine and the math engine their own
// warps, joined by producer/consumer rings, inside a persistent kernel that
// walks a grouped tile order ("GEMM III - warp specialization & clusters to
// SOTA", Step 7; "TIRx GEMM detailed technical notes", V6 "Persistent Kernel
// and Tile Scheduler" and V7 "Warp Specialization and Pipelining").
//
// gfx950 form:
//  * 12 waves (the library's configuration; Cfg takes others): waves 0-7
//    are consumers (two per SIMD), waves 8-11 are producers (one per SIMD).
//    A gfx950 wave's register allocation is fixed for the whole kernel (no
//    per-role reallocation), so every wave gets 512/3 registers; a consumer
//    holds a 128 x 64 fp32 accumulator (128 registers) and reads the next
//    sub-step's fragments while the current one's MFMAs run, the producers
//    hold only addresses.
//  * Producers issue direct-to-LDS loads (no data registers); consumers only
//    read LDS and issue MFMA.  The two roles meet through two counters per
//    ring stage in LDS instead of a workgroup barrier (the pages' full and
//    empty mbarriers of each stage): a producer adds 1 to ready[s] once its
//    own loads of the step in stage s have landed (its vmcnt), a consumer
//    adds 1 to free[s] once its fragment reads of that step are done.  A
//    consumer waits only for the stage it reads next, a producer only for
//    the stage it refills next, so the producers run up to STAGES steps
//    ahead of the consumers, and a consumer never waits for the other
//    consumers.  The targets (handoff_ready_target, handoff_free_target in
//    sched.hpp) start the producers with every stage free and the
//    consumers blocked -- the pages' opposite initial phases -- and the
//    counters never reset, so a wait names an absolute count that no
//    earlier lap can meet.  Only the counters' initialisation takes a
//    workgroup barrier.
//  * Every wait is bounded (kSpinLimit polls); a wave whose wait runs out
//    stops waiting and its tiles are written as NaN, so a protocol error
//    shows as a failed result instead of a hung GPU.
//  * The step counter runs across tiles and never resets, so the producers
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

// CM x CN consumer waves of 128 x 64 outputs each (workgroup tile
// 128*CM x 64*CN) and P producer waves; DBUF: consumers read the next
// sub-step's fragments into a second register set while the MFMAs of the
// current one run (needs the registers of 8 waves or fewer per CU).
template <int BK_, int STAGES_, int SWZ_, int CM_ = 2, int CN_ = 4, int P_ = 4, bool DBUF_ = false>
struct Cfg {
    static constexpr int CM = CM_, CN = CN_;
    static constexpr int BM = 128 * CM_, BN = 64 * CN_, BK = BK_, STAGES = STAGES_, SWZ = SWZ_;
    static constexpr int CONSUMERS = CM_ * CN_, PRODUCERS = P_, WAVES = CM_ * CN_ + P_, THREADS = 64 * WAVES;
    static constexpr bool DBUF = DBUF_;
    static constexpr int CH = BK / 8;
    static constexpr int ROW_BYTES = BK * 2;
    static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;
    static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int A_LOADS = A_BYTES / 1024 / PRODUCERS;
    static constexpr int B_LOADS = B_BYTES / 1024 / PRODUCERS;
    static constexpr int LPW = A_LOADS + B_LOADS;
    static constexpr int WTM = 128, WTN = 64;  // consumer tile
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int KSUB = BK / 16;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert((STAGES - 1) * LPW < 64, "vmcnt range");
};

// Polls of one handoff wait before it gives up (a poll is an LDS read,
// its wait and a short sleep, ~250 cycles: ~0.3 s in all, against a few
// microseconds for the longest wait of a working ring).
constexpr uint32_t kSpinLimit = 1u << 21;

// The handoff counters are read and updated with inline LDS instructions
// on their LDS byte addresses.  As ordinary loads and atomics the compiler
// cannot tell them apart from the producers' direct-to-LDS loads and puts
// a vmcnt(0) wait before each of them, which would leave a producer only
// one k step of loads in flight; the kernel orders its own accesses with
// explicit waits instead (vmcnt before a producer's arrival, lgkmcnt(0)
// before a consumer's).
// The counters of one kind (ready or free) sit in 16 contiguous bytes; a
// poll reads all of them, and the wave keeps the values it saw.  The
// counters only grow, so a kept value that already meets a target is
// proof enough: a wave running behind the other role polls once per
// several k steps instead of once per step.
struct Seen {
    uint32_t v[4];
};

__device__ __forceinline__ void lds_poll(uint32_t addr, Seen& seen)
{
    u32x4 x;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(addr) : "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) seen.v[i] = __builtin_amdgcn_readfirstlane(x[i]);
}

__device__ __forceinline__ uint32_t seen_at(const Seen& seen, int s)
{
    return s == 0 ? seen.v[0] : s == 1 ? seen.v[1] : s == 2 ? seen.v[2] : seen.v[3];
}

// Bounded wait until counter s of the block at `addr` reaches `target`.
__device__ __forceinline__ bool wait_count(uint32_t addr, Seen& seen, int s, uint32_t target)
{
    if (handoff_reached(seen_at(seen, s), target)) return true;
    for (uint32_t n = 0; n < kSpinLimit; ++n) {
        lds_poll(addr, seen);
        if (handoff_reached(seen_at(seen, s), target)) return true;
        // a waiting wave sleeps between polls: it shares its SIMD's issue
        // slots with two consumer waves' MFMA stream
        __builtin_amdgcn_s_sleep(2);
    }
    return false;
}

// One arrival of this wave at the LDS handoff counter at `addr` (lane 0
// adds 1).
__device__ __forceinline__ void arrive(uint32_t addr, int lane)
{
    if (lane == 0) asm volatile("ds_add_u32 %0, %1" : : "v"(addr), "v"(1u) : "memory");
}

// Compiler fence: no memory operation moves across it (the handoff orders
// LDS reads, LDS-DMA loads and counter updates by program order and waits).
__device__ __forceinline__ void handoff_fence()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// vmcnt wait leaving the loads of `younger` later steps (LPW loads each) in flight.
template <int LPW, int STAGES>
__device__ __forceinline__ void wait_steps_in_flight(int64_t younger)
{
    static_assert(STAGES <= 4, "cases below");
    if (younger >= 3 && STAGES > 3)
        wait_vmcnt<3 * LPW>();
    else if (younger == 2 && STAGES > 2)
        wait_vmcnt<2 * LPW>();
    else if (younger == 1)
        wait_vmcnt<LPW>();
    else
        wait_vmcnt<0>();
}

template <class C>
__device__ __forceinline__ void read_substep(const char* As, const char* Bs, int wm, int wn, int lane, int kk,
                                             f16x8 (&a)[C::FM], f16x8 (&b)[C::FN])
{
    const int chunk = 2 * kk + (lane >> 5);
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
        a[i] = *reinterpret_cast<const f16x8*>(As + lds_chunk_offset<C::CH, C::SWZ>(wm + 32 * i + (lane & 31), chunk));
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
        b[j] = *reinterpret_cast<const f16x8*>(Bs + lds_chunk_offset<C::CH, C::SWZ>(wn + 32 * j + (lane & 31), chunk));
}

template <class C>
__device__ __forceinline__ void consume_stage(const char* As, const char* Bs, int wm, int wn, int lane,
                                              f32x16 (&acc)[C::FM][C::FN])
{
    if constexpr (C::DBUF) {
        // two fragment sets: sub-step kk+1 is read while kk's MFMAs run
        f16x8 a[2][C::FM], b[2][C::FN];
        read_substep<C>(As, Bs, wm, wn, lane, 0, a[0], b[0]);
#pragma unroll
        for (int kk = 0; kk < C::KSUB; ++kk) {
            if (kk + 1 < C::KSUB) read_substep<C>(As, Bs, wm, wn, lane, kk + 1, a[(kk + 1) & 1], b[(kk + 1) & 1]);
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma_32x32x16(b[kk & 1][j], a[kk & 1][i], acc[i][j]);
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < C::KSUB; ++kk) {
            f16x8 a[C::FM], b[C::FN];
            read_substep<C>(As, Bs, wm, wn, lane, kk, a, b);
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma_32x32x16(b[j], a[i], acc[i][j]);
        }
    }
}

template <class C, bool EDGE>
__global__ __launch_bounds__(C::THREADS, 1) void ws_kernel(const f16* __restrict__ A, const f16* __restrict__ B,
                                                    f16* __restrict__ D, int64_t M, int64_t N, int64_t K,
                                                    int64_t tiles_m, int64_t tiles_n)
{
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
    static_assert(C::STAGES <= 4, "the counters of one kind fit one 16-byte LDS read");
    __shared__ __attribute__((aligned(16))) uint32_t ready[4], freed[4];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t total = tiles_m * tiles_n;
    const int64_t grid = gridDim.x, wg = blockIdx.x;
    const int64_t slot = xcd_slot(wg, grid);
    const int64_t my_tiles = slot < total ? (total - slot + grid - 1) / grid : 0;
    const int64_t KT = (K + C::BK - 1) / C::BK;
    const int64_t S = my_tiles * KT;  // k steps this workgroup runs, over all its tiles
    const int64_t ldb = K * 2;
    if (t < 4) {
        ready[t] = 0;
        freed[t] = 0;
    }
    __syncthreads();   // the one workgroup barrier: the counters start at 0
    bool ok = true;    // false once a wait has run out
    const uint32_t ready0 = (uint32_t)(uintptr_t)(G16_LDS uint32_t*)ready;
    const uint32_t freed0 = (uint32_t)(uintptr_t)(G16_LDS uint32_t*)freed;
    Seen seen{{0, 0, 0, 0}};   // the counters this wave waits on, as last read

    if (wave >= C::CONSUMERS) {
        // ------------------------------------------------------ producer
        const int p = wave - C::CONSUMERS;
        uint32_t a_off[C::A_LOADS], b_off[C::B_LOADS];
        int a_row[C::A_LOADS], b_row[C::B_LOADS], a_kc[C::A_LOADS], b_kc[C::B_LOADS];
        ring::lane_offsets<C, C::A_LOADS>(p, lane, ldb, a_off, a_row, a_kc);
        ring::lane_offsets<C, C::B_LOADS>(p, lane, ldb, b_off, b_row, b_kc);
        // the tile and k step of the next refill, advanced step by step
        int64_t ti = 0, tkt = 0;
        TileCoord tc = grouped_tile(persistent_tile(wg, 0, grid), tiles_m, tiles_n);
        auto issue = [&](int64_t step) {
            const int64_t m0 = tc.m_idx * C::BM, n0 = tc.n_idx * C::BN;
            char* st = smem + (int)(step % C::STAGES) * C::STAGE_BYTES;
            const int64_t k0 = tkt * C::BK;
            ring::issue_loads<C, C::A_LOADS, EDGE>(reinterpret_cast<const char*>(A) + m0 * ldb, a_off, a_row,
                                                   a_kc, M - m0, K, k0, st, p);
            ring::issue_loads<C, C::B_LOADS, EDGE>(reinterpret_cast<const char*>(B) + n0 * ldb, b_off, b_row,
                                                   b_kc, N - n0, K, k0, st + C::A_BYTES, p);
            if (++tkt == KT) {
                tkt = 0;
                if (++ti < my_tiles) tc = grouped_tile(persistent_tile(wg, ti, grid), tiles_m, tiles_n);
            }
        };
        // iteration g first publishes step g - (STAGES - 1) (once this
        // wave's loads of it have landed; the loads of the steps after it
        // stay in flight), then refills step g (once every consumer is done
        // with step g - STAGES): a publish never waits for a release
        for (int64_t g = 0; g < S + C::STAGES - 1; ++g) {
            const int64_t j = g - (C::STAGES - 1);
            if (j >= 0) {
                wait_steps_in_flight<C::LPW, C::STAGES>((g - 1 < S - 1 ? g - 1 : S - 1) - j);
                handoff_fence();
                arrive(ready0 + 4u * (uint32_t)(j % C::STAGES), lane);
            }
            if (g < S) {
                if (ok) ok = wait_count(freed0, seen, (int)(g % C::STAGES), handoff_free_target(g, C::STAGES, C::CONSUMERS));
                handoff_fence();
                issue(g);
            }
        }
        return;
    }

    // ---------------------------------------------------------- consumer
    const int c = wave;
    const int wm = (c / C::CN) * C::WTM, wn = (c % C::CN) * C::WTN;
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
            const int s = (int)(g % C::STAGES);
            if (ok) ok = wait_count(ready0, seen, s, handoff_ready_target(g, C::STAGES, C::PRODUCERS));
            handoff_fence();
            const char* st = smem + s * C::STAGE_BYTES;
            consume_stage<C>(st, st + C::A_BYTES, wm, wn, lane, acc);
            wait_lgkmcnt0();   // this wave's reads of the stage are done
            handoff_fence();
            arrive(freed0 + 4u * (uint32_t)s, lane);
        }
        if (!ok) {
            // a wait ran out: the result is not trusted, and shows as NaN
#pragma unroll
            for (int a = 0; a < C::FM; ++a)
#pragma unroll
                for (int b = 0; b < C::FN; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[a][b][r] = __builtin_nanf("");
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
