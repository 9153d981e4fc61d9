// Rung 4: pipelined LDS ring fed by direct-to-LDS loads.
//
// The pages' steps 4-5 replace the threads' copy with an asynchronous copy
// engine and then multi-buffer the operand tiles so the next K tile streams
// in while the current one is multiplied ("TIRx GEMM detailed technical
// notes", V4 "TMA Async Load and Store" and V5 "Software Pipeline with
// Double-Buffered SMEM").  On gfx950 the copy engine is the direct-to-LDS
// form of the buffer load (buffer_load_dwordx4 ... lds): each lane names a
// 16-byte global source and the data lands in LDS without passing through
// registers; completion is the issuing wave's vmcnt.
//
// Workgroup tile BM x BN (256 x 256), BK-wide k steps, a STAGES-deep ring
// in LDS, WAVES_M x WAVES_N waves each owning a (BM/WAVES_M) x (BN/WAVES_N)
// accumulator in registers.  Every wave issues its share of the loads and
// multiplies; one workgroup barrier per k step both publishes step k+1 and
// releases the stage of step k.  Schedule of one k step j:
//  * sub-steps 0 .. KSUB-2: the fragments of sub-step kk+1 are read from LDS
//    while the MFMAs of sub-step kk run (two register buffers), and during
//    the first LSPLIT sub-steps this wave's loads of step j + STAGES - 1 go
//    out one per MFMA (into the stage the barrier of step j-1 released);
//  * last sub-step: wait until this wave's LDS reads of step j are complete
//    and its loads of step j+1 have landed, issue PRE MFMAs so the matrix
//    core stays busy, cross the barrier, read the first fragments of step
//    j+1, finish the MFMAs of step j.
// The loop body has no branch on the accumulators (the last step is peeled)
// so they stay in place across iterations.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "sched.hpp"

namespace g16 {

// 16 zero bytes: the source of every out-of-range lane of an edge tile.
__device__ __attribute__((aligned(64))) uint32_t g_zero_line[16] = {0};

// 16 bytes (8 fp16) of an operand row from element kk on, for rows that
// start on any 2-byte boundary (K, leading dimensions or bases not
// multiples of 8 elements).  The load goes through registers: gfx950's
// global loads take unaligned addresses, its direct-to-LDS loads are only
// used here on 16-byte aligned rows.  Nothing past the row's K-th element
// is touched: a chunk that crosses K is read as the row's last 8 elements,
// which chunk_shift then moves into place; a chunk at or beyond K, or of a
// row past the operand, reads the zero line.  Needs K >= 8.
__device__ __forceinline__ u32x4 load_row_chunk(const char* row_ptr, int kk, int K, bool row_ok)
{
    typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
    const int avail = K - kk;
    const char* p = !(row_ok && avail > 0) ? (const char*)g_zero_line
                                           : row_ptr + 2 * (uint32_t)(avail >= 8 ? kk : K - 8);
    return *(const G16_GLOBAL u32x4_a2*)p;
}

// The chunk load_row_chunk returned for element kk, with elements at or
// beyond K set to zero: a chunk that crosses K holds the row's last 8
// elements, of which the last K - kk are this chunk's first ones.
__device__ __forceinline__ u32x4 chunk_shift(u32x4 v, int kk, int K)
{
    const int avail = K - kk;
    const int sh = (avail > 0 && avail < 8) ? (int)(8 - avail) : 0;
    unsigned __int128 x = __builtin_bit_cast(unsigned __int128, v);
    x >>= 16 * sh;
    return __builtin_bit_cast(u32x4, x);
}

namespace ring {

template <int BM_, int BN_, int BK_, int STAGES_, int SWZ_, int WM_ = 2, int WN_ = 2>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, SWZ = SWZ_;
    static constexpr int WAVES_M = WM_, WAVES_N = WN_;     // wave grid over the tile
    static constexpr int WAVES = WM_ * WN_, THREADS = 64 * WAVES;
    static constexpr int CH = BK / 8;                 // 16-byte chunks per LDS row
    static constexpr int ROW_BYTES = BK * 2;
    static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;  // one wave load = 1 KiB
    static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int A_LOADS = A_BYTES / 1024 / WAVES;  // per wave per step
    static constexpr int B_LOADS = B_BYTES / 1024 / WAVES;
    static constexpr int LPW = A_LOADS + B_LOADS;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wave tile
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

// Fragment registers of one 16-wide k sub-step: FM A rows-blocks and FN
// B row-blocks, one 16-byte LDS read each.
template <class C>
__device__ __forceinline__ void read_frags(const char* st, int wm, int wn, int lane, int kk,
                                           f16x8 (&a)[C::FM], f16x8 (&b)[C::FN])
{
    const int chunk = 2 * kk + (lane >> 5);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) a[i] = frag<C>(st, wm + 32 * i + (lane & 31), chunk);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) b[j] = frag<C>(st + C::A_BYTES, wn + 32 * j + (lane & 31), chunk);
}

// MFMAs [first, last) of one sub-step, in (i, j) row-major order.
template <class C, int FIRST, int LAST>
__device__ __forceinline__ void mfma_range(const f16x8 (&a)[C::FM], const f16x8 (&b)[C::FN],
                                           f32x16 (&acc)[C::FM][C::FN])
{
#pragma unroll
    for (int q = FIRST; q < LAST; ++q) {
        const int i = q / C::FN, j = q % C::FN;
        acc[i][j] = mfma_32x32x16(b[j], a[i], acc[i][j]);
    }
}

// Interleave hint for one sub-step: NQ MFMAs, each followed by up to one
// vector-memory load while any remain; the nr LDS reads either go one per
// MFMA (READS_FIRST false) or all ahead of the MFMAs (true), which gives the
// last read a whole sub-step of MFMAs to land in.
// (nr, nl are compile-time constants once the callers' loops are unrolled.)
template <int NQ, bool READS_FIRST = false>
__device__ __forceinline__ void interleave_hint(int nr, int nl)
{
    if (READS_FIRST) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            if (q < nr) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (!READS_FIRST && q < nr) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        if (q < nl) __builtin_amdgcn_sched_group_barrier(kSchedVmem, 1, 0);
    }
}

// Epilogue: round a wave's (FM*32) x (FN*32) accumulator tile to fp16, stage
// it in LDS and write it to D with 16-byte stores that cover whole 128-byte
// lines (the registers hold 4 consecutive columns per lane, which would
// otherwise mean partial-line 8-byte stores).  Row r of the staged tile is FN*64 bytes;
// 16-byte chunk c of row r sits at chunk c ^ (r mod CPR).
// EDGE: rows >= M and columns >= N are not written; a 16-byte chunk off a
// 16-byte boundary of D is stored unaligned (gfx950's global stores take
// any address), and the chunk that crosses N element by element.
template <class C, bool EDGE = false>
__device__ __forceinline__ void epilogue_lds(char* lds, f16* __restrict__ D, int64_t ldd, int64_t row0,
                                             int64_t col0, const f32x16 (&acc)[C::FM][C::FN], int lane,
                                             int64_t M = 0, int64_t N = 0)
{
    constexpr int ROWB = C::FN * 64;      // bytes per staged row
    constexpr int CPR = ROWB / 16;        // chunks per row
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int r = 32 * i + (lane & 31);
                const int c = 4 * j + g;
                const int off = r * ROWB + ((c ^ (r % CPR)) << 4) + ((lane >> 5) << 3);
                *reinterpret_cast<f16x4*>(lds + off) =
                    cvt4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
            }
    wait_lgkmcnt0();
    constexpr int ROWS_PER_STORE = 64 / CPR;
#pragma unroll
    for (int q = 0; q < C::FM * 32 / ROWS_PER_STORE; ++q) {
        const int r = q * ROWS_PER_STORE + lane / CPR;
        const int c = lane % CPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * ROWB + ((c ^ (r % CPR)) << 4));
        f16* dst = D + (row0 + r) * ldd + col0 + 8 * c;
        if (EDGE) {
            typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
            const int64_t col = col0 + 8 * c;
            if (row0 + r >= M || col >= N) continue;
            if (col + 8 > N) {
                const f16x8 h = __builtin_bit_cast(f16x8, v);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (col + e < N) dst[e] = h[e];
                continue;
            }
            if ((uintptr_t)dst & 15) {
                *reinterpret_cast<u32x4_a2*>(dst) = v;
                continue;
            }
        }
        // non-temporal: D is not read again by the kernel
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
    }
}

// Write one 32x32 accumulator block as fp32 partial sums (16-byte stores of
// four consecutive columns; element stores where vec is false or at edges).
__device__ __forceinline__ void store_block_f32(float* __restrict__ P, int64_t ldp, int64_t M, int64_t N,
                                                int64_t m0, int64_t n0, const f32x16& acc, int lane, bool vec)
{
    const int64_t m = m0 + acc_row(lane);
    if (m >= M) return;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
        const int64_t n = n0 + acc_col(lane, g4);
        if (vec && n + 3 < N) {
            *reinterpret_cast<f32x4*>(P + m * ldp + n) =
                f32x4{acc[4 * g4], acc[4 * g4 + 1], acc[4 * g4 + 2], acc[4 * g4 + 3]};
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < N) P[m * ldp + n + r] = acc[4 * g4 + r];
        }
    }
}

// VSTAGE: operands on any 2-byte boundary (EDGE form only, K >= 8).  Each
// wave's loads of step j + STAGES - 1 go to registers during step j
// (load_row_chunk) and are written to their LDS slots just before the
// barrier that ends step j; the slots are the ones the direct-to-LDS form
// fills, so the fragment reads are the same.
template <class C, bool EDGE, int PRE, int LSPLIT, bool EPI_LDS, bool READS_FIRST = false, bool SPLITK = false,
          bool VSTAGE = false>
__global__ __launch_bounds__(C::THREADS, 1) void ring_kernel(const GemmArgs g)
{
    static_assert(LSPLIT >= 1 && LSPLIT < C::KSUB && C::LPW % LSPLIT == 0, "load split");
    static_assert(!VSTAGE || (EDGE && !SPLITK), "register staging is an edge form");
    static_assert(!EPI_LDS || C::WAVES * C::FM * 32 * C::FN * 64 <= C::LDS_BYTES, "epilogue staging");
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);

    // workgroup -> (batch entry, tile): the XCD remap and grouped order run
    // over all batch entries' tiles, batch-major
    const int64_t per_batch = g.tiles_m * g.tiles_n;
    const int64_t slot = xcd_slot(blockIdx.x, per_batch * g.batch);
    const int64_t bidx = slot / per_batch;
    const TileCoord tc = grouped_tile(slot - bidx * per_batch, g.tiles_m, g.tiles_n);
    const int64_t m0 = tc.m_idx * C::BM, n0 = tc.n_idx * C::BN;
    const int64_t M = g.M, N = g.N, ldd = g.ldd;
    // split-K: this workgroup contracts K slice bidx of the one product
    const int64_t k_begin = SPLITK ? bidx * g.k_chunk : 0;
    const int64_t K = SPLITK ? (g.K - k_begin < g.k_chunk ? g.K - k_begin : g.k_chunk) : g.K;
    f16* __restrict__ D = g.D + (SPLITK ? 0 : bidx * g.sd);

    const int64_t lda_b = g.lda * 2, ldb_b = g.ldb * 2;
    const char* a_base = reinterpret_cast<const char*>(g.A + (SPLITK ? k_begin : bidx * g.sa)) + m0 * lda_b;
    const char* b_base = reinterpret_cast<const char*>(g.B + (SPLITK ? k_begin : bidx * g.sb)) + n0 * ldb_b;
    uint32_t a_off[C::A_LOADS], b_off[C::B_LOADS];
    int a_row[C::A_LOADS], b_row[C::B_LOADS], a_kc[C::A_LOADS], b_kc[C::B_LOADS];
    lane_offsets<C, C::A_LOADS>(w, lane, lda_b, a_off, a_row, a_kc);
    lane_offsets<C, C::B_LOADS>(w, lane, ldb_b, b_off, b_row, b_kc);
    const int64_t a_rows = M - m0, b_rows = N - n0;
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(a_base, (uint32_t)(C::BM * lda_b));
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(b_base, (uint32_t)(C::BN * ldb_b));

    // VSTAGE: one step's loads of this wave, held until written to LDS
    u32x4 stg[C::LPW];

    // load q (0 .. LPW-1) of this wave for k step `step`
    auto load_one = [&](int64_t step, int q) {
        char* st = smem + (int)(step % C::STAGES) * C::STAGE_BYTES;
        const int64_t k0 = step * C::BK;
        if (VSTAGE) {
            const int qb = q - C::A_LOADS;
            // (K <= 2^22: the element indices fit 32 bits)
            stg[q] = q < C::A_LOADS ? load_row_chunk(a_base + (a_off[q] - 2 * a_kc[q]), (int)k0 + a_kc[q], (int)K,
                                                     a_row[q] < a_rows)
                                    : load_row_chunk(b_base + (b_off[qb] - 2 * b_kc[qb]), (int)k0 + b_kc[qb], (int)K,
                                                     b_row[qb] < b_rows);
            return;
        }
        if (q < C::A_LOADS) {
            char* d = st + (w * C::A_LOADS + q) * 1024;
            if (EDGE) {
                const bool ok = a_row[q] < a_rows && k0 + a_kc[q] < K;
                load_lds_16(ok ? (const void*)(a_base + k0 * 2 + a_off[q]) : (const void*)g_zero_line, d);
            } else {
                buffer_load_lds_16(a_rsrc, d, a_off[q], (uint32_t)(k0 * 2));
            }
        } else {
            const int qb = q - C::A_LOADS;
            char* d = st + C::A_BYTES + (w * C::B_LOADS + qb) * 1024;
            if (EDGE) {
                const bool ok = b_row[qb] < b_rows && k0 + b_kc[qb] < K;
                load_lds_16(ok ? (const void*)(b_base + k0 * 2 + b_off[qb]) : (const void*)g_zero_line, d);
            } else {
                buffer_load_lds_16(b_rsrc, d, b_off[qb], (uint32_t)(k0 * 2));
            }
        }
    };

    // VSTAGE: the staged loads of step `step` into the slots the
    // direct-to-LDS loads would fill (lane i of a load at 16*i)
    // (the shift of a chunk that crosses K happens here, after the loads
    // have landed, so that no wait for them falls inside the step; only the
    // last step, a wave-uniform test, can hold such a chunk)
    auto stage_write = [&](int64_t step) {
        char* st = smem + (int)(step % C::STAGES) * C::STAGE_BYTES;
        const int k0 = (int)(step * C::BK);
        __builtin_amdgcn_sched_barrier(0);
        if (k0 + C::BK > K) {
#pragma unroll
            for (int q = 0; q < C::LPW; ++q)
                stg[q] = chunk_shift(stg[q], k0 + (q < C::A_LOADS ? a_kc[q] : b_kc[q - C::A_LOADS]), K);
        }
#pragma unroll
        for (int q = 0; q < C::LPW; ++q) {
            const int qb = q - C::A_LOADS;
            char* d = q < C::A_LOADS ? st + (w * C::A_LOADS + q) * 1024 : st + C::A_BYTES + (w * C::B_LOADS + qb) * 1024;
            *reinterpret_cast<u32x4*>(d + 16 * lane) = stg[q];
        }
    };
    // VSTAGE: the barrier also orders the LDS writes before it against
    // every wave's reads after it
    auto staged_barrier = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        wg_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    };

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16{};

    const int64_t KT = (K + C::BK - 1) / C::BK;
    // prologue: steps 0 .. STAGES-2
#pragma unroll
    for (int s = 0; s < C::STAGES - 1; ++s)
        if (s < KT) {
#pragma unroll
            for (int q = 0; q < C::LPW; ++q) load_one(s, q);
            if (VSTAGE) stage_write(s);
        }
    if (VSTAGE)
        staged_barrier();
    else {
        if (KT >= C::STAGES - 1)
            wait_vmcnt<(C::STAGES - 2) * C::LPW>();
        else
            wait_vmcnt<0>();
        wg_barrier();
    }

    const int wm = (w / C::WAVES_N) * C::WTM, wn = (w % C::WAVES_N) * C::WTN;
    constexpr int NQ = C::FM * C::FN;
    constexpr int NR = C::FM + C::FN;
    constexpr int LPS = C::LPW / LSPLIT;   // loads per loading sub-step
    constexpr int LB = (C::KSUB - 1) & 1;
    f16x8 fa[2][C::FM], fb[2][C::FN];
    read_frags<C>(smem, wm, wn, lane, 0, fa[0], fb[0]);

    // sub-steps 0 .. KSUB-2 of step j; LOADS: issue step j+STAGES-1
    auto substeps = [&](int64_t j, auto loads_tag) {
        constexpr bool LOADS = decltype(loads_tag)::value;
        const char* st = smem + (int)(j % C::STAGES) * C::STAGE_BYTES;
#pragma unroll
        for (int kk = 0; kk < C::KSUB - 1; ++kk) {
            read_frags<C>(st, wm, wn, lane, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
            if (LOADS && kk < LSPLIT) {
#pragma unroll
                for (int q = 0; q < LPS; ++q) load_one(j + C::STAGES - 1, kk * LPS + q);
            }
            mfma_range<C, 0, NQ>(fa[kk & 1], fb[kk & 1], acc);
            interleave_hint<NQ, READS_FIRST>(NR, (LOADS && kk < LSPLIT) ? LPS : 0);
        }
    };
    // last sub-step of step j with the handoff to step j+1
    auto handoff = [&](int64_t j, auto exact_tag) {
        constexpr bool EXACT = decltype(exact_tag)::value;
        wait_lgkmcnt0();
        mfma_range<C, 0, PRE>(fa[LB], fb[LB], acc);
        if (VSTAGE) {
            // EXACT steps loaded step j + STAGES - 1; its slot held step
            // j - 1, which every wave finished reading before the last barrier
            if (EXACT) stage_write(j + C::STAGES - 1);
            staged_barrier();
        } else {
            if (EXACT)
                wait_vmcnt<(C::STAGES - 2) * C::LPW>();
            else
                wait_vmcnt<0>();
            wg_barrier();
        }
        read_frags<C>(smem + (int)((j + 1) % C::STAGES) * C::STAGE_BYTES, wm, wn, lane, 0, fa[0], fb[0]);
        mfma_range<C, PRE, NQ>(fa[LB], fb[LB], acc);
        interleave_hint<NQ - PRE, READS_FIRST>(NR, 0);
    };
    using True_ = std::integral_constant<bool, true>;
    using False_ = std::integral_constant<bool, false>;

    const int64_t j_loads_end = KT - C::STAGES + 1;  // steps j < this issue loads
    int64_t j = 0;
    for (; j < j_loads_end && j + 1 < KT; ++j) {
        substeps(j, True_{});
        handoff(j, True_{});
    }
    for (; j + 1 < KT; ++j) {
        substeps(j, False_{});
        handoff(j, False_{});
    }
    substeps(KT - 1, False_{});
    mfma_range<C, 0, NQ>(fa[LB], fb[LB], acc);
    if (SPLITK) {
        float* __restrict__ P = g.P + bidx * M * N;
        const bool vec = N % 4 == 0;
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int jj = 0; jj < C::FN; ++jj)
                store_block_f32(P, N, M, N, m0 + wm + 32 * i, n0 + wn + 32 * jj, acc[i][jj], lane, vec);
    } else if (EPI_LDS) {
        wg_barrier();  // every wave is done reading the ring
        epilogue_lds<C, EDGE>(smem + w * (C::FM * 32 * C::FN * 64), D, ldd, m0 + wm, n0 + wn, acc, lane, M, N);
    } else {
        // 8-byte stores need every row start of this batch entry aligned
        const bool vec = ldd % 4 == 0 && g.sd % 4 == 0 && ((uintptr_t)g.D & 7) == 0;
        const bool full = !EDGE || (m0 + C::BM <= M && n0 + C::BN <= N && vec);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int jj = 0; jj < C::FN; ++jj) {
                const int64_t mb = m0 + wm + 32 * i, nb = n0 + wn + 32 * jj;
                if (full)
                    store_block<true>(D, ldd, M, N, mb, nb, acc[i][jj], lane);
                else
                    store_block<false>(D, ldd, M, N, mb, nb, acc[i][jj], lane, vec);
            }
    }
}

// Split-K reduction: D = fp16(sum over slices s = 0, 1, ... of P[s]), in
// slice order, rounded once (round-to-nearest-even).  Four outputs per
// thread when N % 4 == 0, else one.  The partial sums were written by other
// XCDs, so each read waits on the fabric: with more than 2 * kReduceAhead
// slices a thread loads kReduceAhead of them before adding them (in order);
// measured on MI355X, that cut 256 x 256 x 65536 (64 slices) from 45.9 to
// 35.6 us but cost 3% with 16 slices.
constexpr int kReduceAhead = 8;

template <bool VEC>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P, f16* __restrict__ D,
                                                           int64_t M, int64_t N, int64_t ldd, int64_t splits)
{
    typedef typename std::conditional<VEC, f32x4, float>::type T;
    constexpr int U = kReduceAhead;
    const int64_t MN = M * N;
    const int64_t per = VEC ? 4 : 1;
    const int64_t n_items = MN / per;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < n_items; it += stride) {
        const int64_t e = it * per, row = e / N, col = e - row * N;
        const T* p = reinterpret_cast<const T*>(P + e);
        const int64_t step = MN / per;   // one slice, in units of T
        T s = p[0];
        int64_t k = 1;
        for (; splits > 2 * U && k + U <= splits; k += U) {
            T v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = p[(k + u) * step];
#pragma unroll
            for (int u = 0; u < U; ++u) s += v[u];
        }
        for (; k < splits; ++k) s += p[k * step];
        if constexpr (VEC)
            *reinterpret_cast<f16x4*>(D + row * ldd + col) = cvt4(s[0], s[1], s[2], s[3]);
        else
            D[row * ldd + col] = (f16)s;
    }
}

}  // namespace ring
}  // namespace g16
