// Device building blocks shared by every kernel of the fp16 NT GEMM ladder
// (gfx950 / CDNA4 only).
//
// Operand roles follow the problem statement of "GEMM I - the tiled
// baseline": A is M x K row-major, B is N x K row-major (both stream as
// K-contiguous row bands), D = A * B^T is M x N row-major, products
// accumulate in fp32 and D is rounded to fp16 once, at writeback.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g16 {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define G16_LDS __attribute__((address_space(3)))
#define G16_GLOBAL __attribute__((address_space(1)))

// ---------------------------------------------------------------------------
// MFMA 32x32x16 f16 -> f32.  Per lane (l = lane 0..63):
//   srcA supplies X[i = l%32][k = 8*(l/32) + 0..7]    (8 fp16, 16 bytes)
//   srcB supplies Y[k = 8*(l/32) + 0..7][j = l%32]
//   acc[r] holds  C[i = 8*(r/4) + 4*(l/32) + r%4][j = l%32]
// Both operands of this GEMM are K-contiguous rows, so a lane's fragment is
// one 16-byte read of row (l%32) at k-chunk (l/32).  The kernels feed the
// B row (an output column n) as srcA and the A row (an output row m) as
// srcB, so acc[4g .. 4g+3] are four consecutive output columns of one output
// row: D[m0 + l%32][n0 + 8g + 4*(l/32) + 0..3] -- an 8-byte store.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma_32x32x16(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Output position of accumulator group g (regs 4g..4g+3) of lane l inside a
// 32x32 block: row offset (m) and first column offset (n).
__device__ __forceinline__ int acc_row(int lane) { return lane & 31; }
__device__ __forceinline__ int acc_col(int lane, int g) { return 8 * g + 4 * (lane >> 5); }

// fp32 -> fp16 with the IEEE default rounding (nearest, ties to even):
// v_cvt_f16_f32 under the default mode register.  Overflow gives inf.
__device__ __forceinline__ f16x4 cvt4(float a, float b, float c, float d)
{
    f16x4 h;
    h[0] = (f16)a;
    h[1] = (f16)b;
    h[2] = (f16)c;
    h[3] = (f16)d;
    return h;
}

// Write one 32x32 accumulator block whose top-left output is (m0, n0).
// FULL: the block lies inside D and every row start is 8-byte aligned.
// Otherwise rows >= M and columns >= N are skipped, and 8-byte stores are
// used only where `vec` says row starts are 8-byte aligned.
// The stores are ordinary, not non-temporal: each instruction writes 16
// bytes of 32 rows, and non-temporal partial-line writes left L2 before the
// rest of their lines arrived (measured on MI355X at 4096^3: rung 5 186 ->
// 136 us and rung 3 248 -> 207 us with ordinary stores, bitwise equal).
// The staged epilogues, which write whole lines, keep non-temporal stores.
template <bool FULL>
__device__ __forceinline__ void store_block(f16* __restrict__ D, int64_t ldd, int64_t M, int64_t N,
                                            int64_t m0, int64_t n0, const f32x16& acc, int lane,
                                            bool vec = true)
{
    const int64_t m = m0 + acc_row(lane);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + acc_col(lane, g);
        f16x4 h = cvt4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
        if (FULL) {
            *reinterpret_cast<f16x4*>(D + m * ldd + n) = h;
        } else if (m < M) {
            if (vec && n + 3 < N) {
                *reinterpret_cast<f16x4*>(D + m * ldd + n) = h;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N) D[m * ldd + n + r] = h[r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// LDS tiles: a tile of R rows x BK fp16 is stored row-major with
// CH = BK/8 16-byte chunks per row; chunk c of row r sits at physical chunk
// c ^ swz(r).  A fragment read has 32 lanes read 32 consecutive rows at the
// same logical chunk; the XOR spreads the rows that the LDS serves together
// over distinct banks.  SWZ names the bank window the pattern is built for:
//   SWZ 0: no swizzle
//   SWZ 1: 128-byte window (32 banks x 4 bytes, 8 lanes of 16 bytes per
//          cycle): swz(r) = (r / rows_per_128B) mod CH
//   SWZ 2: 256-byte window (64 banks): swz(r) = (r / rows_per_256B) mod CH
// ---------------------------------------------------------------------------
template <int CH, int SWZ>
__host__ __device__ __forceinline__ int swz_of_row(int r)
{
    constexpr int ROW_BYTES = CH * 16;
    if (SWZ == 0) return 0;
    if (SWZ == 1) return (r / (128 / ROW_BYTES > 0 ? 128 / ROW_BYTES : 1)) & (CH - 1);
    return (r / (256 / ROW_BYTES)) & (CH - 1);
}

template <int CH, int SWZ>
__host__ __device__ __forceinline__ int lds_chunk_offset(int r, int c)
{
    return r * (CH * 16) + ((c ^ swz_of_row<CH, SWZ>(r)) << 4);
}

// s_waitcnt with only vmcnt limited (expcnt, lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// Workgroup barrier without the compiler's memory fence: callers order
// their own LDS reads (consumed before the barrier) and direct-to-LDS loads
// (vmcnt waits before the barrier).  sched_barrier keeps the scheduler from
// moving instructions across it.
__device__ __forceinline__ void wg_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// Direct-to-LDS 16-byte load: lane i's 16 bytes land at lds + 16*i.  The
// LDS pointer must be wave-uniform (it goes to M0).
__device__ __forceinline__ void load_lds_16(const void* gptr, void* lds)
{
    __builtin_amdgcn_global_load_lds((const G16_GLOBAL void*)gptr, (G16_LDS void*)lds, 16, 0, 0);
}

// Problem description passed to the tiled kernels by value.  Leading
// dimensions and batch strides are in elements; batch b reads
// A + b*sa, B + b*sb and writes D + b*sd.
struct GemmArgs {
    const f16* A;
    const f16* B;
    f16* D;
    int64_t M, N, K;
    int64_t lda, ldb, ldd;
    int64_t sa, sb, sd;
    int64_t batch;
    int64_t tiles_m, tiles_n;  // output tiles per batch entry
    // split-K mode (k_chunk > 0): batch entry b is K slice
    // [b*k_chunk, min(K, (b+1)*k_chunk)) of one product, whose fp32 partial
    // sums go to P + b*M*N (row pitch N); A, B and D are not offset by b
    int64_t k_chunk;
    float* P;
};

// Buffer resource over a byte range (raw buffer, 32-bit data format so the
// descriptor is valid for untyped loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct-to-LDS 16-byte buffer load: lane i reads base + voff + soff and
// its 16 bytes land at lds + 16*i (lds wave-uniform, goes to M0).
__device__ __forceinline__ void buffer_load_lds_16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                                   uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (G16_LDS void*)lds, 16, (int)voff, (int)soff, 0, 0);
}

// Scheduling-group masks for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmem = 0x010;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedDsWrite = 0x200;

}  // namespace g16
