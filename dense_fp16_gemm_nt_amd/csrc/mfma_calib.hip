// Matrix-core calibration kernel: each wave issues nothing but
// v_mfma_f32_16x16x32_f16 on random fp16 operands held in registers (the
// GEMM's instruction, with each 16 x 16 accumulator's two k-halves back to
// back as the four-wave rings issue them), so its matrix cores are busy for
// the whole loop.  Run under rocprofv3 with the SQ_VALU_MFMA_BUSY_CYCLES
// counter, it checks the busy-fraction normalisation that the GEMM profiles
// use -- counter cycles per SIMD over (shader clock x kernel duration) --
// against a kernel whose true busy fraction is known to be ~1.  Each wave
// records its shader-cycle (s_memtime) and 100 MHz reference (s_memrealtime)
// counts around the loop, from which the clock follows.  Measurement code,
// not part of the GEMM library.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kBlocksMax = 1024;

// 128 MFMAs (16 accumulators x 2 k-halves, four times) per loop trip: 2048
// matrix-core cycles per wave, against three scalar instructions of loop
// control.
__global__ __launch_bounds__(64 * kWaves, 1) void mfma_calib_kernel(const f16x8* __restrict__ rnd,
                                                                      uint64_t* __restrict__ out, int iters)
{
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int wave = blockIdx.x * kWaves + w;
    // 16 fragments of 8 fp16 per lane from this wave's 16 KiB of the buffer
    const f16x8* src = rnd + (size_t)wave * 16 * 64;
    f16x8 a[8], b[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        a[r] = src[r * 64 + lane];
        b[r] = src[(8 + r) * 64 + lane];
    }
    f32x4 c[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) c[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint64_t t0, t1, r0, r1;
    int it = iters;
    asm volatile(
        "s_waitcnt vmcnt(0) lgkmcnt(0)\n"
        "s_memtime %[t0]\n"
        "s_memrealtime %[r0]\n"
        "s_waitcnt lgkmcnt(0)\n"
        "1:\n"
        "v_mfma_f32_16x16x32_f16 %[c0], %[b00], %[a00], %[c0]\n"
        "v_mfma_f32_16x16x32_f16 %[c0], %[b01], %[a01], %[c0]\n"
        "v_mfma_f32_16x16x32_f16 %[c1], %[b10], %[a00], %[c1]\n"
        "v_mfma_f32_16x16x32_f16 %[c1], %[b11], %[a01], %[c1]\n"
        "v_mfma_f32_16x16x32_f16 %[c2], %[b20], %[a00], %[c2]\n"
        "v_mfma_f32_16x16x32_f16 %[c2], %[b21], %[a01], %[c2]\n"
        "v_mfma_f32_16x16x32_f16 %[c3], %[b30], %[a00], %[c3]\n"
        "v_mfma_f32_16x16x32_f16 %[c3], %[b31], %[a01], %[c3]\n"
        "v_mfma_f32_16x16x32_f16 %[c4], %[b00], %[a10], %[c4]\n"
        "v_mfma_f32_16x16x32_f16 %[c4], %[b01], %[a11], %[c4]\n"
        "v_mfma_f32_16x16x32_f16 %[c5], %[b10], %[a10], %[c5]\n"
        "v_mfma_f32_16x16x32_f16 %[c5], %[b11], %[a11], %[c5]\n"
        "v_mfma_f32_16x16x32_f16 %[c6], %[b20], %[a10], %[c6]\n"
        "v_mfma_f32_16x16x32_f16 %[c6], %[b21], %[a11], %[c6]\n"
        "v_mfma_f32_16x16x32_f16 %[c7], %[b30], %[a10], %[c7]\n"
        "v_mfma_f32_16x16x32_f16 %[c7], %[b31], %[a11], %[c7]\n"
        "v_mfma_f32_16x16x32_f16 %[c8], %[b00], %[a20], %[c8]\n"
        "v_mfma_f32_16x16x32_f16 %[c8], %[b01], %[a21], %[c8]\n"
        "v_mfma_f32_16x16x32_f16 %[c9], %[b10], %[a20], %[c9]\n"
        "v_mfma_f32_16x16x32_f16 %[c9], %[b11], %[a21], %[c9]\n"
        "v_mfma_f32_16x16x32_f16 %[c10], %[b20], %[a20], %[c10]\n"
        "v_mfma_f32_16x16x32_f16 %[c10], %[b21], %[a21], %[c10]\n"
        "v_mfma_f32_16x16x32_f16 %[c11], %[b30], %[a20], %[c11]\n"
        "v_mfma_f32_16x16x32_f16 %[c11], %[b31], %[a21], %[c11]\n"
        "v_mfma_f32_16x16x32_f16 %[c12], %[b00], %[a30], %[c12]\n"
        "v_mfma_f32_16x16x32_f16 %[c12], %[b01], %[a31], %[c12]\n"
        "v_mfma_f32_16x16x32_f16 %[c13], %[b10], %[a30], %[c13]\n"
        "v_mfma_f32_16x16x32_f16 %[c13], %[b11], %[a31], %[c13]\n"
        "v_mfma_f32_16x16x32_f16 %[c14], %[b20], %[a30], %[c14]\n"
        "v_mfma_f32_16x16x32_f16 %[c14], %[b21], %[a31], %[c14]\n"
        "v_mfma_f32_16x16x32_f16 %[c15], %[b30], %[a30], %[c15]\n"
        "v_mfma_f32_16x16x32_f16 %[c15], %[b31], %[a31], %[c15]\n"
        "v_mfma_f32_16x16x32_f16 %[c0], %[b00], %[a00], %[c0]\n"
        "v_mfma_f32_16x16x32_f16 %[c0], %[b01], %[a01], %[c0]\n"
        "v_mfma_f32_16x16x32_f16 %[c1], %[b10], %[a00], %[c1]\n"
        "v_mfma_f32_16x16x32_f16 %[c1], %[b11], %[a01], %[c1]\n"
        "v_mfma_f32_16x16x32_f16 %[c2], %[b20], %[a00], %[c2]\n"
        "v_mfma_f32_16x16x32_f16 %[c2], %[b21], %[a01], %[c2]\n"
        "v_mfma_f32_16x16x32_f16 %[c3], %[b30], %[a00], %[c3]\n"
        "v_mfma_f32_16x16x32_f16 %[c3], %[b31], %[a01], %[c3]\n"
        "v_mfma_f32_16x16x32_f16 %[c4], %[b00], %[a10], %[c4]\n"
        "v_mfma_f32_16x16x32_f16 %[c4], %[b01], %[a11], %[c4]\n"
        "v_mfma_f32_16x16x32_f16 %[c5], %[b10], %[a10], %[c5]\n"
        "v_mfma_f32_16x16x32_f16 %[c5], %[b11], %[a11], %[c5]\n"
        "v_mfma_f32_16x16x32_f16 %[c6], %[b20], %[a10], %[c6]\n"
        "v_mfma_f32_16x16x32_f16 %[c6], %[b21], %[a11], %[c6]\n"
        "v_mfma_f32_16x16x32_f16 %[c7], %[b30], %[a10], %[c7]\n"
        "v_mfma_f32_16x16x32_f16 %[c7], %[b31], %[a11], %[c7]\n"
        "v_mfma_f32_16x16x32_f16 %[c8], %[b00], %[a20], %[c8]\n"
        "v_mfma_f32_16x16x32_f16 %[c8], %[b01], %[a21], %[c8]\n"
        "v_mfma_f32_16x16x32_f16 %[c9], %[b10], %[a20], %[c9]\n"
        "v_mfma_f32_16x16x32_f16 %[c9], %[b11], %[a21], %[c9]\n"
        "v_mfma_f32_16x16x32_f16 %[c10], %[b20], %[a20], %[c10]\n"
        "v_mfma_f32_16x16x32_f16 %[c10], %[b21], %[a21], %[c10]\n"
        "v_mfma_f32_16x16x32_f16 %[c11], %[b30], %[a20], %[c11]\n"
        "v_mfma_f32_16x16x32_f16 %[c11], %[b31], %[a21], %[c11]\n"
        "v_mfma_f32_16x16x32_f16 %[c12], %[b00], %[a30], %[c12]\n"
        "v_mfma_f32_16x16x32_f16 %[c12], %[b01], %[a31], %[c12]\n"
        "v_mfma_f32_16x16x32_f16 %[c13], %[b10], %[a30], %[c13]\n"
        "v_mfma_f32_16x16x32_f16 %[c13], %[b11], %[a31], %[c13]\n"
        "v_mfma_f32_16x16x32_f16 %[c14], %[b20], %[a30], %[c14]\n"
        "v_mfma_f32_16x16x32_f16 %[c14], %[b21], %[a31], %[c14]\n"
        "v_mfma_f32_16x16x32_f16 %[c15], %[b30], %[a30], %[c15]\n"
        "v_mfma_f32_16x16x32_f16 %[c15], %[b31], %[a31], %[c15]\n"
        "v_mfma_f32_16x16x32_f16 %[c0], %[b00], %[a00], %[c0]\n"
        "v_mfma_f32_16x16x32_f16 %[c0], %[b01], %[a01], %[c0]\n"
        "v_mfma_f32_16x16x32_f16 %[c1], %[b10], %[a00], %[c1]\n"
        "v_mfma_f32_16x16x32_f16 %[c1], %[b11], %[a01], %[c1]\n"
        "v_mfma_f32_16x16x32_f16 %[c2], %[b20], %[a00], %[c2]\n"
        "v_mfma_f32_16x16x32_f16 %[c2], %[b21], %[a01], %[c2]\n"
        "v_mfma_f32_16x16x32_f16 %[c3], %[b30], %[a00], %[c3]\n"
        "v_mfma_f32_16x16x32_f16 %[c3], %[b31], %[a01], %[c3]\n"
        "v_mfma_f32_16x16x32_f16 %[c4], %[b00], %[a10], %[c4]\n"
        "v_mfma_f32_16x16x32_f16 %[c4], %[b01], %[a11], %[c4]\n"
        "v_mfma_f32_16x16x32_f16 %[c5], %[b10], %[a10], %[c5]\n"
        "v_mfma_f32_16x16x32_f16 %[c5], %[b11], %[a11], %[c5]\n"
        "v_mfma_f32_16x16x32_f16 %[c6], %[b20], %[a10], %[c6]\n"
        "v_mfma_f32_16x16x32_f16 %[c6], %[b21], %[a11], %[c6]\n"
        "v_mfma_f32_16x16x32_f16 %[c7], %[b30], %[a10], %[c7]\n"
        "v_mfma_f32_16x16x32_f16 %[c7], %[b31], %[a11], %[c7]\n"
        "v_mfma_f32_16x16x32_f16 %[c8], %[b00], %[a20], %[c8]\n"
        "v_mfma_f32_16x16x32_f16 %[c8], %[b01], %[a21], %[c8]\n"
        "v_mfma_f32_16x16x32_f16 %[c9], %[b10], %[a20], %[c9]\n"
        "v_mfma_f32_16x16x32_f16 %[c9], %[b11], %[a21], %[c9]\n"
        "v_mfma_f32_16x16x32_f16 %[c10], %[b20], %[a20], %[c10]\n"
        "v_mfma_f32_16x16x32_f16 %[c10], %[b21], %[a21], %[c10]\n"
        "v_mfma_f32_16x16x32_f16 %[c11], %[b30], %[a20], %[c11]\n"
        "v_mfma_f32_16x16x32_f16 %[c11], %[b31], %[a21], %[c11]\n"
        "v_mfma_f32_16x16x32_f16 %[c12], %[b00], %[a30], %[c12]\n"
        "v_mfma_f32_16x16x32_f16 %[c12], %[b01], %[a31], %[c12]\n"
        "v_mfma_f32_16x16x32_f16 %[c13], %[b10], %[a30], %[c13]\n"
        "v_mfma_f32_16x16x32_f16 %[c13], %[b11], %[a31], %[c13]\n"
        "v_mfma_f32_16x16x32_f16 %[c14], %[b20], %[a30], %[c14]\n"
        "v_mfma_f32_16x16x32_f16 %[c14], %[b21], %[a31], %[c14]\n"
        "v_mfma_f32_16x16x32_f16 %[c15], %[b30], %[a30], %[c15]\n"
        "v_mfma_f32_16x16x32_f16 %[c15], %[b31], %[a31], %[c15]\n"
        "v_mfma_f32_16x16x32_f16 %[c0], %[b00], %[a00], %[c0]\n"
        "v_mfma_f32_16x16x32_f16 %[c0], %[b01], %[a01], %[c0]\n"
        "v_mfma_f32_16x16x32_f16 %[c1], %[b10], %[a00], %[c1]\n"
        "v_mfma_f32_16x16x32_f16 %[c1], %[b11], %[a01], %[c1]\n"
        "v_mfma_f32_16x16x32_f16 %[c2], %[b20], %[a00], %[c2]\n"
        "v_mfma_f32_16x16x32_f16 %[c2], %[b21], %[a01], %[c2]\n"
        "v_mfma_f32_16x16x32_f16 %[c3], %[b30], %[a00], %[c3]\n"
        "v_mfma_f32_16x16x32_f16 %[c3], %[b31], %[a01], %[c3]\n"
        "v_mfma_f32_16x16x32_f16 %[c4], %[b00], %[a10], %[c4]\n"
        "v_mfma_f32_16x16x32_f16 %[c4], %[b01], %[a11], %[c4]\n"
        "v_mfma_f32_16x16x32_f16 %[c5], %[b10], %[a10], %[c5]\n"
        "v_mfma_f32_16x16x32_f16 %[c5], %[b11], %[a11], %[c5]\n"
        "v_mfma_f32_16x16x32_f16 %[c6], %[b20], %[a10], %[c6]\n"
        "v_mfma_f32_16x16x32_f16 %[c6], %[b21], %[a11], %[c6]\n"
        "v_mfma_f32_16x16x32_f16 %[c7], %[b30], %[a10], %[c7]\n"
        "v_mfma_f32_16x16x32_f16 %[c7], %[b31], %[a11], %[c7]\n"
        "v_mfma_f32_16x16x32_f16 %[c8], %[b00], %[a20], %[c8]\n"
        "v_mfma_f32_16x16x32_f16 %[c8], %[b01], %[a21], %[c8]\n"
        "v_mfma_f32_16x16x32_f16 %[c9], %[b10], %[a20], %[c9]\n"
        "v_mfma_f32_16x16x32_f16 %[c9], %[b11], %[a21], %[c9]\n"
        "v_mfma_f32_16x16x32_f16 %[c10], %[b20], %[a20], %[c10]\n"
        "v_mfma_f32_16x16x32_f16 %[c10], %[b21], %[a21], %[c10]\n"
        "v_mfma_f32_16x16x32_f16 %[c11], %[b30], %[a20], %[c11]\n"
        "v_mfma_f32_16x16x32_f16 %[c11], %[b31], %[a21], %[c11]\n"
        "v_mfma_f32_16x16x32_f16 %[c12], %[b00], %[a30], %[c12]\n"
        "v_mfma_f32_16x16x32_f16 %[c12], %[b01], %[a31], %[c12]\n"
        "v_mfma_f32_16x16x32_f16 %[c13], %[b10], %[a30], %[c13]\n"
        "v_mfma_f32_16x16x32_f16 %[c13], %[b11], %[a31], %[c13]\n"
        "v_mfma_f32_16x16x32_f16 %[c14], %[b20], %[a30], %[c14]\n"
        "v_mfma_f32_16x16x32_f16 %[c14], %[b21], %[a31], %[c14]\n"
        "v_mfma_f32_16x16x32_f16 %[c15], %[b30], %[a30], %[c15]\n"
        "v_mfma_f32_16x16x32_f16 %[c15], %[b31], %[a31], %[c15]\n"
        "s_sub_u32 %[it], %[it], 1\n"
        "s_cmp_eq_u32 %[it], 0\n"
        "s_cbranch_scc0 1b\n"
        "s_nop 7\n"
        "s_nop 7\n"
        "s_memtime %[t1]\n"
        "s_memrealtime %[r1]\n"
        "s_waitcnt lgkmcnt(0)\n"
        : [t0] "=&s"(t0), [t1] "=&s"(t1), [r0] "=&s"(r0), [r1] "=&s"(r1), [it] "+s"(it),
          [c0] "+a"(c[0]), [c1] "+a"(c[1]), [c2] "+a"(c[2]), [c3] "+a"(c[3]), [c4] "+a"(c[4]), [c5] "+a"(c[5]), [c6] "+a"(c[6]), [c7] "+a"(c[7]), [c8] "+a"(c[8]), [c9] "+a"(c[9]), [c10] "+a"(c[10]), [c11] "+a"(c[11]), [c12] "+a"(c[12]), [c13] "+a"(c[13]), [c14] "+a"(c[14]), [c15] "+a"(c[15])
        : [a00] "v"(a[0]), [a01] "v"(a[1]), [a10] "v"(a[2]), [a11] "v"(a[3]), [a20] "v"(a[4]), [a21] "v"(a[5]), [a30] "v"(a[6]), [a31] "v"(a[7]), [b00] "v"(b[0]), [b01] "v"(b[1]), [b10] "v"(b[2]), [b11] "v"(b[3]), [b20] "v"(b[4]), [b21] "v"(b[5]), [b30] "v"(b[6]), [b31] "v"(b[7])
        : "memory", "scc");
    // one lane per wave stores the stamps and a checksum of its accumulators
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += c[r][0] + c[r][1] + c[r][2] + c[r][3];
    if (lane == 0) {
        out[3 * wave] = t1 - t0;
        out[3 * wave + 1] = r1 - r0;
        out[3 * wave + 2] = (uint64_t)__float_as_uint(sum);
    }
}

// blocks: workgroups of 4 waves (one per SIMD); rnd: device buffer of at
// least blocks * 64 KiB of fp16; out: device buffer of 3 * 4 * blocks
// uint64 (per wave: shader cycles, 100 MHz ticks, checksum bits); iters:
// loop trips.  Returns 0, -1 for a bad argument, -3 if the launch failed.
extern "C" int mfma_calib_launch(int blocks, const void* rnd, uint64_t* out, int iters, void* stream)
{
    if (blocks < 1 || blocks > kBlocksMax || iters < 1 || rnd == nullptr || out == nullptr) return -1;
    hipLaunchKernelGGL(mfma_calib_kernel, dim3(blocks), dim3(64 * kWaves), 0, (hipStream_t)stream,
                       (const f16x8*)rnd, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
