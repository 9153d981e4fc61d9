// C-ABI boundary of the fp16 NT GEMM library: argument validation (before
// any HIP call), device checks, rung dispatch and launch.  The contract of
// every entry point is in include/gemm_f16_nt.h.
#include "gemm_f16_nt.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <numeric>

#include "common.hpp"
#include "ladder.hpp"
#include "persistent_ws.hpp"
#include "ring.hpp"
#include "ring4.hpp"
#include "ring_wide.hpp"
#include "sched.hpp"
#include "skinny.hpp"

using namespace g16;

// Scratch memory of gemm_f16_nt_splitk_noalloc (see splitk_run below): 64
// MiB of device memory per device, held until the process ends.
constexpr int64_t kScratchBytes = int64_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

// Kernel configurations of the fast rungs (measured on MI355X; see the
// bench): rung 4 = 256 x 256 tile, 64-wide k steps, 2-stage ring, 8 waves of
// 128 x 64 (two per SIMD), loads issued in the first sub-step, 2 MFMAs ahead
// of each barrier, LDS-staged epilogue; rung 5 = 32-wide k steps, 4 stages;
// rung 8 = rung 4's ring with 4 waves of 128 x 128 on 16x16x32 MFMAs and a
// generated instruction schedule, persistent (ring4.hpp), release and
// publish barriers per step, at most one instruction between two MFMAs
// (rungs 6 and 7, earlier forms of it, were removed); rung 9
// = rung 4's ring with 128 x 128 tiles, 8 waves of 64 x 32 and 4 stages (the
// library's choice when 256 x 256 tiles would leave most compute units
// idle); rung 10 = rung 8 with each block's two sub-steps back to back (the
// library's choice when M, N >= 256).
using RingCfg = ring::Cfg<256, 256, 64, 2, 2, 2, 4>;
using RingSmallCfg = ring::Cfg<128, 128, 64, 4, 2, 2, 4>;
constexpr int kRingPre = 2, kRingLsplit = 1;
// The library's choice takes 128 x 128 tiles when 256 x 256 tiles would
// number at most this many per 10 compute units: measured on MI355X, the
// two tie at ~100 tiles of 256 x 256 on 256 CUs (2560^3), 128 x 128 is
// 1.6-2.2x faster at 16-64 tiles and 256 x 256 is 1.4x faster at 144.
constexpr int64_t kSmallTilesPer10Cus = 4;
// Rung 5's ring: two stages of 64-wide k steps (measured on MI355X against
// four stages of 32-wide steps: 188.6 against 215.0 us at 4096^3, 1221.5
// against 1391.6 us at 8192^3, bitwise equal outputs; half as many handoffs
// per FLOP, each consumer wait covering twice the MFMAs), 8 consumer and 4
// producer waves, consumers reading the next sub-step's fragments while
// the current one's MFMAs run (1% faster at 4096^3 and 8192^3).  4 consumer
// and 4 producer waves on 256 x 128 tiles (256 registers each, 3 stages)
// were 15-18% slower: the smaller tile moves 1.5x the operand bytes per
// FLOP and one consumer per SIMD leaves its MFMA pipe idle during waits.
using WsCfg = ws::Cfg<64, 2, 2, 2, 4, 4, true>;
constexpr int kFastTile = 256;
// the library's choice takes the four-wave scheduled ring where it applies
constexpr bool kDefaultRing4 = true;

__global__ void fill_zero_kernel(uint16_t* __restrict__ D, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) D[i] = 0;
}

// --------------------------------------------------------------- devices
constexpr int kMaxDevices = 64;
struct DeviceInfo {
    std::atomic<int> state{0};  // 0 unknown, 1 ok, -1 unusable
    int cu_count = 0;
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_lock;

int device_info(int* cu_count)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GEMM_F16_NT_DEVICE;
    DeviceInfo& d = g_dev[dev];
    int st = d.state.load(std::memory_order_acquire);
    if (st == 0) {
        std::lock_guard<std::mutex> lock(g_dev_lock);
        st = d.state.load(std::memory_order_relaxed);
        if (st == 0) {
            hipDeviceProp_t prop;
            int cus = 0;
            st = -1;
            if (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                cus > 0) {
                d.cu_count = cus;
                st = 1;
            }
            d.state.store(st, std::memory_order_release);
        }
    }
    if (st != 1) return GEMM_F16_NT_DEVICE;
    *cu_count = d.cu_count;
    return GEMM_F16_NT_OK;
}

// ------------------------------------------------------------ validation
bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes)
{
    if (abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// Shapes the four-wave scheduled ring implements: M, N >= 256 (the last
// tile row and column are moved back to end at M and N, so every tile is
// whole), N a multiple of 8 (16-byte stores of the moved column), and at
// least two whole 64-wide k steps (M = 0 or N = 0 is a no-op everywhere).
bool ring4_shape(int64_t M, int64_t N, int64_t K)
{
    return M >= ring4::C::BM && N >= ring4::C::BN && N % 8 == 0 && K % ring4::C::BK == 0 &&
           K >= 2 * ring4::C::BK;
}

// The fourth form (rung 10, the library's choice) also takes K that is not
// a multiple of 64, as long as it is a multiple of 8 above 64: its first
// step is the partial one, whose chunks before a row's first element are
// moved out of range by a mask that needs every operand band of 256 rows
// under 2^30 bytes (lda, ldb < 2^21).  It also takes any N >= 256: its
// 16-byte output stores go to any 2-byte boundary (gfx950's buffer stores
// take unaligned addresses), where the other forms keep N % 8 == 0.
bool ring4_paired_shape(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb)
{
    if (M < ring4::C::BM || N < ring4::C::BN || K % 8 != 0 || K <= ring4::C::BK) return false;
    return K % ring4::C::BK == 0 || (lda < (int64_t(1) << 21) && ldb < (int64_t(1) << 21));
}

// The four-wave ring's output buffer resource spans the 128 rows of a
// wave's block, 256 * ldd bytes in a 32-bit size: the output row pitch
// must stay under 2^24 elements (above, the size would wrap and the
// hardware's range check would drop stores).
bool ring4_pitch_ok(int64_t ldd) { return ldd < (int64_t(1) << 24); }

// Operands the 16-byte-load kernels take: every row of A and B starts on a
// 16-byte boundary (K, leading dimensions and batch strides multiples of 8
// elements, 16-byte aligned bases) and D's base is 16-byte aligned.  Other
// operands go to the general kernel (ladder::r3_any).
bool fast_operands(int64_t K, int64_t lda, int64_t ldb, int64_t sa, int64_t sb, const void* A, const void* B,
                   const void* D)
{
    if (K % 8 || lda % 8 || ldb % 8 || sa % 8 || sb % 8) return false;
    if (K > 0 && ((((uintptr_t)A) | ((uintptr_t)B)) & 15)) return false;
    return ((uintptr_t)D & 15) == 0;
}

// Rung numbers the library implements (6 and 7 are no longer used).
bool known_rung(int rung)
{
    return rung >= 0 && rung <= GEMM_F16_NT_R13_KSPLIT && rung != 6 && rung != 7;
}

// Shapes of rung 12: one side of at most 96 rows, K >= 8 (the chunk that
// crosses K is read as a row's last 8 elements), rows on any 2-byte boundary.
bool skinny_shape(int64_t M, int64_t N, int64_t K)
{
    return (M <= skinny::kMaxSmall || N <= skinny::kMaxSmall) && K >= 8;
}

// Where the library's choice takes rung 12: a single product whose small
// side has at most 32 rows, at most 64 with a large side of at most 16384
// rows, or at most 96 with a large side of at most 12288.  Measured on
// MI355X against the 128 x 128 tiles that ran these shapes before
// (interleaved, best of two): 16 x 4096 x 14336 120.7 -> 24.3 us, 64 x 8192
// x 8192 70.8 -> 28.1 us, 80 x 8192 x 8192 71.6 -> 29.8 us, 96 x 4096 x
// 14336 121.3 -> 42.2 us; the workgroups' re-reads of the small side cost
// more than those tiles from 64 rows with a large side of 28672 (119.6
// against 108.6 us) and break even from 96 rows at 14336 to 16384.
bool skinny_pays(int64_t M, int64_t N, int64_t K, int64_t batch)
{
    if (batch != 1 || !skinny_shape(M, N, K)) return false;
    const int64_t small = M < N ? M : N, large = M < N ? N : M;
    return small <= 32 || (small <= 64 && large <= 16384) || large <= 12288;
}

// Shapes of rung 13: K >= 8 (as rung 12), and tile counts within a 1-D
// grid for its smallest tile (16 x 16).
bool ksplit_shape(int64_t M, int64_t N, int64_t K)
{
    return K >= 8 && ((M + 15) / 16) * ((N + 15) / 16) <= (int64_t(1) << 31) - 1;
}

// Models, in microseconds on MI355X, of the ring kernels and of rung 13 on
// shapes whose 128- and 256-row tiles number fewer than the compute units
// (the case rung 13 is for; elsewhere the ring's model is optimistic, which
// keeps rung 13 away).  The ring: the better of 128 x 128 tiles (R9, ~0.40
// us per 64-wide k step of a round of tiles when few compute units are
// busy, 1.4x in its bounds-checked form for M, N not multiples of 128 or K
// of 64: 200 x 1024 x 8192 70.4 us against 49.6 at 128 rows) and 256 x 256
// ones (~1.1 us), plus ~2 us, 1.5x with register-staged loads (K % 8 !=
// 0), and at least its compulsory bytes at ~6 TB/s.
// Rung 13: skinny::ksplit_tile's model, and at least its bytes from HBM at
// ~6 TB/s, where the larger side is read once when the S tiles of an L tile
// run together (in one round, or in the S-major order of the 64-row L
// tiles, skinny::kSMajorMinBytes) or when it fits the last-level cache
// (taken as 128 MiB), else once per round, at most once per tile row.
constexpr double kRingStepUs128 = 0.40, kRingEdge128 = 1.4, kRingStepUs256 = 1.1, kRingFixedUs = 2.0;
constexpr double kHbmBytesPerUs = 6.0e6;
constexpr int64_t kCachedSideBytes = int64_t(128) << 20;
// rung 13 runs where its model is at most this fraction of the ring's.
// Measured on MI355X: on 75 shapes every one below 0.8 ran 1.2-4.9x faster
// on rung 13; on 71 shapes between 0.6 and 1.0, those from 0.83 to 0.87 ran
// 1.06-1.37x faster on rung 13 except three with 128 rows against 6144-8192
// (0.84-0.97x), those around 0.91 and above gained nothing on balance.
constexpr double kKsplitGain = 0.87;

double ring_model_us(int64_t M, int64_t N, int64_t K, int cus)
{
    const int64_t kt = (K + 63) / 64;
    auto rounds = [&](int64_t t) { return (((M + t - 1) / t) * ((N + t - 1) / t) + cus - 1) / cus; };
    const bool edge = M % 128 || N % 128 || K % 64;
    const double r128 = (double)rounds(128) * (double)kt * kRingStepUs128 * (edge ? kRingEdge128 : 1.0);
    const double r256 = (double)rounds(256) * (double)kt * kRingStepUs256;
    double t = (r128 < r256 ? r128 : r256) * (K % 8 != 0 ? 1.5 : 1.0) + kRingFixedUs;
    const double hbm = (double)((M + N) * K * 2) / kHbmBytesPerUs;
    return t > hbm ? t : hbm;
}

double ksplit_model_us(int64_t M, int64_t N, int64_t K, int cus, skinny::Tile* tile)
{
    const int64_t s_rows = M <= N ? M : N, l_rows = M <= N ? N : M;
    double t = 0;
    const skinny::Tile tl = skinny::ksplit_tile(s_rows, l_rows, K, cus, &t);
    const int64_t s_tiles = (s_rows + 16 * tl.mt - 1) / (16 * tl.mt);
    const int64_t wgs = s_tiles * ((l_rows + 16 * tl.nf - 1) / (16 * tl.nf));
    const int64_t rounds = (wgs + cus - 1) / cus;
    const int64_t l_bytes = l_rows * K * 2;
    const bool once = l_bytes <= kCachedSideBytes || rounds <= 1 || skinny::smajor_tile(tl);
    const int64_t l_reads = once ? 1 : (rounds < s_tiles ? rounds : s_tiles);
    const double hbm = (double)(l_bytes * l_reads + s_rows * K * 2) / kHbmBytesPerUs;
    if (tile) *tile = tl;
    return t > hbm ? t : hbm;
}

// Where the library's choice takes rung 13: single products not taken by
// rung 12 whose model beats the ring's by kKsplitGain.
bool ksplit_pays(int64_t M, int64_t N, int64_t K, int64_t batch, int cus)
{
    if (batch != 1 || !ksplit_shape(M, N, K) || skinny_pays(M, N, K, 1) || M == 0 || N == 0) return false;
    return ksplit_model_us(M, N, K, cus, nullptr) <= kKsplitGain * ring_model_us(M, N, K, cus);
}

// Shapes of the 384 x 256 ring (rung 11): one tile row and column at least
// (the last ones move back to end at M and N), whole 64-wide k steps, at
// least two, and an output pitch under 2^23 (its output blocks span 384 *
// ldd bytes in a 32-bit buffer size).
bool wide_shape(int64_t M, int64_t N, int64_t K, int64_t ldd)
{
    return M >= wide::C::BM && N >= wide::C::BN && K % wide::C::BK == 0 && K >= 2 * wide::C::BK &&
           ldd < (int64_t(1) << 23);
}

int validate(int rung, int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* D)
{
    if (!known_rung(rung)) return GEMM_F16_NT_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0) return GEMM_F16_NT_INVALID_ARG;
    const bool any_out = M > 0 && N > 0;
    if (any_out && K > 0 && (A == nullptr || B == nullptr)) return GEMM_F16_NT_INVALID_ARG;
    if (any_out && D == nullptr) return GEMM_F16_NT_INVALID_ARG;
    // index ranges the kernels are built for: per-lane 32-bit byte offsets
    // within a 256-row band, 2^31 tiles, 2D grid limits of the 128-tile rungs
    if (K > (int64_t(1) << 22) || M > (int64_t(1) << 31) || N > (int64_t(1) << 31)) return GEMM_F16_NT_UNSUPPORTED;
    // rungs other than R3, R4 and R9 (and the library's choice) need 16-byte
    // rows; R4's and R9's register-staged forms need K >= 8
    const bool general_ok = rung == 0 || rung == GEMM_F16_NT_R3_GRID ||
                            ((rung == GEMM_F16_NT_R4_RING || rung == GEMM_F16_NT_R9_RING_SMALL ||
                              rung == GEMM_F16_NT_R12_SKINNY || rung == GEMM_F16_NT_R13_KSPLIT) &&
                             K >= 8);
    if (K % 8 != 0 && !general_ok) return GEMM_F16_NT_UNSUPPORTED;
    if (rung == GEMM_F16_NT_R1_SINGLE_TILE && !(M == 128 && N == 128 && K == 64)) return GEMM_F16_NT_UNSUPPORTED;
    if (rung == GEMM_F16_NT_R2_KLOOP && !(M == 128 && N == 128)) return GEMM_F16_NT_UNSUPPORTED;
    if (rung == GEMM_F16_NT_R3_GRID && (N + 127) / 128 > 65535) return GEMM_F16_NT_UNSUPPORTED;
    if (rung == GEMM_F16_NT_R8_RING4_GAP && !(ring4_shape(M, N, K) && ring4_pitch_ok(N)))
        return GEMM_F16_NT_UNSUPPORTED;
    if (rung == GEMM_F16_NT_R10_RING4_PAIRED && !(ring4_paired_shape(M, N, K, K, K) && ring4_pitch_ok(N)))
        return GEMM_F16_NT_UNSUPPORTED;
    if (rung == GEMM_F16_NT_R11_WIDE && !wide_shape(M, N, K, N)) return GEMM_F16_NT_UNSUPPORTED;
    if (rung == GEMM_F16_NT_R12_SKINNY && !skinny_shape(M, N, K)) return GEMM_F16_NT_UNSUPPORTED;
    if (rung == GEMM_F16_NT_R13_KSPLIT && !ksplit_shape(M, N, K)) return GEMM_F16_NT_UNSUPPORTED;
    if (!any_out) return GEMM_F16_NT_OK;
    // fp16 elements are 2-byte aligned; the fast kernels need 16 bytes
    if ((K > 0 && (((uintptr_t)A & 1) || ((uintptr_t)B & 1))) || ((uintptr_t)D & 1)) return GEMM_F16_NT_UNSUPPORTED;
    if (!fast_operands(K, K, K, 0, 0, A, B, D)) {
        if (!general_ok) return GEMM_F16_NT_UNSUPPORTED;
        // grid y of R3's general form (rung 3, and the library's choice for K < 8)
        if ((rung == GEMM_F16_NT_R3_GRID || K < 8) && (N + 127) / 128 > 65535) return GEMM_F16_NT_UNSUPPORTED;
    }
    const int64_t dbytes = M * N * 2;
    if (K > 0 && (overlaps(A, M * K * 2, D, dbytes) || overlaps(B, N * K * 2, D, dbytes)))
        return GEMM_F16_NT_INVALID_ARG;
    return GEMM_F16_NT_OK;
}

// Extent in elements of a batch of row-major matrices, for the overlap check.
int64_t span_elems(int64_t rows, int64_t cols, int64_t ld, int64_t stride, int64_t batch)
{
    if (rows <= 0 || cols <= 0 || batch <= 0) return 0;
    return (batch - 1) * stride + (rows - 1) * ld + cols;
}

int validate_strided(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int64_t sa, const void* B,
                     int64_t ldb, int64_t sb, const void* D, int64_t ldd, int64_t sd, int64_t batch)
{
    if (M < 0 || N < 0 || K < 0 || batch < 0) return GEMM_F16_NT_INVALID_ARG;
    if (lda < K || ldb < K || ldd < N || sa < 0 || sb < 0 || sd < 0) return GEMM_F16_NT_INVALID_ARG;
    const bool any_out = M > 0 && N > 0 && batch > 0;
    if (!any_out) return GEMM_F16_NT_OK;
    if (D == nullptr || (K > 0 && (A == nullptr || B == nullptr))) return GEMM_F16_NT_INVALID_ARG;
    // batch entries of D must not overlap each other (they are written concurrently)
    if (batch > 1 && sd < (M - 1) * ldd + N) return GEMM_F16_NT_INVALID_ARG;
    if (K > (int64_t(1) << 22) || lda > (int64_t(1) << 22) || ldb > (int64_t(1) << 22) || M > (int64_t(1) << 31) ||
        N > (int64_t(1) << 31) || batch > (int64_t(1) << 31))
        return GEMM_F16_NT_UNSUPPORTED;
    if ((K > 0 && (((uintptr_t)A & 1) || ((uintptr_t)B & 1))) || ((uintptr_t)D & 1)) return GEMM_F16_NT_UNSUPPORTED;
    // R3's general form (K < 8 on operands without 16-byte rows) has the
    // grid (tiles_m, tiles_n <= 65535, batch <= 65535)
    if (!fast_operands(K, lda, ldb, sa, sb, A, B, D) && K < 8 && ((N + 127) / 128 > 65535 || batch > 65535))
        return GEMM_F16_NT_UNSUPPORTED;
    const int64_t dbytes = span_elems(M, N, ldd, sd, batch) * 2;
    if (K > 0 && (overlaps(A, span_elems(M, K, lda, sa, batch) * 2, D, dbytes) ||
                  overlaps(B, span_elems(N, K, ldb, sb, batch) * 2, D, dbytes)))
        return GEMM_F16_NT_INVALID_ARG;
    return GEMM_F16_NT_OK;
}

__global__ void fill_zero_strided_kernel(uint16_t* __restrict__ D, int64_t M, int64_t N, int64_t ldd, int64_t sd,
                                         int64_t batch)
{
    const int64_t per = M * N, n = per * batch;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int64_t b = i / per, r = (i - b * per) / N, c = i - b * per - r * N;
        D[b * sd + r * ldd + c] = 0;
    }
}

int launched()
{
    return hipGetLastError() == hipSuccess ? GEMM_F16_NT_OK : GEMM_F16_NT_LAUNCH;
}

int launch_fill_zero(void* D, int64_t n, hipStream_t s)
{
    const int64_t blocks = (n + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, s, (uint16_t*)D, n);
    return launched();
}

// Whether the four-wave scheduled ring (its fourth form) covers this
// problem: its shapes and an output row pitch under 2^24 elements.
bool ring4_fits(const GemmArgs& g)
{
    return ring4_paired_shape(g.M, g.N, g.K, g.lda, g.ldb) && ring4_pitch_ok(g.ldd);
}

// Persistent launch: one workgroup per compute unit (fewer when there are
// fewer tiles); every workgroup walks its share of the tiles.  form: the
// k loop (3 = release and publish barriers with one instruction per MFMA
// gap, 4 = each block's two sub-steps back to back, 0 = the library's
// choice, 4: the fastest at every size measured, whether the operands
// stay in the last-level cache or stream from HBM).
int launch_ring4(const GemmArgs& g0, hipStream_t s, int form = 0)
{
    GemmArgs g = g0;
    g.tiles_m = (g.M + ring4::C::BM - 1) / ring4::C::BM;
    g.tiles_n = (g.N + ring4::C::BN - 1) / ring4::C::BN;
    const int64_t tiles = g.tiles_m * g.tiles_n * g.batch;
    int cus = 0;
    const int st = device_info(&cus);
    if (st != GEMM_F16_NT_OK) return st;
    const int64_t grid = tiles < cus ? tiles : cus;
    if (form == 0) form = 4;
    // only the fourth form has the partial first step
    if (form != 4 && g.K % ring4::C::BK != 0) return GEMM_F16_NT_UNSUPPORTED;
    if (form == 4)
        hipLaunchKernelGGL(ring4::ring4_kernel<4>, dim3((unsigned)grid), dim3(ring4::C::THREADS), 0, s, g);
    else
        hipLaunchKernelGGL(ring4::ring4_kernel<3>, dim3((unsigned)grid), dim3(ring4::C::THREADS), 0, s, g);
    return launched();
}

// Rung 11: the four-wave ring on 384 x 256 tiles, persistent like rung 10.
int launch_wide(const GemmArgs& g0, hipStream_t s)
{
    GemmArgs g = g0;
    g.tiles_m = (g.M + wide::C::BM - 1) / wide::C::BM;
    g.tiles_n = (g.N + wide::C::BN - 1) / wide::C::BN;
    const int64_t tiles = g.tiles_m * g.tiles_n;
    if (tiles > 0x7fffffff) return GEMM_F16_NT_UNSUPPORTED;
    int cus = 0;
    const int st = device_info(&cus);
    if (st != GEMM_F16_NT_OK) return st;
    const int64_t grid = tiles < cus ? tiles : cus;
    hipLaunchKernelGGL(wide::wide_kernel, dim3((unsigned)grid), dim3(wide::C::THREADS), 0, s, g);
    return launched();
}

// Rung 4's ring with 128 x 128 tiles (4 stages), one workgroup per tile.
int launch_ring_small(const GemmArgs& g0, hipStream_t s)
{
    using C = RingSmallCfg;
    GemmArgs g = g0;
    g.tiles_m = (g.M + C::BM - 1) / C::BM;
    g.tiles_n = (g.N + C::BN - 1) / C::BN;
    const int64_t blocks = g.tiles_m * g.tiles_n * g.batch;
    if (blocks > 0x7fffffff) return GEMM_F16_NT_UNSUPPORTED;
    const bool edge = (g.M % C::BM) || (g.N % C::BN) || (g.K % C::BK) || (g.ldd % 8) || (g.sd % 8);
    if (edge)
        hipLaunchKernelGGL((ring::ring_kernel<C, true, kRingPre, kRingLsplit, true>), dim3((unsigned)blocks),
                           dim3(C::THREADS), 0, s, g);
    else
        hipLaunchKernelGGL((ring::ring_kernel<C, false, kRingPre, kRingLsplit, true>), dim3((unsigned)blocks),
                           dim3(C::THREADS), 0, s, g);
    return launched();
}

// Whether 128 x 128 tiles (R9) beat 256 x 256 ones (R4) on a shape the
// four-wave ring does not take, counted in rounds of tiles over the compute
// units: a 128-wide tile is a quarter of the work at about 0.75 of R4's
// rate (measured on MI355X at 4096^3: 929 against 1232 TFLOP/s).  When M or
// N is small, most of a 256-wide tile is padding and its tiles may not fill
// the device (128 x 32768 x 4096: 128 tiles of 256^2, 91 us on R4 against
// 48 us on R9's 256 tiles).
constexpr double kSmallTileRate = 0.75;

bool small_tiles_pay(int64_t M, int64_t N, int64_t batch, int cus)
{
    auto rounds = [&](int64_t t) {
        const int64_t tiles = ((M + t - 1) / t) * ((N + t - 1) / t) * batch;
        return (double)((tiles + cus - 1) / cus);
    };
    return rounds(RingSmallCfg::BM) * 0.25 / kSmallTileRate < rounds(kFastTile);
}

// Whether 256 x 256 tiles would leave most compute units idle.
bool tile_starved(const GemmArgs& g)
{
    int cus = 0;
    if (device_info(&cus) != GEMM_F16_NT_OK) return false;
    const int64_t tiles = ((g.M + kFastTile - 1) / kFastTile) * ((g.N + kFastTile - 1) / kFastTile) * g.batch;
    return tiles * 10 <= (int64_t)cus * kSmallTilesPer10Cus;
}

// A small last round of 256 x 256 tiles (at most a third of the compute
// units busy in it, after at least one full round): the top rows that fill
// whole rounds run on the four-wave ring, and the remaining rows on 128 x
// 128 tiles (R9), which spread the last round's work over four times as
// many workgroups.  No workspace.  Measured on MI355X against the
// four-wave ring alone: 6144^3 -10%, 4352^2 x 4096 -20%, 7168^2 x 4096 -6%,
// 6144^2 x 1024 -4%; with more than a third of a round left (5120^2 x 4096)
// it is 6% slower.  Short K (under 16 steps) is left alone: the second
// launch costs about what it saves.
constexpr int64_t kRoundSplitMinSteps = 16;

bool round_split(const GemmArgs& g, int cus, int64_t* m_top)
{
    if (g.batch != 1 || (g.K + RingCfg::BK - 1) / RingCfg::BK < kRoundSplitMinSteps) return false;
    const int64_t tm = (g.M + kFastTile - 1) / kFastTile, tn = (g.N + kFastTile - 1) / kFastTile;
    const int64_t tiles = tm * tn, rounds = tiles / cus, rest = tiles % cus;
    if (rounds < 1 || rest == 0 || rest * 3 > cus) return false;
    const int64_t r_top = rounds * cus / tn;   // whole tile rows that fit in whole rounds
    if (r_top < 1 || r_top >= tm) return false;
    const int64_t m_rest = g.M - r_top * kFastTile;
    const int64_t small = (m_rest + RingSmallCfg::BM - 1) / RingSmallCfg::BM * ((g.N + RingSmallCfg::BN - 1) / RingSmallCfg::BN);
    if (small > 2 * (int64_t)cus) return false;
    *m_top = r_top * kFastTile;
    return true;
}

// Rows of the product that run on rung 11's 384 x 256 tiles: 0 (none), M
// (all of it), or the top rows, with the rest on the four-wave ring's 256 x
// 256 tiles as a second launch.  The choice counts rounds of tiles over the
// compute units.  Per FLOP the wider tile moves a sixth fewer operand bytes;
// measured on MI355X at 12288 x 4096 x 4096, where both tile sizes fill
// whole rounds, it runs 2.5% faster, so one 384-row tile costs 1.5 / 1.025
// of a 256-row one.  It pays where its tiles fill the rounds better (6144 x
// 4096 x 4096: one round against 1.5, 128 against 174 us) or equally well,
// and as the top rows of products whose 256-row tiles fill whole rounds but
// whose 384-row tiles do not (8192^3: two rounds of 384-row tiles over the
// top 6144 rows plus one round of 256-row tiles, 707 against 722 us; the
// output is bitwise that of the four-wave ring alone, both accumulating
// each block's k steps in the same order).  A second launch is counted as
// kWideSplitCost of a round.  Where the 256 x 256 tiles leave a small last
// round, the split of round_split is kept, and so is the four-wave ring for
// short K (at most kCarryMaxSteps steps), where it carries its ring from
// tile to tile and rung 11 does not.
constexpr double kWideTileCost = 1.5 / 1.025;
constexpr double kWideSplitCost = 0.02;

int64_t wide_rows(const GemmArgs& g, int cus)
{
    if (g.batch != 1 || !wide_shape(g.M, g.N, g.K, g.ldd) || g.K / wide::C::BK <= ring4::kCarryMaxSteps) return 0;
    int64_t m_top = 0;
    if (round_split(g, cus, &m_top)) return 0;
    const int64_t tn = (g.N + kFastTile - 1) / kFastTile;
    const auto rounds = [&](int64_t rows, int64_t tile) {
        return (double)(((rows + tile - 1) / tile * tn + cus - 1) / cus);
    };
    double best = rounds(g.M, kFastTile);   // the four-wave ring alone
    int64_t best_rows = 0;
    if (rounds(g.M, wide::C::BM) * kWideTileCost < best) {
        best = rounds(g.M, wide::C::BM) * kWideTileCost;
        best_rows = g.M;
    }
    // top rows in 384-row tile rows that fill whole rounds of the compute
    // units; the rest (at least one 256-row tile row, as the four-wave ring
    // needs) on 256 x 256 tiles
    const int64_t step_rows = cus / std::gcd(tn, (int64_t)cus);   // tile rows per whole round
    for (int64_t m = step_rows * wide::C::BM; m + kFastTile <= g.M; m += step_rows * wide::C::BM) {
        const double c = rounds(m, wide::C::BM) * kWideTileCost + rounds(g.M - m, kFastTile) + kWideSplitCost;
        if (c < best) {
            best = c;
            best_rows = m;
        }
    }
    return best_rows;
}

int launch_ring(const GemmArgs& g0, hipStream_t s, bool allow_ring4 = false)
{
    if (allow_ring4 && tile_starved(g0)) return launch_ring_small(g0, s);
    if (allow_ring4 && ring4_fits(g0)) {
        int cus = 0, st = device_info(&cus);
        if (st != GEMM_F16_NT_OK) return st;
        const int64_t m_wide = wide_rows(g0, cus);
        if (m_wide == g0.M) return launch_wide(g0, s);
        if (m_wide > 0) {
            GemmArgs top = g0, rest = g0;
            top.M = m_wide;
            rest.M = g0.M - m_wide;
            rest.A = g0.A + m_wide * g0.lda;
            rest.D = g0.D + m_wide * g0.ldd;
            st = launch_wide(top, s);
            return st != GEMM_F16_NT_OK ? st : launch_ring4(rest, s);
        }
        int64_t m_top = 0;
        if (!round_split(g0, cus, &m_top)) return launch_ring4(g0, s);
        GemmArgs top = g0, rest = g0;
        top.M = m_top;
        rest.M = g0.M - m_top;
        rest.A = g0.A + m_top * g0.lda;
        rest.D = g0.D + m_top * g0.ldd;
        st = launch_ring4(top, s);
        return st != GEMM_F16_NT_OK ? st : launch_ring_small(rest, s);
    }
    if (allow_ring4) {
        int cus = 0, st = device_info(&cus);
        if (st != GEMM_F16_NT_OK) return st;
        if (small_tiles_pay(g0.M, g0.N, g0.batch, cus)) return launch_ring_small(g0, s);
    }
    GemmArgs g = g0;
    g.tiles_m = (g.M + kFastTile - 1) / kFastTile;
    g.tiles_n = (g.N + kFastTile - 1) / kFastTile;
    const int64_t blocks = g.tiles_m * g.tiles_n * g.batch;
    if (blocks > 0x7fffffff) return GEMM_F16_NT_UNSUPPORTED;
    // the fast variant needs whole tiles and 16-byte aligned rows of D
    const bool edge = (g.M % kFastTile) || (g.N % kFastTile) || (g.K % RingCfg::BK) || (g.ldd % 8) || (g.sd % 8);
    if (edge)
        hipLaunchKernelGGL((ring::ring_kernel<RingCfg, true, kRingPre, kRingLsplit, true>), dim3((unsigned)blocks),
                           dim3(RingCfg::THREADS), 0, s, g);
    else
        hipLaunchKernelGGL((ring::ring_kernel<RingCfg, false, kRingPre, kRingLsplit, true>), dim3((unsigned)blocks),
                           dim3(RingCfg::THREADS), 0, s, g);
    return launched();
}

// ------------------------------------------------------------- split-K
// Slices of K for a tile-starved product: enough to give every CU a
// workgroup, but at least kMinStepsPerSlice 64-wide steps per slice (a
// slice pays a prologue, a partial-sum write and its share of the
// reduction; measured on MI355X, K = 512 on one 256 x 256 tile is faster
// unsplit) and at most kMaxSplits slices.  With at most kFewTiles tiles
// and K of at least 32 steps, half as many steps per slice pay (32 slices
// against 16, interleaved:
// 256 x 1024 x 8192 29.0 -> 25.4 us, 64 x 1024 x 8192 21.3 -> 17.8 us,
// 128 x 1024 x 8192 25.0 -> 22.7 us).
constexpr int64_t kMaxSplits = 64;
constexpr int64_t kMinStepsPerSlice = 8;
constexpr int64_t kFewTiles = 4;

int64_t choose_splits(int64_t M, int64_t N, int64_t K, int cus)
{
    // one small side: rung 12 splits K inside its workgroups without a
    // workspace, faster than slices (measured on MI355X: 64 x 8192 x 8192
    // 28.3 us against 34.7 us in 8 slices, 64 x 1024 x 8192 15.3 against 17.7)
    if (skinny_pays(M, N, K, 1)) return 1;
    const int64_t tiles = ((M + kFastTile - 1) / kFastTile) * ((N + kFastTile - 1) / kFastTile);
    const int64_t kt = (K + RingCfg::BK - 1) / RingCfg::BK;
    if (tiles * 2 >= cus) return 1;
    const int64_t min_steps =
        tiles <= kFewTiles && kt >= 4 * kMinStepsPerSlice ? kMinStepsPerSlice / 2 : kMinStepsPerSlice;
    int64_t s = cus / tiles;
    s = s < kt / min_steps ? s : kt / min_steps;
    s = s < kMaxSplits ? s : kMaxSplits;
    return s > 1 ? s : 1;
}

// k elements per slice (a whole number of 64-wide steps) and the slice count
void split_plan(int64_t K, int64_t splits, int64_t* k_chunk, int64_t* n_slices)
{
    const int64_t kt = (K + RingCfg::BK - 1) / RingCfg::BK;
    const int64_t steps = (kt + splits - 1) / splits;
    *k_chunk = steps * RingCfg::BK;
    *n_slices = (K + *k_chunk - 1) / *k_chunk;
}

// Shapes with at least one full round of 256 x 256 tiles and a small last
// round: the top rows that fill whole rounds run whole on the four-wave
// ring, and the remaining rows split K, so that the last round's work is
// shared by every compute unit instead of a few.  A cost model in units of
// one four-wave k step per tile picks the slice count; the split is taken
// when it models at most kHybridGain of the unsplit time.  Measured on
// MI355X: the rows split K on the 8-wave ring at ~0.78 of the four-wave
// ring's rate, and its partial sums (written once, read once) move at ~8
// TB/s from the last-level cache, ~10 MB per step time.
constexpr double kHybridGain = 0.90;
constexpr double kSplitSlowdown = 1.28;
constexpr double kBytesPerStepTime = 10.3e6;
constexpr double kSplitFixedSteps = 6.7;   // two more launches and a slice's prologue and epilogue

GemmArgs contiguous_args(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D);

bool hybrid_plan(int64_t M, int64_t N, int64_t K, int cus, int64_t* m_top, int64_t* splits)
{
    if (K % 8 != 0 || !ring4_paired_shape(ring4::C::BM, N, K, K, K) || !ring4_pitch_ok(N)) return false;
    // where the unsplit call already moves a small last round to 128 x 128
    // tiles that fit in one round, that is as fast (measured: 4352^2 x 4096
    // 120 us unsplit against 128 us split); it loses to the split when they
    // need two rounds (6144^3: 353 against 330 us)
    int64_t rs_top = 0;
    if (round_split(contiguous_args(M, N, K, nullptr, nullptr, nullptr), cus, &rs_top)) {
        const int64_t small = (M - rs_top + RingSmallCfg::BM - 1) / RingSmallCfg::BM *
                              ((N + RingSmallCfg::BN - 1) / RingSmallCfg::BN);
        if (small <= (int64_t)cus) return false;
    }
    const int64_t tm = (M + kFastTile - 1) / kFastTile, tn = (N + kFastTile - 1) / kFastTile;
    const int64_t tiles = tm * tn, kt = (K + RingCfg::BK - 1) / RingCfg::BK;
    const int64_t rounds = tiles / cus;
    if (rounds < 1 || tiles % cus == 0) return false;
    const int64_t r_top = rounds * cus / tn;   // whole tile rows that fit in whole rounds
    if (r_top < 1 || r_top >= tm) return false;
    const int64_t m_rest = M - r_top * kFastTile;
    const int64_t t_rest = (m_rest + kFastTile - 1) / kFastTile * tn;
    const double plain = (double)((tiles + cus - 1) / cus * kt);
    const double top = (double)((r_top * tn + cus - 1) / cus * kt);
    double best = kHybridGain * plain;
    int64_t best_s = 0;
    for (int64_t sl = 2; sl <= kMaxSplits && sl <= kt / kMinStepsPerSlice; ++sl) {
        int64_t k_chunk = 0, n_slices = 0;
        split_plan(K, sl, &k_chunk, &n_slices);
        const double rounds_sk = (double)((t_rest * n_slices + cus - 1) / cus);
        const double bytes = (2.0 * (double)n_slices + 0.5) * (double)m_rest * (double)N * 4.0;
        const double t = top + rounds_sk * (double)(k_chunk / RingCfg::BK) * kSplitSlowdown +
                         bytes / kBytesPerStepTime + kSplitFixedSteps;
        if (t < best) {
            best = t;
            best_s = sl;
        }
    }
    if (best_s == 0) return false;
    *m_top = r_top * kFastTile;
    *splits = best_s;
    return true;
}

// Modeled time (us) of a split-K call with `splits` slices, in the units of
// hybrid_plan (one four-wave k step of a round of tiles, ~1.1 us when few
// compute units are busy).
double splitk_model_us(int64_t M, int64_t N, int64_t K, int64_t splits, int cus)
{
    int64_t k_chunk = 0, n_slices = 0;
    split_plan(K, splits, &k_chunk, &n_slices);
    const int64_t tiles = ((M + kFastTile - 1) / kFastTile) * ((N + kFastTile - 1) / kFastTile);
    const double rounds = (double)((tiles * n_slices + cus - 1) / cus);
    const double bytes = (2.0 * (double)n_slices + 0.5) * (double)M * (double)N * 4.0;
    return (rounds * (double)(k_chunk / RingCfg::BK) * kSplitSlowdown + bytes / kBytesPerStepTime + kSplitFixedSteps) *
           kRingStepUs256;
}

// The split-K entry's choice for splits = 0 (before hybrid_plan's split of
// whole rounds): choose_splits' slice count, or 1 for one launch when a
// model of that beats the slices' -- rung 13 when *r13 is set (its model
// the smallest), else gemm_f16_nt's choice.  Measured on MI355X (one box,
// interleaved): 256 x 1024 x 8192 14.1 us on rung 13 against 25.2 in 32
// slices; 256 x 4096 x 4096 25.3 on rung 13 against 28.1 in 8 slices;
// 128 x 14336 x 4096 28.6 unsplit against 38.9 in 4 slices; with a long K
// on a small output the slices' 256 x 256 tiles win (256 x 256 x 65536:
// 35.6 against 50.1 on rung 13).
int64_t plan_splits(int64_t M, int64_t N, int64_t K, int cus, bool* r13)
{
    *r13 = false;
    const int64_t s = choose_splits(M, N, K, cus);
    if (s <= 1) return 1;
    const double split = splitk_model_us(M, N, K, s, cus);
    const double ring = ring_model_us(M, N, K, cus);
    const bool k13 = ksplit_shape(M, N, K) && !skinny_pays(M, N, K, 1);
    const double t13 = k13 ? ksplit_model_us(M, N, K, cus, nullptr) : 0.0;
    if (k13 && t13 <= split && t13 <= ring) {
        *r13 = true;
        return 1;
    }
    return ring <= split ? 1 : s;
}

int launch_splitk(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D, int64_t splits,
                  float* P, hipStream_t s)
{
    int64_t k_chunk = 0, n_slices = 0;
    split_plan(K, splits, &k_chunk, &n_slices);
    GemmArgs g{};
    g.A = (const f16*)A;
    g.B = (const f16*)B;
    g.D = (f16*)D;
    g.M = M;
    g.N = N;
    g.K = K;
    g.lda = K;
    g.ldb = K;
    g.ldd = N;
    g.batch = n_slices;
    g.k_chunk = k_chunk;
    g.P = P;
    g.tiles_m = (M + kFastTile - 1) / kFastTile;
    g.tiles_n = (N + kFastTile - 1) / kFastTile;
    const int64_t blocks = g.tiles_m * g.tiles_n * n_slices;
    if (blocks > 0x7fffffff) return GEMM_F16_NT_UNSUPPORTED;
    const bool edge = (M % kFastTile) || (N % kFastTile) || (K % RingCfg::BK);
    if (edge)
        hipLaunchKernelGGL((ring::ring_kernel<RingCfg, true, kRingPre, kRingLsplit, false, false, true>),
                           dim3((unsigned)blocks), dim3(RingCfg::THREADS), 0, s, g);
    else
        hipLaunchKernelGGL((ring::ring_kernel<RingCfg, false, kRingPre, kRingLsplit, false, false, true>),
                           dim3((unsigned)blocks), dim3(RingCfg::THREADS), 0, s, g);
    int st = launched();
    if (st != GEMM_F16_NT_OK) return st;
    // one wave per workgroup when 4-wave ones would not reach every compute
    // unit (a 256 x 256 output is 16384 items)
    int cus = 0;
    st = device_info(&cus);
    if (st != GEMM_F16_NT_OK) return st;
    const bool vec = N % 4 == 0;
    const int64_t items = vec ? M * N / 4 : M * N;
    const int threads = items < 256 * (int64_t)cus ? 64 : 256;
    const int64_t rblocks = (items + threads - 1) / threads;
    const unsigned rgrid = (unsigned)(rblocks < 16384 ? rblocks : 16384);
    if (vec)
        hipLaunchKernelGGL(ring::splitk_reduce_kernel<true>, dim3(rgrid), dim3(threads), 0, s, P, (f16*)D, M, N, N,
                           n_slices);
    else
        hipLaunchKernelGGL(ring::splitk_reduce_kernel<false>, dim3(rgrid), dim3(threads), 0, s, P, (f16*)D, M, N,
                           N, n_slices);
    return launched();
}

// General operands (any K, strides, 2-byte alignment): R3's structure with
// element-wise operand copies.
int launch_r3_any(const GemmArgs& g, hipStream_t s)
{
    const dim3 grid((unsigned)((g.M + 127) / 128), (unsigned)((g.N + 127) / 128), (unsigned)g.batch);
    hipLaunchKernelGGL(ladder::r3_any, grid, dim3(ladder::THREADS), 0, s, g);
    return launched();
}

// R4 (256 x 256 tiles) or R9 (128 x 128, `small`) on general operands: the
// pipelined ring with its loads staged through registers, which take rows
// on any 2-byte boundary.  Needs K >= 8.
template <int MT, int NF, int DB, bool TRANS, int NW = skinny::kWaves>
void launch_skinny_t(const skinny::Args& a, int64_t grid, hipStream_t s)
{
    hipLaunchKernelGGL((skinny::skinny_kernel<MT, NF, DB, TRANS, false, NW>), dim3((unsigned)grid), dim3(64 * NW), 0,
                       s, a);
}

// Rung 13's tiles with 64 L rows in the S-major order (skinny::kSMajorMinBytes).
template <int MT, int NF, int DB, bool TRANS, int NW = skinny::kWaves>
void launch_skinny_smaj(const skinny::Args& a, int64_t grid, hipStream_t s)
{
    hipLaunchKernelGGL((skinny::skinny_kernel<MT, NF, DB, TRANS, true, NW>), dim3((unsigned)grid), dim3(64 * NW), 0,
                       s, a);
}

// The instantiated tiles: rung 12's (skinny::skinny_tile: mt = 1..6 blocks
// of S, 1 or 2 of L) and rung 13's (skinny::kTiles13, two of them with 4
// waves).
template <bool TRANS>
int launch_skinny_tile(const skinny::Args& a, const skinny::Tile& t, int64_t grid, bool smaj, hipStream_t s)
{
    if (t.nw == 4) {
        switch (t.mt * 100 + t.nf * 10 + t.db) {
        case 241:
            if (smaj)
                launch_skinny_smaj<2, 4, 1, TRANS, 4>(a, grid, s);
            else
                launch_skinny_t<2, 4, 1, TRANS, 4>(a, grid, s);
            break;
        case 441:
            if (smaj) return GEMM_F16_NT_UNSUPPORTED;
            launch_skinny_t<4, 4, 1, TRANS, 4>(a, grid, s);
            break;
        default: return GEMM_F16_NT_UNSUPPORTED;
        }
        return launched();
    }
    if (t.nw != skinny::kWaves) return GEMM_F16_NT_UNSUPPORTED;
    if (smaj) {
        switch (t.mt * 100 + t.nf * 10 + t.db) {
        case 241: launch_skinny_smaj<2, 4, 1, TRANS>(a, grid, s); break;
        case 341: launch_skinny_smaj<3, 4, 1, TRANS>(a, grid, s); break;
        default: return GEMM_F16_NT_UNSUPPORTED;
        }
        return launched();
    }
    switch (t.mt * 100 + t.nf * 10 + t.db) {
    case 112: launch_skinny_t<1, 1, 2, TRANS>(a, grid, s); break;
    case 121: launch_skinny_t<1, 2, 1, TRANS>(a, grid, s); break;
    case 122: launch_skinny_t<1, 2, 2, TRANS>(a, grid, s); break;
    case 211: launch_skinny_t<2, 1, 1, TRANS>(a, grid, s); break;
    case 221: launch_skinny_t<2, 2, 1, TRANS>(a, grid, s); break;
    case 241: launch_skinny_t<2, 4, 1, TRANS>(a, grid, s); break;
    case 311: launch_skinny_t<3, 1, 1, TRANS>(a, grid, s); break;
    case 321: launch_skinny_t<3, 2, 1, TRANS>(a, grid, s); break;
    case 341: launch_skinny_t<3, 4, 1, TRANS>(a, grid, s); break;
    case 411: launch_skinny_t<4, 1, 1, TRANS>(a, grid, s); break;
    case 421: launch_skinny_t<4, 2, 1, TRANS>(a, grid, s); break;
    case 511: launch_skinny_t<5, 1, 1, TRANS>(a, grid, s); break;
    case 521: launch_skinny_t<5, 2, 1, TRANS>(a, grid, s); break;
    case 611: launch_skinny_t<6, 1, 1, TRANS>(a, grid, s); break;
    case 621: launch_skinny_t<6, 2, 1, TRANS>(a, grid, s); break;
    default: return GEMM_F16_NT_UNSUPPORTED;
    }
    return launched();
}

// The workgroup tile rung 12 or 13 takes for a product (S = the side with
// fewer rows, A on a tie).
skinny::Tile ksplit_tile_for(int rung, int64_t M, int64_t N, int64_t K, int cus)
{
    const int64_t s_rows = M <= N ? M : N, l_rows = M <= N ? N : M;
    if (rung == GEMM_F16_NT_R12_SKINNY) return skinny::skinny_tile(s_rows, l_rows, K, cus);
    return skinny::ksplit_tile(s_rows, l_rows, K, cus, nullptr);
}

// Rungs 12 and 13 on one product (batch 1): the side with fewer rows is S
// (A on a tie); rung 12 puts all of it in every workgroup (one row of
// tiles), rung 13 tiles it too.
int launch_skinny(const GemmArgs& g, hipStream_t s, int rung = GEMM_F16_NT_R12_SKINNY)
{
    if (g.batch != 1) return GEMM_F16_NT_UNSUPPORTED;
    if (rung == GEMM_F16_NT_R12_SKINNY ? !skinny_shape(g.M, g.N, g.K) : !ksplit_shape(g.M, g.N, g.K))
        return GEMM_F16_NT_UNSUPPORTED;
    int cus = 0;
    const int st = device_info(&cus);
    if (st != GEMM_F16_NT_OK) return st;
    const bool trans = g.N < g.M;
    skinny::Args a;
    a.S = trans ? g.B : g.A;
    a.ld_s = trans ? g.ldb : g.lda;
    a.s_rows = trans ? g.N : g.M;
    a.L = trans ? g.A : g.B;
    a.ld_l = trans ? g.lda : g.ldb;
    a.l_rows = trans ? g.M : g.N;
    a.K = g.K;
    a.D = g.D;
    a.ldd = g.ldd;
    const skinny::Tile t = ksplit_tile_for(rung, g.M, g.N, g.K, cus);
    const int64_t l_tiles = (a.l_rows + 16 * t.nf - 1) / (16 * t.nf);
    const int64_t s_tiles = (a.s_rows + 16 * t.mt - 1) / (16 * t.mt);
    const int64_t grid = l_tiles * s_tiles;
    if (grid > (int64_t(1) << 31) - 1) return GEMM_F16_NT_UNSUPPORTED;
    a.l_tiles = (uint32_t)l_tiles;
    a.s_tiles = (uint32_t)s_tiles;
    const bool smaj = rung == GEMM_F16_NT_R13_KSPLIT && skinny::smajor_tile(t) &&
                      a.l_rows * a.K * 2 > skinny::kSMajorMinBytes && grid > cus;
    return trans ? launch_skinny_tile<true>(a, t, grid, smaj, s) : launch_skinny_tile<false>(a, t, grid, smaj, s);
}

int launch_staged(const GemmArgs& g0, hipStream_t s, bool small)
{
    GemmArgs g = g0;
    const int64_t tile = small ? RingSmallCfg::BM : kFastTile;
    g.tiles_m = (g.M + tile - 1) / tile;
    g.tiles_n = (g.N + tile - 1) / tile;
    const int64_t blocks = g.tiles_m * g.tiles_n * g.batch;
    if (blocks > 0x7fffffff) return GEMM_F16_NT_UNSUPPORTED;
    if (small)
        hipLaunchKernelGGL((ring::ring_kernel<RingSmallCfg, true, kRingPre, kRingLsplit, true, false, false, true>),
                           dim3((unsigned)blocks), dim3(RingSmallCfg::THREADS), 0, s, g);
    else
        hipLaunchKernelGGL((ring::ring_kernel<RingCfg, true, kRingPre, kRingLsplit, true, false, false, true>),
                           dim3((unsigned)blocks), dim3(RingCfg::THREADS), 0, s, g);
    return launched();
}

// The library's kernel for general operands: the staged ring, on 128 x 128
// tiles when 256 x 256 ones would leave most compute units idle.  K < 8 (a
// row shorter than one 16-byte load) runs on R3's general form.
int launch_any(const GemmArgs& g, hipStream_t s)
{
    if (g.K < 8) return launch_r3_any(g, s);
    int cus = 0, st = device_info(&cus);
    if (st != GEMM_F16_NT_OK) return st;
    return launch_staged(g, s, tile_starved(g) || small_tiles_pay(g.M, g.N, g.batch, cus));
}

GemmArgs contiguous_args(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D)
{
    GemmArgs g{};
    g.A = (const f16*)A;
    g.B = (const f16*)B;
    g.D = (f16*)D;
    g.M = M;
    g.N = N;
    g.K = K;
    g.lda = K;
    g.ldb = K;
    g.ldd = N;
    g.sa = g.sb = g.sd = 0;
    g.batch = 1;
    return g;
}

int launch_ws(int64_t M, int64_t N, int64_t K, const f16* A, const f16* B, f16* D, int64_t grid,
              hipStream_t s)
{
    const int64_t tm = (M + WsCfg::BM - 1) / WsCfg::BM, tn = (N + WsCfg::BN - 1) / WsCfg::BN;
    const bool edge = (M % WsCfg::BM) || (N % WsCfg::BN) || (K % WsCfg::BK) || (N % 4);
    if (grid > tm * tn) grid = tm * tn;
    if (edge)
        hipLaunchKernelGGL((ws::ws_kernel<WsCfg, true>), dim3((unsigned)grid), dim3(WsCfg::THREADS), 0, s, A, B, D,
                           M, N, K, tm, tn);
    else
        hipLaunchKernelGGL((ws::ws_kernel<WsCfg, false>), dim3((unsigned)grid), dim3(WsCfg::THREADS), 0, s, A, B, D,
                           M, N, K, tm, tn);
    return launched();
}

int run(int rung, int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D, int64_t grid_override,
        void* stream)
{
    int st = validate(rung, M, N, K, A, B, D);
    if (st != GEMM_F16_NT_OK) return st;
    if (M == 0 || N == 0) return GEMM_F16_NT_OK;
    int cus = 0;
    st = device_info(&cus);
    if (st != GEMM_F16_NT_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (K == 0) return launch_fill_zero(D, M * N, s);
    const f16* a = (const f16*)A;
    const f16* b = (const f16*)B;
    f16* d = (f16*)D;
    switch (rung) {
    case GEMM_F16_NT_R1_SINGLE_TILE:
        hipLaunchKernelGGL(ladder::r1_single_tile, dim3(1), dim3(ladder::THREADS), 0, s, a, b, d);
        return launched();
    case GEMM_F16_NT_R2_KLOOP:
    case GEMM_F16_NT_R3_GRID: {
        if (!fast_operands(K, K, K, 0, 0, A, B, D)) return launch_r3_any(contiguous_args(M, N, K, A, B, D), s);
        const dim3 grid((unsigned)((M + 127) / 128), (unsigned)((N + 127) / 128));
        hipLaunchKernelGGL(ladder::r23_kloop_grid, grid, dim3(ladder::THREADS), 0, s, a, b, d, M, N, K);
        return launched();
    }
    case GEMM_F16_NT_R4_RING:
        if (!fast_operands(K, K, K, 0, 0, A, B, D)) return launch_staged(contiguous_args(M, N, K, A, B, D), s, false);
        return launch_ring(contiguous_args(M, N, K, A, B, D), s);
    case GEMM_F16_NT_R5_PERSISTENT_WS:
        return launch_ws(M, N, K, a, b, d, grid_override > 0 ? grid_override : cus, s);
    case GEMM_F16_NT_R8_RING4_GAP:
        return launch_ring4(contiguous_args(M, N, K, A, B, D), s, 3);
    case GEMM_F16_NT_R9_RING_SMALL:
        if (!fast_operands(K, K, K, 0, 0, A, B, D)) return launch_staged(contiguous_args(M, N, K, A, B, D), s, true);
        return launch_ring_small(contiguous_args(M, N, K, A, B, D), s);
    case GEMM_F16_NT_R10_RING4_PAIRED:
        return launch_ring4(contiguous_args(M, N, K, A, B, D), s, 4);
    case GEMM_F16_NT_R11_WIDE:
        return launch_wide(contiguous_args(M, N, K, A, B, D), s);
    case GEMM_F16_NT_R12_SKINNY:
        return launch_skinny(contiguous_args(M, N, K, A, B, D), s);
    case GEMM_F16_NT_R13_KSPLIT:
        return launch_skinny(contiguous_args(M, N, K, A, B, D), s, GEMM_F16_NT_R13_KSPLIT);
    default:  // 0: the library's choice
        if (skinny_pays(M, N, K, 1)) return launch_skinny(contiguous_args(M, N, K, A, B, D), s);
        if (ksplit_pays(M, N, K, 1, cus))
            return launch_skinny(contiguous_args(M, N, K, A, B, D), s, GEMM_F16_NT_R13_KSPLIT);
        if (!fast_operands(K, K, K, 0, 0, A, B, D)) return launch_any(contiguous_args(M, N, K, A, B, D), s);
        return launch_ring(contiguous_args(M, N, K, A, B, D), s, kDefaultRing4);
    }
}

// ------------------------------------------------- no-allocation scratch
// The split-K partial sums of gemm_f16_nt_splitk_noalloc live in this
// file-scope device array, one copy per device the library runs on, held
// until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is passed to kernels.
struct ScratchSlot {
    std::atomic<int> state{0};  // 0 unknown, 1 ok, -1 unusable
    void* ptr = nullptr;
};
ScratchSlot g_scratch[kMaxDevices];
std::mutex g_scratch_lock;

int scratch_address(void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GEMM_F16_NT_DEVICE;
    ScratchSlot& sl = g_scratch[dev];
    int st = sl.state.load(std::memory_order_acquire);
    if (st == 0) {
        std::lock_guard<std::mutex> lock(g_scratch_lock);
        st = sl.state.load(std::memory_order_relaxed);
        if (st == 0) {
            void* p = nullptr;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            st = (e == hipSuccess && p != nullptr) ? 1 : -1;
            if (st == 1) sl.ptr = p;
            sl.state.store(st, std::memory_order_release);
        }
    }
    if (st != 1) return GEMM_F16_NT_DEVICE;
    *out = sl.ptr;
    return GEMM_F16_NT_OK;
}

// gemm_f16_nt_splitk's body: the partial sums go to the caller's workspace,
// or (noalloc) to this device's scratch array.
int splitk_run(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D, int splits, void* workspace,
               int64_t workspace_bytes, bool noalloc, hipStream_t s)
{
    int st = validate(0, M, N, K, A, B, D);
    if (st != GEMM_F16_NT_OK) return st;
    if (M == 0 || N == 0) return GEMM_F16_NT_OK;
    // an explicit slice count fixes the scratch size before any HIP call
    if (noalloc && splits > 0 && K > 0 && fast_operands(K, K, K, 0, 0, A, B, D)) {
        int64_t k_chunk = 0, n_slices = 1;
        if (splits > 1) split_plan(K, splits, &k_chunk, &n_slices);
        if (n_slices > 1 && n_slices * M * N * 4 > kScratchBytes) return GEMM_F16_NT_SCRATCH;
    }
    int cus = 0;
    st = device_info(&cus);
    if (st != GEMM_F16_NT_OK) return st;
    if (K == 0) return launch_fill_zero(D, M * N, s);
    // one slice, or rows off 16-byte boundaries: gemm_f16_nt's choice
    const auto unsplit = [&]() {
        const GemmArgs g = contiguous_args(M, N, K, A, B, D);
        if (skinny_pays(M, N, K, 1)) return launch_skinny(g, s);
        if (ksplit_pays(M, N, K, 1, cus)) return launch_skinny(g, s, GEMM_F16_NT_R13_KSPLIT);
        return fast_operands(K, K, K, 0, 0, A, B, D) ? launch_ring(g, s, kDefaultRing4) : launch_any(g, s);
    };
    if (!fast_operands(K, K, K, 0, 0, A, B, D)) return unsplit();
    bool r13 = false;
    int64_t want = splits == 0 ? plan_splits(M, N, K, cus, &r13) : splits, m_top = 0;
    if (splits == 0 && want <= 1 && !hybrid_plan(M, N, K, cus, &m_top, &want)) m_top = 0;
    int64_t k_chunk = 0, n_slices = 1;
    if (want > 1) split_plan(K, want, &k_chunk, &n_slices);
    if (n_slices <= 1)
        return r13 ? launch_skinny(contiguous_args(M, N, K, A, B, D), s, GEMM_F16_NT_R13_KSPLIT) : unsplit();
    // rows [m_top, M) split K; rows [0, m_top) (whole rounds of tiles) do not
    const int64_t m_rest = M - m_top;
    const int64_t need = n_slices * m_rest * N * 4;
    if (noalloc) {
        if (need > kScratchBytes) return GEMM_F16_NT_SCRATCH;
        st = scratch_address(&workspace);
        if (st != GEMM_F16_NT_OK) return st;
        workspace_bytes = kScratchBytes;
    } else {
        if (workspace == nullptr || workspace_bytes < need) return GEMM_F16_NT_INVALID_ARG;
        if ((uintptr_t)workspace & 15) return GEMM_F16_NT_UNSUPPORTED;
        if (overlaps(workspace, need, A, M * K * 2) || overlaps(workspace, need, B, N * K * 2) ||
            overlaps(workspace, need, D, M * N * 2))
            return GEMM_F16_NT_INVALID_ARG;
    }
    if (m_top > 0) {
        st = launch_ring(contiguous_args(m_top, N, K, A, B, D), s, kDefaultRing4);
        if (st != GEMM_F16_NT_OK) return st;
    }
    return launch_splitk(m_rest, N, K, (const f16*)A + m_top * K, B, (f16*)D + m_top * N, want, (float*)workspace,
                         s);
}

}  // namespace

extern "C" {

int gemm_f16_nt(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D, void* stream)
{
    return run(0, M, N, K, A, B, D, 0, stream);
}

int gemm_f16_nt_rung(int rung, int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D,
                     void* stream)
{
    if (rung < 1) return GEMM_F16_NT_INVALID_ARG;
    return run(rung, M, N, K, A, B, D, 0, stream);
}

int gemm_f16_nt_persistent(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D,
                           int64_t num_workgroups, void* stream)
{
    if (num_workgroups < 1 || num_workgroups > (int64_t(1) << 31) - 1) return GEMM_F16_NT_INVALID_ARG;
    return run(GEMM_F16_NT_R5_PERSISTENT_WS, M, N, K, A, B, D, num_workgroups, stream);
}

int gemm_f16_nt_strided_batched(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int64_t stride_a,
                                const void* B, int64_t ldb, int64_t stride_b, void* D, int64_t ldd,
                                int64_t stride_d, int64_t batch, void* stream)
{
    int st = validate_strided(M, N, K, A, lda, stride_a, B, ldb, stride_b, D, ldd, stride_d, batch);
    if (st != GEMM_F16_NT_OK) return st;
    if (M == 0 || N == 0 || batch == 0) return GEMM_F16_NT_OK;
    int cus = 0;
    st = device_info(&cus);
    if (st != GEMM_F16_NT_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (K == 0) {
        const int64_t n = M * N * batch, blocks = (n + 255) / 256;
        hipLaunchKernelGGL(fill_zero_strided_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                           (uint16_t*)D, M, N, ldd, stride_d, batch);
        return launched();
    }
    GemmArgs g{};
    g.A = (const f16*)A;
    g.B = (const f16*)B;
    g.D = (f16*)D;
    g.M = M;
    g.N = N;
    g.K = K;
    g.lda = lda;
    g.ldb = ldb;
    g.ldd = ldd;
    g.sa = stride_a;
    g.sb = stride_b;
    g.sd = stride_d;
    g.batch = batch;
    if (skinny_pays(M, N, K, batch)) return launch_skinny(g, s);
    if (ksplit_pays(M, N, K, batch, cus)) return launch_skinny(g, s, GEMM_F16_NT_R13_KSPLIT);
    if (!fast_operands(K, lda, ldb, stride_a, stride_b, A, B, D)) return launch_any(g, s);
    return launch_ring(g, s, kDefaultRing4);
}

int64_t gemm_f16_nt_splitk_workspace(int64_t M, int64_t N, int64_t K, int splits)
{
    if (M < 0 || N < 0 || K < 0 || splits < 0 || splits > kMaxSplits) return GEMM_F16_NT_INVALID_ARG;
    int64_t s = splits, m_top = 0;
    if (s == 0) {
        int cus = 0;
        if (device_info(&cus) != GEMM_F16_NT_OK) return GEMM_F16_NT_DEVICE;
        bool r13 = false;
        s = plan_splits(M, N, K, cus, &r13);
        if (s <= 1 && !hybrid_plan(M, N, K, cus, &m_top, &s)) m_top = 0;
    }
    if (s <= 1 || K == 0 || K % 8 != 0) return 0;
    int64_t k_chunk = 0, n_slices = 0;
    split_plan(K, s, &k_chunk, &n_slices);
    return n_slices > 1 ? n_slices * (M - m_top) * N * 4 : 0;
}

int gemm_f16_nt_splitk(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D, int splits,
                       void* workspace, int64_t workspace_bytes, void* stream)
{
    if (splits < 0 || splits > kMaxSplits || workspace_bytes < 0) return GEMM_F16_NT_INVALID_ARG;
    return splitk_run(M, N, K, A, B, D, splits, workspace, workspace_bytes, false, (hipStream_t)stream);
}

int gemm_f16_nt_splitk_noalloc(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D, int splits,
                               void* stream)
{
    if (splits < 0 || splits > kMaxSplits) return GEMM_F16_NT_INVALID_ARG;
    return splitk_run(M, N, K, A, B, D, splits, nullptr, 0, true, (hipStream_t)stream);
}

int gemm_f16_nt_check_strided(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int64_t stride_a,
                              const void* B, int64_t ldb, int64_t stride_b, const void* D, int64_t ldd,
                              int64_t stride_d, int64_t batch)
{
    return validate_strided(M, N, K, A, lda, stride_a, B, ldb, stride_b, D, ldd, stride_d, batch);
}

int gemm_f16_nt_check(int rung, int64_t M, int64_t N, int64_t K, const void* A, const void* B, const void* D)
{
    return validate(rung, M, N, K, A, B, D);
}

const char* gemm_f16_nt_status_string(int status)
{
    switch (status) {
    case GEMM_F16_NT_OK: return "ok";
    case GEMM_F16_NT_INVALID_ARG: return "invalid argument";
    case GEMM_F16_NT_UNSUPPORTED: return "unsupported shape, alignment or rung";
    case GEMM_F16_NT_LAUNCH: return "kernel launch failed";
    case GEMM_F16_NT_DEVICE: return "no usable gfx950 device";
    case GEMM_F16_NT_SCRATCH: return "the split-K partial sums exceed the library's 64 MiB scratch array";
    default: return "unknown status";
    }
}

int64_t gemm_f16_nt_schedule(int64_t M, int64_t N, int64_t num_workgroups, int64_t* wg, int64_t* tile_m,
                             int64_t* tile_n, int64_t capacity)
{
    if (M < 0 || N < 0 || num_workgroups < 1 || capacity < 0) return GEMM_F16_NT_INVALID_ARG;
    if (capacity > 0 && (wg == nullptr || tile_m == nullptr || tile_n == nullptr)) return GEMM_F16_NT_INVALID_ARG;
    const int64_t tm = (M + kFastTile - 1) / kFastTile, tn = (N + kFastTile - 1) / kFastTile;
    const int64_t total = tm * tn;
    const int64_t grid = num_workgroups < total ? num_workgroups : (total > 0 ? total : 1);
    int64_t n = 0;
    for (int64_t w = 0; w < grid; ++w)
        for (int64_t i = 0;; ++i) {
            const int64_t t = persistent_tile(w, i, grid);
            if (t >= total) break;
            const TileCoord c = grouped_tile(t, tm, tn);
            if (n < capacity) {
                wg[n] = w;
                tile_m[n] = c.m_idx;
                tile_n[n] = c.n_idx;
            }
            ++n;
        }
    return n;
}

int64_t gemm_f16_nt_tile_walk(int rung, int64_t M, int64_t N, int cus, int64_t* wg, int64_t* row0, int64_t* col0,
                              int64_t capacity)
{
    if (M < 0 || N < 0 || cus < 1 || capacity < 0) return GEMM_F16_NT_INVALID_ARG;
    if (capacity > 0 && (wg == nullptr || row0 == nullptr || col0 == nullptr)) return GEMM_F16_NT_INVALID_ARG;
    const bool wide_r = rung == GEMM_F16_NT_R11_WIDE;
    const bool four_wave = rung == GEMM_F16_NT_R8_RING4_GAP || rung == GEMM_F16_NT_R10_RING4_PAIRED || wide_r;
    if (!four_wave && rung != GEMM_F16_NT_R4_RING && rung != GEMM_F16_NT_R5_PERSISTENT_WS &&
        rung != GEMM_F16_NT_R9_RING_SMALL)
        return GEMM_F16_NT_INVALID_ARG;
    if (M == 0 || N == 0) return 0;
    const bool ws_r = rung == GEMM_F16_NT_R5_PERSISTENT_WS;
    const int64_t tile = rung == GEMM_F16_NT_R9_RING_SMALL ? RingSmallCfg::BM : ws_r ? WsCfg::BN : kFastTile;
    // tile rows (M) and columns (N)
    const int64_t tile_m = wide_r ? wide::C::BM : ws_r ? WsCfg::BM : tile;
    if (four_wave && (M < tile_m || N < tile)) return GEMM_F16_NT_UNSUPPORTED;
    const int64_t tm = (M + tile_m - 1) / tile_m, tn = (N + tile - 1) / tile, total = tm * tn;
    if (total > 0x7fffffff) return GEMM_F16_NT_UNSUPPORTED;
    // the grids the launches use: one workgroup per tile (rungs 4 and 9),
    // one per compute unit or fewer (the persistent rungs)
    const int64_t grid = (rung == GEMM_F16_NT_R4_RING || rung == GEMM_F16_NT_R9_RING_SMALL) ? total
                         : (total < cus ? total : cus);
    int64_t n = 0;
    for (int64_t w = 0; w < grid; ++w)
        for (int64_t i = 0;; ++i) {
            const int64_t t = persistent_tile(w, i, grid);
            if (t >= total) break;
            int64_t r, c;
            if (four_wave) {
                uint32_t mi, ni;
                grouped_tile_in<uint32_t>((uint32_t)t, (uint32_t)tm, (uint32_t)tn,
                                          wide_r ? wide::kGroupM : ring4::kRing4GroupM, &mi, &ni);
                r = clamped_origin(mi, tile_m, M);
                c = clamped_origin(ni, tile, N);
            } else {
                const TileCoord tc = grouped_tile(t, tm, tn);
                r = tc.m_idx * tile_m;
                c = tc.n_idx * tile;
            }
            if (n < capacity) {
                wg[n] = w;
                row0[n] = r;
                col0[n] = c;
            }
            ++n;
        }
    return n;
}

int gemm_f16_nt_plan(int64_t M, int64_t N, int64_t K, int cus, int* rung_top, int64_t* m_top, int* rung_rest)
{
    if (M < 0 || N < 0 || K < 0 || cus < 1 || rung_top == nullptr || m_top == nullptr || rung_rest == nullptr)
        return GEMM_F16_NT_INVALID_ARG;
    GemmArgs g = contiguous_args(M, N, K, nullptr, nullptr, nullptr);
    *m_top = M;
    *rung_rest = 0;
    if (skinny_pays(M, N, K, 1)) {
        *rung_top = GEMM_F16_NT_R12_SKINNY;
        return GEMM_F16_NT_OK;
    }
    if (ksplit_pays(M, N, K, 1, cus)) {
        *rung_top = GEMM_F16_NT_R13_KSPLIT;
        return GEMM_F16_NT_OK;
    }
    const int64_t tiles = ((M + kFastTile - 1) / kFastTile) * ((N + kFastTile - 1) / kFastTile);
    if (K % 8 != 0) {   // R3's general form, or R9's / R4's register-staged form
        const bool small = tiles * 10 <= (int64_t)cus * kSmallTilesPer10Cus || small_tiles_pay(M, N, 1, cus);
        *rung_top = K < 8 ? GEMM_F16_NT_R3_GRID : (small ? GEMM_F16_NT_R9_RING_SMALL : GEMM_F16_NT_R4_RING);
        return GEMM_F16_NT_OK;
    }
    if (tiles * 10 <= (int64_t)cus * kSmallTilesPer10Cus) {
        *rung_top = GEMM_F16_NT_R9_RING_SMALL;
    } else if (ring4_fits(g) && wide_rows(g, cus) > 0) {
        *rung_top = GEMM_F16_NT_R11_WIDE;
        *m_top = wide_rows(g, cus);
        if (*m_top < M) *rung_rest = GEMM_F16_NT_R10_RING4_PAIRED;
    } else if (ring4_fits(g)) {
        *rung_top = GEMM_F16_NT_R10_RING4_PAIRED;
        if (round_split(g, cus, m_top))
            *rung_rest = GEMM_F16_NT_R9_RING_SMALL;
        else
            *m_top = M;
    } else {
        *rung_top = small_tiles_pay(M, N, 1, cus) ? GEMM_F16_NT_R9_RING_SMALL : GEMM_F16_NT_R4_RING;
    }
    return GEMM_F16_NT_OK;
}

int gemm_f16_nt_splitk_plan(int64_t M, int64_t N, int64_t K, int cus, int64_t* m_top, int64_t* splits)
{
    if (M < 0 || N < 0 || K < 0 || cus < 1 || m_top == nullptr || splits == nullptr) return GEMM_F16_NT_INVALID_ARG;
    *m_top = 0;
    bool r13 = false;
    *splits = plan_splits(M, N, K, cus, &r13);
    if (*splits <= 1 && !hybrid_plan(M, N, K, cus, m_top, splits)) {
        *m_top = 0;
        *splits = 1;
    }
    return GEMM_F16_NT_OK;
}

int gemm_f16_nt_ksplit_plan(int rung, int64_t M, int64_t N, int64_t K, int cus, int* mt, int* nf, int* db,
                            int* waves)
{
    if ((rung != GEMM_F16_NT_R12_SKINNY && rung != GEMM_F16_NT_R13_KSPLIT) || M < 1 || N < 1 || K < 0 || cus < 1 ||
        mt == nullptr || nf == nullptr || db == nullptr || waves == nullptr)
        return GEMM_F16_NT_INVALID_ARG;
    if (rung == GEMM_F16_NT_R12_SKINNY ? !skinny_shape(M, N, K) : !ksplit_shape(M, N, K))
        return GEMM_F16_NT_UNSUPPORTED;
    const skinny::Tile t = ksplit_tile_for(rung, M, N, K, cus);
    *mt = t.mt;
    *nf = t.nf;
    *db = t.db;
    *waves = t.nw;
    return GEMM_F16_NT_OK;
}

int gemm_f16_nt_handoff_plan(int depth, int producers, int consumers, int64_t steps, uint32_t* ready_target,
                             uint32_t* free_target)
{
    if (depth < 1 || producers < 1 || consumers < 1 || steps < 0) return GEMM_F16_NT_INVALID_ARG;
    if (steps > 0 && (ready_target == nullptr || free_target == nullptr)) return GEMM_F16_NT_INVALID_ARG;
    for (int64_t k = 0; k < steps; ++k) {
        ready_target[k] = handoff_ready_target(k, depth, producers);
        free_target[k] = handoff_free_target(k, depth, consumers);
    }
    return GEMM_F16_NT_OK;
}

int gemm_f16_nt_ring_plan(int depth, int64_t steps, int* stage, int64_t* lap, int64_t* refill)
{
    if (depth < 1 || steps < 0) return GEMM_F16_NT_INVALID_ARG;
    if (steps > 0 && (stage == nullptr || lap == nullptr || refill == nullptr)) return GEMM_F16_NT_INVALID_ARG;
    for (int64_t k = 0; k < steps; ++k) {
        stage[k] = ring_stage(k, depth);
        lap[k] = ring_lap(k, depth);
        refill[k] = ring_refill_after(k, depth, steps);
    }
    return GEMM_F16_NT_OK;
}

}  // extern "C"
