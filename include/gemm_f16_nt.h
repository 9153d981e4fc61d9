/*
 * gemm_f16_nt -- dense fp16 GEMM  D = A * B^T  on AMD Instinct MI355X (gfx950).
 *
 * The operation ("GEMM I - the tiled baseline", problem statement; "TIRx GEMM
 * detailed technical notes", V3 "Spatial Tiling with Multiple CTAs" and V8
 * "Operand Partition"):
 *
 *     D[m][n] = fp16( sum_k A[m][k] * B[n][k] ),   0 <= m < M, 0 <= n < N
 *
 *   A  M x K fp16, row-major (leading dimension K)
 *   B  N x K fp16, row-major (leading dimension K) -- B is stored N x K so
 *      both operands stream as K-contiguous row bands
 *   D  M x N fp16, row-major (leading dimension N), fully overwritten
 *
 * Products accumulate in fp32 and are rounded to fp16 once, at writeback,
 * round-to-nearest-even; magnitudes >= 65520 become +-inf.  D is
 * overwritten, never accumulated into (the first K step starts the sum,
 * "GEMM I", Step 1 "Why accum=False").  The fp32 summation order is the
 * kernel's own and is not part of the contract.
 *
 * Pointers: A, B and D are device pointers (HIP device memory of the current
 * device).  The caller owns them; the library never frees, retains or
 * allocates memory.  They must be 2-byte (fp16) aligned.  D must not
 * overlap A or B.  `stream` is a hipStream_t (NULL = the null stream).
 *
 * Calls are asynchronous and stream-ordered: they validate, enqueue and
 * return.  Validation happens before any HIP call, so an invalid call
 * launches nothing and leaves D untouched.  Faults inside a kernel surface
 * at the caller's next synchronisation of the stream.
 *
 * Shapes: M, N, K >= 0.  M = 0 or N = 0 is a no-op; K = 0 writes +0.0 to
 * all of D.  The fastest kernels need every operand row to start on a
 * 16-byte boundary (K % 8 == 0 and A, B, D 16-byte aligned).  Other
 * operands (any 2-byte aligned A, B, D) run on the library's choice, rung 3,
 * and rungs 4 and 9 for K >= 8: rungs 4 and 9 then stage their loads
 * through registers (about two thirds of the aligned speed), rung 3 copies
 * operands element by element (several times slower; the library's choice
 * for K < 8).  The result contract is the same.
 *
 * Return value: GEMM_F16_NT_OK (0) or a negative status below.
 */
#ifndef GEMM_F16_NT_H
#define GEMM_F16_NT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GEMM_F16_NT_OK 0
#define GEMM_F16_NT_INVALID_ARG (-1) /* negative size, null pointer with data, unknown or removed rung, overlap */
#define GEMM_F16_NT_UNSUPPORTED (-2) /* shape or alignment a rung does not implement, odd addresses */
#define GEMM_F16_NT_LAUNCH (-3)      /* the HIP launch itself failed */
#define GEMM_F16_NT_DEVICE (-4)      /* no usable device / device query failed / not gfx950 */
#define GEMM_F16_NT_SCRATCH (-5)     /* gemm_f16_nt_splitk_noalloc: partial sums beyond its scratch array */

/* The ladder of kernels ("GEMM I", Steps 1-3; "GEMM III", Step 7; "TIRx
 * GEMM detailed technical notes", V1-V7).  Every rung computes the same D. */
#define GEMM_F16_NT_R1_SINGLE_TILE 1 /* M = N = 128, K = 64 only, one workgroup */
#define GEMM_F16_NT_R2_KLOOP 2       /* M = N = 128, any K: K-loop into one accumulator */
#define GEMM_F16_NT_R3_GRID 3        /* any shape and alignment: 2D grid of 128 x 128 tiles */
#define GEMM_F16_NT_R4_RING 4        /* any shape: 256 x 256 tiles, direct-to-LDS pipelined ring
                                        (loads staged through registers on rows off 16-byte
                                        boundaries, K >= 8) */
#define GEMM_F16_NT_R5_PERSISTENT_WS 5 /* any shape: persistent, producer/consumer waves */
/* Rungs 6 and 7 (earlier forms of rung 8: one barrier per k step, then a
 * release and a publish barrier with clumped instructions) were removed;
 * their numbers are not reused and return GEMM_F16_NT_INVALID_ARG. */
#define GEMM_F16_NT_R8_RING4_GAP 8 /* rung 4's ring with 4 waves of 128 x 128 on 16x16x32 MFMAs, a generated
                                      instruction schedule with a release and a publish barrier per k step
                                      and at most one instruction between two MFMAs, persistent: M, N >=
                                      256, N a multiple of 8 and under 2^24, K a multiple of 64, K >= 128
                                      (when M or N is not a multiple of 256 the last tile row or column ends
                                      at M or N and overlaps its neighbour) */
#define GEMM_F16_NT_R9_RING_SMALL 9 /* any shape: rung 4's ring with 128 x 128 tiles, 8 waves of 64 x 32 and
                                       4 stages (the same register staging on general rows); the
                                       library's choice when 256 x 256 tiles would number at most 0.4
                                       per compute unit, and, off the four-wave ring, where its tiles
                                       take fewer rounds of the compute units than rung 4's */
#define GEMM_F16_NT_R10_RING4_PAIRED 10 /* rung 8 with each 16 x 16 block's two 32-wide sub-steps issued
                                           back to back into its accumulator; the shapes of rung 8 with
                                           any N >= 256 (rows of D on any 2-byte boundary), and also K a
                                           multiple of 8 above 64 that is not a multiple of 64 (the
                                           partial k step goes first; rows of A and B then shorter than
                                           2^21 elements); the library's choice for those shapes */

#define GEMM_F16_NT_R11_WIDE 11 /* rung 10's four-wave ring on 384 x 256 tiles (each staged B band feeds
                                   two waves of 192 A rows: a sixth fewer operand bytes per FLOP; "GEMM
                                   III", Step 9, and "TIRx GEMM detailed technical notes", V9 "Why Share
                                   B?"), one barrier per k step: M >= 384, N >= 256, K a multiple of 64,
                                   K >= 128, N < 2^23 (the last tile row or column ends at M or N and
                                   overlaps its neighbour); the library's choice, on every row or on the
                                   top rows, where its rounds of tiles cost less than rung 10's */
#define GEMM_F16_NT_R12_SKINNY 12 /* one side of at most 96 rows (M <= 96 or N <= 96), K >= 8, rows on
                                     any 2-byte boundary: each workgroup owns 16 or 32 rows of the large
                                     side and all of the small side, its 8 waves split K, and their fp32
                                     partial sums are added in LDS before the one rounding (no
                                     workspace); the library's choice for single products whose small
                                     side has at most 32 rows, at most 64 with a large side of at most
                                     16384 rows, or at most 96 with a large side of at most 12288 */
#define GEMM_F16_NT_R13_KSPLIT 13 /* rung 12's kernel on a 2-D grid of small tiles (16-96 rows of the
                                     side with fewer rows by 16-64 rows of the other, picked by a
                                     model of the tile's load time), any M, N >= 1 and K >= 8, rows on
                                     any 2-byte boundary, no workspace; the library's choice for single
                                     products that rung 12 does not take and whose 128- and 256-row
                                     tiles would leave most compute units idle over a long K, where
                                     that model is at most 0.87 of the ring's (gemm_f16_nt_plan) */

/* D = A * B^T with the library's choice of kernel for the shape (see
 * gemm_f16_nt_plan; products with one small side run on rung 12, and
 * products with few tiles and a long K on rung 13).  Some
 * shapes take two launches on the stream: when
 * the 256 x 256 tiles leave a small last round, the rows past the whole
 * rounds run on 128 x 128 tiles; when whole rounds of 384 x 256 tiles fit
 * over the top rows but not over all of them, the top rows run on rung 11
 * and the rest on rung 10. */
int gemm_f16_nt(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D, void* stream);

/* The same product on one named rung of the ladder (for tests and the
 * bench).  Returns GEMM_F16_NT_UNSUPPORTED if the rung does not implement
 * the shape (R1 and R2 are single-tile rungs). */
int gemm_f16_nt_rung(int rung, int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D,
                     void* stream);

/* Persistent rung R5 with an explicit number of workgroups (>= 1) instead
 * of one per compute unit.  The result must not depend on it; tests use it
 * to check that every grid size gives identical bits. */
int gemm_f16_nt_persistent(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D,
                           int64_t num_workgroups, void* stream);

/* Strided, batched form (general leading dimensions; "GEMM I" claims any
 * M, N, K, and the batch covers per-head products such as attention
 * scores Q*K^T, the bridge to attention at the end of "GEMM III"):
 *
 *   for b in [0, batch):  D_b = A_b * B_b^T
 *     A_b = A + b*stride_a, M x K, row r at A_b + r*lda
 *     B_b = B + b*stride_b, N x K, row r at B_b + r*ldb
 *     D_b = D + b*stride_d, M x N, row r at D_b + r*ldd
 *
 * All leading dimensions and strides are in elements (fp16).  lda, ldb >= K;
 * stride_a, stride_b >= 0 (0 repeats one operand for every batch entry);
 * ldd >= N; stride_d >= 0, and for batch > 1 at least (M-1)*ldd + N so the
 * outputs do not overlap.  With K, lda, ldb, stride_a, stride_b multiples
 * of 8 and 16-byte aligned A, B and D the fastest kernels run; otherwise
 * the register-staged ring (K >= 8) or R3's general form (K < 8, which also
 * limits batch to 65535).  Same precision, rounding, ownership and error
 * behaviour as gemm_f16_nt. */
int gemm_f16_nt_strided_batched(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int64_t stride_a,
                                const void* B, int64_t ldb, int64_t stride_b, void* D, int64_t ldd,
                                int64_t stride_d, int64_t batch, void* stream);

/* Split-K form for products with fewer output tiles than compute units
 * (the persistent scheduler of "TIRx GEMM detailed technical notes", V6,
 * has nothing to balance when a shape has a handful of tiles): K is cut
 * into `splits` slices of whole 64-wide steps (0 = the library's choice,
 * at most 64), each slice's fp32 partial sums go to `workspace`, and a
 * second kernel adds the slices in slice order and rounds once to fp16 --
 * the single rounding at writeback is kept.  With splits = 0 the library
 * also splits products whose 256 x 256 tiles fill whole rounds of the
 * compute units plus a small last round: the top rows that fill the whole
 * rounds run unsplit and only the remaining rows split K.  The fp32 summation order
 * differs from gemm_f16_nt's (any order is within the contract).
 * `workspace` is caller-owned device memory of at least
 * gemm_f16_nt_splitk_workspace(M, N, K, splits) bytes, 16-byte aligned,
 * not overlapping A, B or D; its contents are scratch.  With splits = 0 the
 * library compares models of the slices, of rung 13 and of the ring kernels
 * and may run one launch instead: rung 13 where it is modeled fastest,
 * otherwise gemm_f16_nt's choice; then, as for one slice or operand rows
 * off 16-byte boundaries (see above), the workspace is not touched. */
int gemm_f16_nt_splitk(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D, int splits,
                       void* workspace, int64_t workspace_bytes, void* stream);

/* gemm_f16_nt_splitk without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The fp32 partial sums go to a scratch array of 64 MiB (67108864 bytes)
 * that the library holds in device memory, one per device, for the life of
 * the process (its address is taken on the first call on each device).
 * Same arguments, kernel choice, slice plan and result bits as
 * gemm_f16_nt_splitk with `splits`; where that call would need more than
 * 64 MiB of workspace (gemm_f16_nt_splitk_workspace), this one returns
 * GEMM_F16_NT_SCRATCH and launches nothing (with an explicit `splits` that
 * is decided before any HIP call).  Every call on one device shares that
 * device's array: calls that may overlap on one device (on different
 * streams, or from different threads without ordering) race and may write
 * wrong results; calls ordered on one stream do not.  Nothing in the array
 * needs clearing between calls: every slice overwrites its partial sums
 * before the reduction reads them. */
int gemm_f16_nt_splitk_noalloc(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* D, int splits,
                               void* stream);

/* Bytes of workspace gemm_f16_nt_splitk needs (0 if it will not split), or
 * a negative status.  With splits = 0 this queries the current device's
 * compute-unit count (the only HIP call). */
int64_t gemm_f16_nt_splitk_workspace(int64_t M, int64_t N, int64_t K, int splits);

/* Validation only for the strided form, no HIP call. */
int gemm_f16_nt_check_strided(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int64_t stride_a,
                              const void* B, int64_t ldb, int64_t stride_b, const void* D, int64_t ldd,
                              int64_t stride_d, int64_t batch);

/* Validation only, no HIP call: the status the call above would return for
 * these arguments before launching anything (rung 0 = gemm_f16_nt). */
int gemm_f16_nt_check(int rung, int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                      const void* D);

/* Static description of a status code (never NULL). */
const char* gemm_f16_nt_status_string(int status);

/* Host evaluation of the persistent rung's tile schedule, no HIP call.  For
 * a grid of `num_workgroups` on an M x N output (256 x 256 tiles), writes
 * one entry per (workgroup, visit) in workgroup-major visit order:
 * wg[i], tile_m[i], tile_n[i].  Returns the number of entries (the tile
 * count) or a negative status; writes at most `capacity` entries. */
int64_t gemm_f16_nt_schedule(int64_t M, int64_t N, int64_t num_workgroups, int64_t* wg, int64_t* tile_m,
                             int64_t* tile_n, int64_t capacity);

/* Host evaluation of the tile walk a rung's launch runs on a device with
 * `cus` compute units, no HIP call ("TIRx GEMM detailed technical notes",
 * V3 "Spatial Tiling with Multiple CTAs" for the tile origins, V6 "Better
 * L2 Locality" for the grouped order).  rung: 4 and 9 (one workgroup per
 * 256 x 256 or 128 x 128 tile, grouped order with groups of 8 tile rows),
 * 5 (persistent, one workgroup per compute unit, the same order) or 8,
 * 10 and 11 (the four-wave ring: persistent, groups of 4 tile rows, the
 * last tile row and column moved back to end at M and N; tiles of 256 x
 * 256, 384 x 256 for rung 11; M, N at least one tile, else
 * GEMM_F16_NT_UNSUPPORTED).  Writes one entry per tile visit in
 * workgroup-major visit order: workgroup wg[i] computes the output block
 * whose first row is row0[i] and first column col0[i].  Returns the number
 * of entries or a negative status; writes at most `capacity` entries. */
int64_t gemm_f16_nt_tile_walk(int rung, int64_t M, int64_t N, int cus, int64_t* wg, int64_t* row0, int64_t* col0,
                              int64_t capacity);

/* Host evaluation of the operand ring's bookkeeping for `depth` stages and
 * `steps` k steps: stage[k], lap[k] (the pages' phase is lap & 1) and
 * refill[k] = the step loaded into stage[k] once step k is consumed (-1 if
 * none).  Returns 0 or a negative status. */
int gemm_f16_nt_ring_plan(int depth, int64_t steps, int* stage, int64_t* lap, int64_t* refill);
/* Host evaluation of rung 5's producer/consumer handoff ("GEMM III",
 * Step 7 "Four barriers = two producer-consumer rings"), no HIP call: each
 * ring stage has a ready and a free counter in LDS that never reset;
 * every producer wave adds 1 to ready[k % depth] once its loads of step k
 * have landed, every consumer wave adds 1 to free[k % depth] once it has
 * read step k.  For each k step, writes the count a consumer waits for
 * before reading it (ready_target[k]) and the count a producer waits for
 * before refilling its stage with it (free_target[k]).  Returns 0 or a
 * negative status. */
int gemm_f16_nt_handoff_plan(int depth, int producers, int consumers, int64_t steps, uint32_t* ready_target,
                             uint32_t* free_target);
/* Host evaluation of gemm_f16_nt's kernel choice for contiguous, 16-byte
 * aligned operands on a device with `cus` compute units, no HIP call: rows
 * [0, *m_top) run on rung *rung_top and rows [*m_top, M) on rung
 * *rung_rest (0 and *m_top = M when one kernel takes every row).  For
 * K % 8 != 0 rungs 4 and 9 stand for their register-staged forms and
 * rung 3 for its general form; rungs 12 and 13 take any K >= 8.  Returns 0
 * or a negative status. */
int gemm_f16_nt_plan(int64_t M, int64_t N, int64_t K, int cus, int* rung_top, int64_t* m_top, int* rung_rest);
/* Host evaluation of gemm_f16_nt_splitk's choice for `splits` = 0 on a
 * device with `cus` compute units, no HIP call: *m_top rows (0 or a
 * multiple of 256) run unsplit, the other M - *m_top rows split K into
 * *splits slices (1: no split).  Returns 0 or a negative status. */
int gemm_f16_nt_splitk_plan(int64_t M, int64_t N, int64_t K, int cus, int64_t* m_top, int64_t* splits);
/* Host evaluation of the workgroup tile rung 12 or 13 (`rung`) launches for
 * an M x N x K product on a device with `cus` compute units, no HIP call:
 * 16 * *mt rows of the side with fewer rows (A on a tie), 16 * *nf rows of
 * the other, *db groups of 128 k elements in flight per wave, and *waves
 * waves (8, or 4 on two of rung 13's tiles) splitting K.  Returns 0,
 * GEMM_F16_NT_INVALID_ARG (another rung, M or N < 1, null outputs) or
 * GEMM_F16_NT_UNSUPPORTED (a shape the rung does not take). */
int gemm_f16_nt_ksplit_plan(int rung, int64_t M, int64_t N, int64_t K, int cus, int* mt, int* nf, int* db,
                            int* waves);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F16_NT_H */
