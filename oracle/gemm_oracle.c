/*
 * CPU oracle for the dense fp16 "NT" GEMM  D = A * B^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP kernels.
 *
 * What it computes (the plain definition, written out):
 *
 *   D[m][n] = round_fp16_rne( sum_{k=0}^{K-1} A[m][k] * B[n][k] ),
 *             0 <= m < M, 0 <= n < N,
 *
 * with A stored M x K row-major and B stored N x K row-major (a row-band of B
 * is a column-band of B^T).  Sources:
 *   - "GEMM I - the tiled baseline", section "The one invariant the whole
 *     ladder hangs on" and the problem statement after it: fp16 operands,
 *     accumulation in fp32, a single cast to fp16 at writeback, B kept N x K.
 *   - "TIRx GEMM detailed technical notes", V3 "Spatial Tiling with Multiple
 *     CTAs": CTA (bx, by) reads A rows m_st.., B rows n_st.. and owns
 *     D[m_st.., n_st..]  (the index roles used below).
 *   - same notes, V8 "Operand Partition" and V9 "Why Share B?": the
 *     operation is D = A B^T.
 *   - "GEMM I", Step 1 "Why accum=False": the first K tile overwrites the
 *     accumulator, so D is overwritten, never added to.
 *
 * Reading of the precision (the pages do not fix one for a checker): the
 * sum is carried in fp64.  Every fp16*fp16 product is exact in fp64 (11+11
 * significand bits), and the fp64 running sum stays ~10 orders of magnitude
 * below an fp16 ulp at the sizes used, so the result is the correctly
 * rounded fp16 value of the exact dot product except within ~1e-12 of a
 * rounding midpoint.  The single rounding goes straight from fp64 to fp16
 * (never through fp32, which would round twice).
 *
 * Rounding: IEEE round-to-nearest, ties to even.  |x| >= 65520 (the
 * midpoint between 65504 and the next step 65536) becomes +-inf; values
 * below 2^-14 round on the subnormal grid of step 2^-24 (gradual underflow).
 * The sum starts at +0.0; K = 0 therefore gives +0.0 everywhere.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ---- fp16 codec (own implementation, binary16 layout: 1 sign, 5 exponent
 * bits with bias 15, 10 fraction bits) ----------------------------------- */

double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);              /* zero / subnormal */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(frac | 0x400), expo - 25); /* 1.f * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Round a non-negative integer-valued-or-not double q to the nearest
 * integer, ties to even.  q is small (< 2^12) and exact. */
static double round_half_even(double q)
{
    double lo = floor(q);
    double diff = q - lo;                         /* exact */
    if (diff > 0.5) return lo + 1.0;
    if (diff < 0.5) return lo;
    return (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;
}

uint16_t oracle_f64_to_f16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return 0x7e00;
    double a = fabs(x);
    if (a >= 65520.0) return sign | 0x7c00;       /* overflow -> inf */
    if (a < ldexp(1.0, -14)) {
        /* subnormal grid: value = q * 2^-24, q in [0, 1024]; q == 1024 is
         * the smallest normal, whose bit pattern is exactly 0x400 */
        double q = round_half_even(ldexp(a, 24));
        return sign | (uint16_t)q;
    }
    int e2;
    frexp(a, &e2);                                /* a in [2^(e2-1), 2^e2) */
    int e = e2 - 1;                               /* unbiased exponent, -14..15 */
    double q = round_half_even(ldexp(a, 10 - e)); /* significand in [1024, 2048] */
    /* q == 2048 carries into the next binade; the sum below does that */
    unsigned bits = (unsigned)(e + 15) * 1024u + (unsigned)(q - 1024.0);
    return sign | (uint16_t)bits;
}

/* ---- the GEMM ---------------------------------------------------------- */

static double g_lut[65536];
static int g_lut_ready = 0;
static pthread_mutex_t g_lut_lock = PTHREAD_MUTEX_INITIALIZER;

static void ensure_lut(void)
{
    pthread_mutex_lock(&g_lut_lock);
    if (!g_lut_ready) {
        for (unsigned i = 0; i < 65536u; ++i) g_lut[i] = oracle_f16_to_f64((uint16_t)i);
        g_lut_ready = 1;
    }
    pthread_mutex_unlock(&g_lut_lock);
}

/* One output element: fp64 sum over k in increasing order, one rounding. */
static uint16_t dot_nt(const uint16_t *arow, const uint16_t *brow, int64_t K)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += g_lut[arow[k]] * g_lut[brow[k]];
    return oracle_f64_to_f16(acc);
}

typedef struct {
    int64_t M, N, K;
    const uint16_t *A, *B;
    uint16_t *D;
    /* full mode: rows [row0, row1); sampled mode: entries [row0, row1) */
    int64_t row0, row1;
    const int64_t *sm, *sn;
} job_t;

static void *full_worker(void *p)
{
    job_t *j = (job_t *)p;
    for (int64_t m = j->row0; m < j->row1; ++m)
        for (int64_t n = 0; n < j->N; ++n)
            j->D[m * j->N + n] = dot_nt(j->A + m * j->K, j->B + n * j->K, j->K);
    return NULL;
}

static void *sample_worker(void *p)
{
    job_t *j = (job_t *)p;
    for (int64_t i = j->row0; i < j->row1; ++i)
        j->D[i] = dot_nt(j->A + j->sm[i] * j->K, j->B + j->sn[i] * j->K, j->K);
    return NULL;
}

static int resolve_threads(int nthreads, int64_t work_items)
{
    if (nthreads <= 0) {
        long c = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = c > 0 ? (int)c : 1;
    }
    if (nthreads > 256) nthreads = 256;
    if (work_items < nthreads) nthreads = work_items > 0 ? (int)work_items : 1;
    return nthreads;
}

static int run_split(void *(*fn)(void *), job_t base, int64_t items, int nthreads)
{
    pthread_t th[256];
    job_t jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].row0 = items * t / nthreads;
        jobs[t].row1 = items * (t + 1) / nthreads;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, fn, &jobs[t]) != 0) break;
        started = t;
    }
    fn(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    /* any job whose thread failed to start runs here */
    for (int t = started + 1; t < nthreads; ++t) fn(&jobs[t]);
    return nthreads;
}

/* Full product.  A: M*K fp16 bits, B: N*K, D: M*N (overwritten).
 * nthreads <= 0 means one thread per online core.  Returns threads used. */
int oracle_gemm_nt(int64_t M, int64_t N, int64_t K, const uint16_t *A,
                   const uint16_t *B, uint16_t *D, int nthreads)
{
    ensure_lut();
    job_t base = {M, N, K, A, B, D, 0, 0, NULL, NULL};
    int nt = resolve_threads(nthreads, M);
    if (M <= 0 || N <= 0) return nt;
    return run_split(full_worker, base, M, nt);
}

/* Selected elements only: out[i] = D[sm[i]][sn[i]].  Returns threads used. */
int oracle_gemm_nt_sampled(int64_t M, int64_t N, int64_t K, const uint16_t *A,
                           const uint16_t *B, int64_t count, const int64_t *sm,
                           const int64_t *sn, uint16_t *out, int nthreads)
{
    ensure_lut();
    for (int64_t i = 0; i < count; ++i)
        if (sm[i] < 0 || sm[i] >= M || sn[i] < 0 || sn[i] >= N) return -1;
    job_t base = {M, N, K, A, B, out, 0, 0, sm, sn};
    int nt = resolve_threads(nthreads, count);
    if (count <= 0) return nt;
    return run_split(sample_worker, base, count, nt);
}

/* Array forms of the codec, for the self-tests. */
void oracle_f16_to_f64_n(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(h[i]);
}

void oracle_f64_to_f16_n(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_f16(x[i]);
}
