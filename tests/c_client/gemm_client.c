/*
 * A plain C caller of the library's C-ABI (include/gemm_f16_nt.h): device
 * memory and a stream from the HIP runtime, one gemm_f16_nt call per shape,
 * the result checked on the host.  The operands are -1, 0 or 1 with
 * K <= 2048, so every product sum is an integer of magnitude at most 2048,
 * exact in fp32 and in fp16: the check is bitwise against the integer sums.  It also checks an invalid call's status and
 * that it leaves D untouched.  Prints "ok" and exits 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "gemm_f16_nt.h"

/* fp16 bits of a small integer (|v| <= 2048): exact. */
static uint16_t f16_of_int(int v)
{
    if (v == 0) return 0;
    uint16_t sign = v < 0 ? 0x8000 : 0;
    unsigned m = (unsigned)(v < 0 ? -v : v);
    int e = 0;
    while ((m >> e) > 1) ++e;                       /* 2^e <= m < 2^(e+1) */
    unsigned frac = (m << (10 - e)) & 0x3ff;        /* exact for m < 2048 */
    return (uint16_t)(sign | ((e + 15) << 10) | frac);
}

#define CHECK_HIP(x)                                                     \
    do {                                                                 \
        hipError_t err_ = (x);                                           \
        if (err_ != hipSuccess) {                                        \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(err_));    \
            return 2;                                                    \
        }                                                                \
    } while (0)

static int run_shape(int rung, int64_t M, int64_t N, int64_t K, hipStream_t s)
{
    size_t na = (size_t)(M * K), nb = (size_t)(N * K), nd = (size_t)(M * N);
    uint16_t* a = malloc(na * 2);
    uint16_t* b = malloc(nb * 2);
    uint16_t* d = malloc(nd * 2);
    int* ai = malloc(na * sizeof(int));
    int* bi = malloc(nb * sizeof(int));
    if (!a || !b || !d || !ai || !bi) return 2;
    for (size_t i = 0; i < na; ++i) {
        ai[i] = (int)((i * 7 + i / 13) % 3) - 1;
        a[i] = f16_of_int(ai[i]);
    }
    for (size_t i = 0; i < nb; ++i) {
        bi[i] = (int)((i * 5 + i / 11) % 3) - 1;
        b[i] = f16_of_int(bi[i]);
    }
    void *da, *db, *dd;
    CHECK_HIP(hipMalloc(&da, na * 2));
    CHECK_HIP(hipMalloc(&db, nb * 2));
    CHECK_HIP(hipMalloc(&dd, nd * 2));
    CHECK_HIP(hipMemcpyAsync(da, a, na * 2, hipMemcpyHostToDevice, s));
    CHECK_HIP(hipMemcpyAsync(db, b, nb * 2, hipMemcpyHostToDevice, s));
    CHECK_HIP(hipMemsetAsync(dd, 0xff, nd * 2, s));             /* NaN everywhere */
    int st = rung == 0 ? gemm_f16_nt(M, N, K, da, db, dd, (void*)s)
                       : gemm_f16_nt_rung(rung, M, N, K, da, db, dd, (void*)s);
    if (st != GEMM_F16_NT_OK) {
        fprintf(stderr, "rung %d, %ld x %ld x %ld: %s\n", rung, (long)M, (long)N, (long)K,
                gemm_f16_nt_status_string(st));
        return 1;
    }
    CHECK_HIP(hipMemcpyAsync(d, dd, nd * 2, hipMemcpyDeviceToHost, s));
    CHECK_HIP(hipStreamSynchronize(s));
    long bad = 0;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            long sum = 0;
            for (int64_t k = 0; k < K; ++k) sum += (long)ai[m * K + k] * bi[n * K + k];
            if (d[m * N + n] != f16_of_int((int)sum) && bad++ < 5)
                fprintf(stderr, "D[%ld][%ld] = 0x%04x, want %ld (0x%04x)\n", (long)m, (long)n, d[m * N + n], sum,
                        f16_of_int((int)sum));
        }
    /* an invalid call (negative K) returns its status and writes nothing */
    st = gemm_f16_nt(M, N, -1, da, db, dd, (void*)s);
    CHECK_HIP(hipMemcpyAsync(a, dd, 2, hipMemcpyDeviceToHost, s));
    CHECK_HIP(hipStreamSynchronize(s));
    if (st != GEMM_F16_NT_INVALID_ARG || a[0] != d[0]) {
        fprintf(stderr, "invalid call: status %d\n", st);
        return 1;
    }
    CHECK_HIP(hipFree(da));
    CHECK_HIP(hipFree(db));
    CHECK_HIP(hipFree(dd));
    free(a); free(b); free(d); free(ai); free(bi);
    if (bad) {
        fprintf(stderr, "%ld wrong outputs at %ld x %ld x %ld\n", bad, (long)M, (long)N, (long)K);
        return 1;
    }
    printf("rung %d, %ld x %ld x %ld: every output exact\n", rung, (long)M, (long)N, (long)K);
    return 0;
}

int main(void)
{
    hipStream_t s;
    CHECK_HIP(hipStreamCreate(&s));
    /* the library's choice: the four-wave ring (ragged M and N, partial
     * first k step) and 128 x 128 tiles; rungs 11 and 5 by name */
    const int64_t shapes[][4] = {{0, 300, 520, 1000}, {0, 100, 130, 1000}, {11, 400, 300, 1024}, {5, 260, 300, 2048}};
    for (int i = 0; i < 4; ++i) {
        int r = run_shape((int)shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], s);
        if (r) return r;
    }
    CHECK_HIP(hipStreamDestroy(s));
    printf("ok\n");
    return 0;
}
