/*
 * The library used from plain C through include/fa.h alone: device buffers
 * from hipMalloc, fa_fwd on a stream, results copied back and compared with
 * the fp64 oracle (test infrastructure, linked here as liboracle.so).
 *
 * With the argument "args" it only checks that bad arguments come back as
 * the documented status codes (no GPU needed).
 *
 * Inputs come from the seeded C generator (include/fa_gen.h: N(0,1) values
 * rounded to the storage type on the host), streams 0/1/2 for Q/K/V.  Exit
 * status 0 when every case meets its bar:
 * 16-bit O max-abs <= 2e-2, mean-abs <= 2e-3, lse max-abs <= 1e-3; fp32 O and
 * lse within 1e-5 relative (to max|O| and max(1, max|lse|)).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fa.h"
#include "fa_gen.h"
#include "fa_oracle.h"

#define HIP_OK(x)                                                          \
    do {                                                                   \
        hipError_t e_ = (x);                                               \
        if (e_ != hipSuccess) {                                            \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_)); \
            exit(2);                                                       \
        }                                                                  \
    } while (0)

static float bf16_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static int run_case(int dtype, int B, int H, int L, int d, int causal, float scale, uint64_t seed) {
    const size_t n = (size_t)B * H * L * d, rows = (size_t)B * H * L;
    const size_t esz = dtype == FA_F32 ? 4 : 2;
    void* host[3];
    for (int t = 0; t < 3; ++t) {
        host[t] = malloc(n * esz);
        if (fa_gen_fill(host[t], dtype, n, seed, (uint64_t)t, 1.0) != 0) {
            fprintf(stderr, "fa_gen_fill rejected the case\n");
            return 1;
        }
    }
    void *q, *k, *v, *o;
    float* lse;
    HIP_OK(hipMalloc(&q, n * esz));
    HIP_OK(hipMalloc(&k, n * esz));
    HIP_OK(hipMalloc(&v, n * esz));
    HIP_OK(hipMalloc(&o, n * esz));
    HIP_OK(hipMalloc((void**)&lse, rows * 4));
    HIP_OK(hipMemcpy(q, host[0], n * esz, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(k, host[1], n * esz, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v, host[2], n * esz, hipMemcpyHostToDevice));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    const int rc = fa_fwd(q, k, v, o, lse, B, H, L, d, scale, causal, dtype, stream);
    if (rc != FA_OK) {
        fprintf(stderr, "fa_fwd returned %d (%s)\n", rc, fa_strerror(rc));
        return 1;
    }
    HIP_OK(hipStreamSynchronize(stream));
    void* o_h = malloc(n * esz);
    float* lse_h = (float*)malloc(rows * 4);
    HIP_OK(hipMemcpy(o_h, o, n * esz, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse_h, lse, rows * 4, hipMemcpyDeviceToHost));

    double* o_ref = (double*)malloc(n * 8);
    double* lse_ref = (double*)malloc(rows * 8);
    const int odt = dtype == FA_F32 ? ORACLE_F32 : ORACLE_BF16;
    if (fa_oracle_fwd(host[0], host[1], host[2], odt, B, H, L, d, scale, causal, NULL, L, o_ref, lse_ref, 0) != 0) {
        fprintf(stderr, "oracle rejected the case\n");
        return 1;
    }
    double emax = 0, esum = 0, omax = 0, lmax = 0, lref = 1;
    for (size_t i = 0; i < n; ++i) {
        const double g = dtype == FA_F32 ? ((float*)o_h)[i] : bf16_to_float(((uint16_t*)o_h)[i]);
        const double e = fabs(g - o_ref[i]);
        if (!(e == e)) emax = INFINITY;
        emax = e > emax ? e : emax;
        esum += e;
        omax = fabs(o_ref[i]) > omax ? fabs(o_ref[i]) : omax;
    }
    for (size_t i = 0; i < rows; ++i) {
        const double e = fabs((double)lse_h[i] - lse_ref[i]);
        lmax = (e > lmax || !(e == e)) ? e : lmax;
        lref = fabs(lse_ref[i]) > lref ? fabs(lse_ref[i]) : lref;
    }
    int ok;
    if (dtype == FA_F32) ok = emax <= 1e-5 * omax && lmax <= 1e-5 * lref;
    else ok = emax <= 2e-2 && esum / n <= 2e-3 && lmax <= 1e-3;
    printf("[c] fa_fwd %s B=%d H=%d L=%d d=%d causal=%d: O max abs %.3e mean abs %.3e, lse max abs %.3e: %s\n",
           dtype == FA_F32 ? "fp32" : "bf16", B, H, L, d, causal, emax, esum / n, lmax, ok ? "ok" : "FAIL");
    fflush(stdout);
    HIP_OK(hipStreamDestroy(stream));
    HIP_OK(hipFree(q));
    HIP_OK(hipFree(k));
    HIP_OK(hipFree(v));
    HIP_OK(hipFree(o));
    HIP_OK(hipFree(lse));
    for (int t = 0; t < 3; ++t) free(host[t]);
    free(o_h);
    free(lse_h);
    free(o_ref);
    free(lse_ref);
    return ok ? 0 : 1;
}

/* "args": only the argument checks, which need no GPU */
int main(int argc, char** argv) {
    const int args_only = argc > 1 && strcmp(argv[1], "args") == 0;
    int fails = 0;
    /* argument errors come back before anything is enqueued */
    const int e1 = fa_fwd(NULL, NULL, NULL, NULL, NULL, 1, 1, 1, 64, 1.f, 0, FA_BF16, 0);
    const int e2 = fa_fwd((void*)256, (void*)256, (void*)256, (void*)256, (float*)256, 1, 1, 1, 96, 1.f, 0, FA_BF16, 0);
    printf("[c] null pointers -> %d (%s); d = 96 -> %d (%s)\n", e1, fa_strerror(e1), e2, fa_strerror(e2));
    if (e1 != FA_ERR_INVALID_ARG || e2 != FA_ERR_UNSUPPORTED) ++fails;
    if (args_only) return fails ? 1 : 0;
    fails += run_case(FA_BF16, 1, 2, 300, 128, 1, 0.088388f, 1);
    fails += run_case(FA_BF16, 2, 3, 129, 64, 0, 0.125f, 2);
    fails += run_case(FA_F32, 1, 1, 77, 64, 0, 0.125f, 3);
    printf("[c] %s\n", fails ? "FAILED" : "all cases passed");
    return fails ? 1 : 0;
}
