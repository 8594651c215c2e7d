/*
 * c_abi_check.c -- a plain C99 consumer of libmxfp4.so through include/mxfp4.h
 * (test infrastructure; built and run by tests/test_c_abi.py).
 *
 *   c_abi_check host   host-only entry points: size queries, plans, errors;
 *   c_abi_check gpu    one GEMM on the GPU through the HIP runtime's C API:
 *                      B quantized by the CPU oracle (liboracle.so) and
 *                      repacked by mxfp4_pack_b, A quantized by the library
 *                      inside mxfp4_gemm; C checked against the oracle's fp32
 *                      sum elementwise (|d| <= 1e-2 |ref| + 1e-2),
 *                      mxfp4_quant_a's bytes against the oracle's, exactly,
 *                      and mxfp4_gemm_noalloc's C against mxfp4_gemm's, bit
 *                      for bit.
 *
 * Exit status 0 when every check holds; a message names the first failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "mxfp4.h"

/* the oracle's C entry points (oracle/mxfp4_oracle.c) */
int oracle_quantize_rows(const uint16_t *x, int64_t rows, int64_t K, int64_t ld, uint8_t *fp4,
                         uint8_t *scale);
int oracle_dequantize(const uint8_t *fp4, const uint8_t *scale, int64_t rows, int64_t K,
                      double *out);
int oracle_gemm(const double *a_deq, const double *b_deq, int64_t M, int64_t N, int64_t K,
                float *c32, double *c64);

#define CHECK(cond, ...)                                \
    do {                                                \
        if (!(cond)) {                                  \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);               \
            fputc('\n', stderr);                        \
            return 1;                                   \
        }                                               \
    } while (0)
#define HIP(call) CHECK((call) == hipSuccess, "%s", #call)

/* bf16 bits of a value in roughly N(0,1): sum of uniforms, rounded to
 * nearest even (a fixed-seed xorshift; the inputs only need to be varied) */
static uint32_t rng_state = 12345u;
static uint32_t xorshift(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return rng_state;
}
static uint16_t rand_bf16(void) {
    float x = -6.0f;
    for (int i = 0; i < 12; ++i) x += (float)(xorshift() >> 8) / 16777216.0f;
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static int host_checks(void) {
    CHECK(mxfp4_packed_bytes(32, 512) == (size_t)2 * 4 * 1024 + (size_t)2 * 1 * 256,
          "packed bytes of 32 x 512");
    CHECK(mxfp4_packed_bytes(0, 512) == 0, "packed bytes of 0 rows");
    CHECK(mxfp4_packed_bytes(16, 100) == 0, "packed bytes, K not a multiple of 32");
    mxfp4_plan p;
    CHECK(mxfp4_default_plan(32, 4096, 512, &p) == MXFP4_OK, "default plan");
    CHECK(mxfp4_check_plan(&p, 32, 4096, 512) == MXFP4_OK, "default plan checks");
    CHECK(mxfp4_default_plan(32, 4096, 100, &p) == MXFP4_EINVAL, "K not a multiple of 32 refused");
    CHECK(strlen(mxfp4_last_error()) > 0, "error text set");
    CHECK(mxfp4_default_plan(32, 4096, 512, NULL) == MXFP4_ENULL, "NULL plan refused");
    CHECK(mxfp4_gemm(NULL, 512, NULL, 0, NULL, 4096, 32, 4096, 512, NULL, 0, NULL) == MXFP4_ENULL,
          "NULL pointers refused before any launch");
    CHECK(mxfp4_gemm(NULL, 512, NULL, 0, NULL, 4096, 0, 4096, 512, NULL, 0, NULL) == MXFP4_OK,
          "an empty call (M = 0) returns at once");
    CHECK(mxfp4_quant_a(NULL, 0, 512, 512, NULL, 256, NULL, 16, NULL) == MXFP4_OK,
          "an empty quantization returns at once");
    /* plan fields far out of range are refused without overflowing the
     * checks' arithmetic (the sanitizer build traps signed overflow) */
    mxfp4_plan huge = p; /* K = 512: 4 steps of 128 */
    huge.waves_n = 1 << 30;
    huge.waves_k = 4;
    huge.k_steps_per_wave = 1;
    huge.split_k = 1;
    CHECK(mxfp4_check_plan(&huge, 32, 4096, 512) == MXFP4_EINVAL, "huge waves_n refused");
    huge.waves_n = 2;
    huge.waves_k = 1 << 30;
    huge.k_steps_per_wave = 4;
    huge.split_k = 1 << 30;
    CHECK(mxfp4_check_plan(&huge, 32, 4096, 512) == MXFP4_EINVAL, "huge waves_k and split refused");
    huge = p;
    huge.split_k = 0x7FFFFFFF;
    CHECK(mxfp4_check_plan(&huge, 32, 4096, 512) == MXFP4_EINVAL, "huge split refused");
    huge.split_reduce = MXFP4_REDUCE_ATOMIC;
    CHECK(mxfp4_plan_workspace_bytes(&huge, 32, 4096, 512) == 0, "no workspace for a huge split");
    CHECK(mxfp4_gemm_noalloc(NULL, 512, NULL, 0, NULL, 4096, 32, 4096, 512, NULL) == MXFP4_ENULL,
          "noalloc: NULL pointers refused");
    CHECK(mxfp4_gemm_noalloc_max_scratch_bytes() == ((size_t)16 << 20), "noalloc scratch size");
    printf("host checks ok\n");
    return 0;
}

static int gpu_check(void) {
    const int M = 48, N = 272, K = 640; /* ragged against 128-K steps: 5 steps */
    const size_t na = (size_t)M * K, nb = (size_t)N * K;
    uint16_t *a = malloc(na * 2), *b = malloc(nb * 2), *c = malloc((size_t)M * N * 2);
    uint8_t *aq = malloc(na / 2), *as = malloc(na / 32), *bq = malloc(nb / 2), *bs = malloc(nb / 32);
    uint8_t *gq = malloc(na / 2), *gs = malloc(na / 32);
    double *ad = malloc(na * sizeof(double)), *bd = malloc(nb * sizeof(double));
    float *ref = malloc((size_t)M * N * sizeof(float));
    CHECK(a && b && c && aq && as && bq && bs && gq && gs && ad && bd && ref, "host allocation");
    for (size_t i = 0; i < na; ++i) a[i] = rand_bf16();
    for (size_t i = 0; i < nb; ++i) b[i] = rand_bf16();

    /* the oracle: both operands quantized, dequantized, fp32 sum */
    CHECK(oracle_quantize_rows(a, M, K, K, aq, as) == 0, "oracle quantize A");
    CHECK(oracle_quantize_rows(b, N, K, K, bq, bs) == 0, "oracle quantize B");
    CHECK(oracle_dequantize(aq, as, M, K, ad) == 0 && oracle_dequantize(bq, bs, N, K, bd) == 0,
          "oracle dequantize");
    CHECK(oracle_gemm(ad, bd, M, N, K, ref, NULL) == 0, "oracle gemm");

    /* the library, through the C ABI only */
    void *da, *dbq, *dbs, *dbp, *dc, *dws = NULL, *dq, *ds;
    const size_t bp_bytes = mxfp4_packed_bytes(N, K);
    const size_t ws_bytes = mxfp4_gemm_workspace_bytes(M, N, K);
    HIP(hipMalloc(&da, na * 2));
    HIP(hipMalloc(&dbq, nb / 2));
    HIP(hipMalloc(&dbs, nb / 32));
    HIP(hipMalloc(&dbp, bp_bytes));
    HIP(hipMalloc(&dc, (size_t)M * N * 2));
    HIP(hipMalloc(&dq, na / 2));
    HIP(hipMalloc(&ds, na / 32));
    if (ws_bytes) {
        HIP(hipMalloc(&dws, ws_bytes));
        HIP(hipMemset(dws, 0, ws_bytes));
    }
    HIP(hipMemcpy(da, a, na * 2, hipMemcpyHostToDevice));
    HIP(hipMemcpy(dbq, bq, nb / 2, hipMemcpyHostToDevice));
    HIP(hipMemcpy(dbs, bs, nb / 32, hipMemcpyHostToDevice));
    CHECK(mxfp4_pack_b(dbq, dbs, N, K, dbp, bp_bytes, NULL) == MXFP4_OK, "pack_b: %s",
          mxfp4_last_error());
    CHECK(mxfp4_gemm(da, K, dbp, bp_bytes, dc, N, M, N, K, dws, ws_bytes, NULL) == MXFP4_OK,
          "gemm: %s", mxfp4_last_error());
    CHECK(mxfp4_quant_a(da, M, K, K, dq, K / 2, ds, K / 32, NULL) == MXFP4_OK, "quant_a: %s",
          mxfp4_last_error());
    /* the allocation-free entry on the same operands: the same bits */
    void *dc2;
    uint16_t *c2 = malloc((size_t)M * N * 2);
    CHECK(c2 != NULL, "host allocation");
    HIP(hipMalloc(&dc2, (size_t)M * N * 2));
    CHECK(mxfp4_gemm_noalloc(da, K, dbp, bp_bytes, dc2, N, M, N, K, NULL) == MXFP4_OK,
          "gemm_noalloc: %s", mxfp4_last_error());
    HIP(hipDeviceSynchronize());
    HIP(hipMemcpy(c, dc, (size_t)M * N * 2, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(c2, dc2, (size_t)M * N * 2, hipMemcpyDeviceToHost));
    CHECK(memcmp(c, c2, (size_t)M * N * 2) == 0, "gemm_noalloc differs from gemm");
    HIP(hipMemcpy(gq, dq, na / 2, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(gs, ds, na / 32, hipMemcpyDeviceToHost));

    CHECK(memcmp(gq, aq, na / 2) == 0 && memcmp(gs, as, na / 32) == 0,
          "quant_a bytes differ from the oracle's");
    int bad = 0;
    double worst = 0.0;
    for (int i = 0; i < M * N; ++i) {
        uint32_t u = (uint32_t)c[i] << 16;
        float got;
        memcpy(&got, &u, sizeof got);
        const double d = fabs((double)got - (double)ref[i]);
        if (!(d <= 1e-2 * fabs((double)ref[i]) + 1e-2)) ++bad;
        if (d > worst) worst = d;
    }
    CHECK(bad == 0, "%d of %d outputs outside the tolerance (max |d| %g)", bad, M * N, worst);
    printf("gpu check ok: %dx%dx%d, max |d| %g\n", M, N, K, worst);
    hipFree(da);
    hipFree(dbq);
    hipFree(dbs);
    hipFree(dbp);
    hipFree(dc);
    hipFree(dc2);
    free(c2);
    hipFree(dq);
    hipFree(ds);
    if (dws) hipFree(dws);
    free(a); free(b); free(c); free(aq); free(as); free(bq); free(bs); free(gq); free(gs);
    free(ad); free(bd); free(ref);
    return 0;
}

int main(int argc, char **argv) {
    if (argc < 2) {
        fprintf(stderr, "usage: %s host|gpu\n", argv[0]);
        return 2;
    }
    if (strcmp(argv[1], "host") == 0) return host_checks();
    if (strcmp(argv[1], "gpu") == 0) return gpu_check();
    fprintf(stderr, "unknown mode %s\n", argv[1]);
    return 2;
}
