/*
 * mxfp4_oracle.c -- plain, slow, scalar CPU oracle for the MXFP4 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load this file
 * or the library built from it: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header or table
 * with the HIP library under block_scaled_precision_quant_amd/csrc.
 *
 * What it computes (pages: kernelindex.com "kernelbot amd-mxfp4-mm"
 * submissions 752099, 739530, 694791 and 754549):
 *
 *   quantize   one e8m0 scale per 32 consecutive K-elements of a row, then
 *              one e2m1 code per element, two codes per byte;
 *   dequantize code value times 2^(scale byte - 127);
 *   gemm       C[m][n] = sum_k deqA[m][k] * deqB[n][k], an fp32 running sum
 *              in increasing k, plus an fp64 sum for cross-checking.
 *
 * Every function below says which passage it follows.  Floating point that
 * the pages leave open is done in double.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_GROUP 32

/* The eight magnitudes an e2m1 code can take, indexed by the low three bits
 * of the code.  Submission 694791 (page 4), `_mxfp4_quant_tile`: the largest
 * magnitude is 6 = 1.5 * 2^2; codes below 1.0 are the subnormal 0 and 0.5. */
static const double E2M1_MAGNITUDE[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

static uint32_t f32_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

static float bf16_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Scale byte of one group, from its largest magnitude.
 *
 * Submission 752099 (page 1), `_bf16_to_fp4_hw`, and submission 754549
 * (page 5), `_quantize_mxfp4`: add 0x200000 to the fp32 bit pattern of the
 * group maximum and keep only sign and exponent (this rounds the maximum up
 * to the next power of two only when its significand is at least 1.75);
 * take the unbiased exponent, subtract 2 (the largest e2m1 magnitude, 6, lies
 * in the binade of 2^2), clamp to [-127, 127] and add the bias 127.
 * Submission 739530 (page 2), `hw_quant32`, treats an all-zero group as
 * exponent -127, which the clamp already gives. */
int oracle_scale_byte(float amax) {
    uint32_t u = f32_bits(amax);
    u = (u + 0x00200000u) & 0xFF800000u;
    int biased = (int)((u >> 23) & 0xFFu);
    int s = biased - 127 - 2;
    if (s < -127) s = -127;
    if (s > 127) s = 127;
    return s + 127;
}

/* e2m1 code of one element, given the scale byte of its group.
 *
 * Submission 694791 (page 4), `_mxfp4_quant_tile`: the element is multiplied
 * by 2^-s (s = byte - 127); magnitudes of 6 and above saturate to code 7;
 * otherwise the magnitude rounds to the nearest representable e2m1 value,
 * ties to the even code (the round-to-nearest-even of the e2m1 mantissa);
 * the sign of the input goes to bit 3, also when the magnitude rounds to 0.
 * The product x * 2^-s is exact in double for every bf16 x and every byte. */
int oracle_e2m1_code(float x, int scale_byte) {
    double q = ldexp((double)x, 127 - scale_byte);
    double mag = fabs(q);
    int code;
    if (mag >= 6.0) {
        code = 7;
    } else {
        code = 0;
        double best = mag; /* distance to E2M1_MAGNITUDE[0] == 0 */
        for (int c = 1; c < 8; ++c) {
            double d = fabs(mag - E2M1_MAGNITUDE[c]);
            if (d < best || (d == best && (c % 2) == 0)) {
                best = d;
                code = c;
            }
        }
    }
    if (signbit(x)) code |= 8;
    return code;
}

/* Batch form of oracle_e2m1_code over n (value, scale byte) pairs, so that the
 * tests can sweep every bf16 value under every scale byte. */
int oracle_e2m1_codes(const float *x, const int32_t *scale_bytes, int64_t n, uint8_t *codes) {
    for (int64_t i = 0; i < n; ++i) codes[i] = (uint8_t)oracle_e2m1_code(x[i], scale_bytes[i]);
    return 0;
}

/* Value of one code under one scale byte: (-1)^(bit 3) * magnitude *
 * 2^(byte - 127).  Byte 127 means a factor of exactly 1 (submission 705642,
 * page 3, pads its scale buffer with 127 for that reason). */
double oracle_dequant_value(int code, int scale_byte) {
    double v = ldexp(E2M1_MAGNITUDE[code & 7], scale_byte - 127);
    return (code & 8) ? -v : v;
}

/* Quantize `rows` rows of K bf16 values (row stride `ld` elements) into
 * linear fp4x2 [rows][K/2] and e8m0 [rows][K/32].
 *
 * Groups are 32 consecutive K-elements of one row starting at k = 0.
 * Packing (submission 694791, page 4): byte j of a row holds the code of
 * element 2j in its low nibble and of element 2j+1 in its high nibble.
 * Returns 0, or -1 when K is not a multiple of 32. */
int oracle_quantize_rows(const uint16_t *x, int64_t rows, int64_t K, int64_t ld,
                         uint8_t *fp4, uint8_t *scale) {
    if (K % ORACLE_GROUP != 0 || rows < 0 || ld < K) return -1;
    const int64_t groups = K / ORACLE_GROUP;
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *row = x + r * ld;
        for (int64_t g = 0; g < groups; ++g) {
            const uint16_t *grp = row + g * ORACLE_GROUP;
            float amax = 0.0f;
            for (int i = 0; i < ORACLE_GROUP; ++i) {
                float a = fabsf(bf16_value(grp[i]));
                if (a > amax) amax = a;
            }
            int byte = oracle_scale_byte(amax);
            scale[r * groups + g] = (uint8_t)byte;
            for (int i = 0; i < ORACLE_GROUP; i += 2) {
                int lo = oracle_e2m1_code(bf16_value(grp[i]), byte);
                int hi = oracle_e2m1_code(bf16_value(grp[i + 1]), byte);
                fp4[r * (K / 2) + g * (ORACLE_GROUP / 2) + i / 2] =
                    (uint8_t)(lo | (hi << 4));
            }
        }
    }
    return 0;
}

/* Dequantize linear fp4x2 [rows][K/2] + e8m0 [rows][K/32] into double
 * [rows][K]. */
int oracle_dequantize(const uint8_t *fp4, const uint8_t *scale, int64_t rows, int64_t K,
                      double *out) {
    if (K % ORACLE_GROUP != 0 || rows < 0) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = fp4[r * (K / 2) + k / 2];
            int code = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
            out[r * K + k] = oracle_dequant_value(code, scale[r * (K / ORACLE_GROUP) + k / ORACLE_GROUP]);
        }
    }
    return 0;
}

/* C[m][n] = sum over k of deqA[m][k] * deqB[n][k], B given as [N][K].
 *
 * The block-scaled dot of the pages (`tl.dot_scaled` with two e2m1 operands
 * and an fp32 accumulator; submission 752099, `_quant_gemm_fused_launcher`)
 * accumulates in fp32.  `c32` is that sum taken in increasing k, each
 * product formed in double and rounded once to fp32 before it is added;
 * `c64` is the same sum in double.  Either output may be NULL. */
int oracle_gemm(const double *a_deq, const double *b_deq, int64_t M, int64_t N, int64_t K,
                float *c32, double *c64) {
    if (M < 0 || N < 0 || K < 0) return -1;
    for (int64_t m = 0; m < M; ++m) {
        const double *a = a_deq + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const double *b = b_deq + n * K;
            float s32 = 0.0f;
            double s64 = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = a[k] * b[k];
                s32 += (float)p;
                s64 += p;
            }
            if (c32) c32[m * N + n] = s32;
            if (c64) c64[m * N + n] = s64;
        }
    }
    return 0;
}

/* Sum of |deqA[m][k] * deqB[n][k]| over k, for the fp32-vs-fp64 error bound
 * (an fp32 running sum of K terms differs from the exact sum by at most about
 * K * 2^-24 times this). */
int oracle_gemm_abs(const double *a_deq, const double *b_deq, int64_t M, int64_t N, int64_t K,
                    double *cabs) {
    if (M < 0 || N < 0 || K < 0) return -1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += fabs(a_deq[m * K + k] * b_deq[n * K + k]);
            cabs[m * N + n] = s;
        }
    return 0;
}
