/*
 * nvfp4_oracle.c -- plain CPU reference for the NVFP4 block-scaled GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * What it computes (for every m < M, n < N):
 *
 *   C[m][n] = bf16_rne( alpha * S[m][n] ),
 *   S[m][n] = sum_{k<K} e2m1(A[m][k]) * e4m3(SA[m][k/16])
 *                     * e2m1(B[n][k]) * e4m3(SB[n][k/16])
 *
 * i.e. C = alpha * (A . B^T) on block-scaled FP4 operands.  Sources:
 *   - "The SM120 FP4 Kernel Disaster", section "Input Knowledge Required",
 *     item 3: each byte holds a pair of 4-bit codes, and blocks of codes
 *     share a scale.
 *   - "Peeling the Kernel Onion", section "The Benchmark Design": the data is
 *     packed as uint8 (two codes per byte), the scales are FP8 with one scale
 *     per 16 elements, and the output is 2 bytes per element.
 *   - same page, section "The Chain of Reasoning": the GEMM takes an alpha
 *     argument and a caller-provided output tensor.
 *   - element formats (E2M1 codes, E4M3 scales): OCP Microscaling Formats
 *     (MX) specification v1.0, sections on the FP4 E2M1 and FP8 E4M3 types.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *   - nibble order: element k = 2j sits in bits 3:0 of byte j, k = 2j+1 in
 *     bits 7:4;
 *   - scale layout: scales[r][k/16], block b covers k in [16b, 16b+16);
 *   - B is stored N x K (row n holds column n of B^T), so C = A . B^T;
 *   - E4M3 is the OCP "FN" variant: bias 7, no infinities, 0x7F/0xFF are NaN,
 *     subnormals are honoured; the scale's sign bit is honoured;
 *   - alpha multiplies the exact sum once, in fp64; the result is rounded
 *     once to bfloat16 with round-to-nearest-even, overflow to +-inf, NaN
 *     propagates.
 *
 * Accumulation is fp64.  Every product e2m1 * e4m3 * e2m1 * e4m3 is a
 * multiple of 2^-20 whose magnitude is below 2^23, so the fp64 sum is exact
 * (in any order) while |partial sums| < 2^33; no blocking or reordering is
 * applied anyway: k runs in increasing order.
 *
 * Build:  gcc -O2 -fopenmp -shared -fPIC nvfp4_oracle.c -o liboracle.so -lm
 * Build with -DORACLE_MUTANT=<n> to plant one deliberate mistake (used only
 * by the test that checks the pins catch mistakes).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

int oracle_mutant_id(void) { return ORACLE_MUTANT; }

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* FP4 E2M1 (OCP MX v1.0): bit 3 sign, bits 2:1 exponent (bias 1), bit 0
 * mantissa.  Exponent field 0 is the subnormal range: value = m * 2^-1. */
double oracle_e2m1(unsigned code) {
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag;
#if ORACLE_MUTANT == 8
    if (e == 3 && m == 1) return s ? -5.0 : 5.0; /* wrong top value */
#endif
    if (e == 0)
        mag = 0.5 * (double)m;
    else
        mag = ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
#if ORACLE_MUTANT == 3
    s = 0; /* sign dropped */
#endif
    return s ? -mag : mag;
}

/* FP8 E4M3 "FN" (OCP MX v1.0): bit 7 sign, bits 6:3 exponent (bias 7),
 * bits 2:0 mantissa; exponent 0 is subnormal (f/8 * 2^-6); S.1111.111 is NaN;
 * there is no infinity, so the largest finite value is 448. */
double oracle_e4m3(unsigned byte) {
    unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, f = byte & 7u;
    double mag;
    if (e == 15 && f == 7) return NAN;
    if (e == 0) {
#if ORACLE_MUTANT == 2
        mag = 0.0; /* subnormals flushed */
#else
        mag = ldexp((double)f, -9); /* (f/8) * 2^(1-7) */
#endif
    } else {
#if ORACLE_MUTANT == 7
        mag = ldexp(1.0 + (double)f / 8.0, (int)e - 8); /* wrong bias */
#else
        mag = ldexp(1.0 + (double)f / 8.0, (int)e - 7);
#endif
    }
    return s ? -mag : mag;
}

/* Round an fp64 value once to bfloat16 (1 sign, 8 exponent bits with bias
 * 127, 7 stored mantissa bits), round-to-nearest, ties to even.  Returns the
 * 16-bit pattern. */
uint16_t oracle_bf16(double x) {
    uint64_t bits;
    memcpy(&bits, &x, sizeof bits);
    uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
    if (isinf(x)) return (uint16_t)(sign | 0x7F80u);
    double ax = fabs(x);
    if (ax == 0.0) return sign;
    int e2;
    (void)frexp(ax, &e2);       /* ax in [2^(e2-1), 2^e2) */
    int ex = e2 - 1;            /* floor(log2(ax)) */
    if (ex < -126) ex = -126;   /* below the normal range the spacing is fixed */
    double q = ldexp(1.0, ex - 7);  /* spacing of bf16 values near ax */
    double r;
#if ORACLE_MUTANT == 10
    r = floor(ax / q); /* truncation instead of round-to-nearest-even */
#else
    r = nearbyint(ax / q); /* ax/q is exact; default mode rounds ties to even */
#endif
    double v = r * q;
    if (v >= 0x1p128) return (uint16_t)(sign | 0x7F80u); /* overflow */
    if (v < 0x1p-126) {
        /* subnormal bf16: stored mantissa = v / 2^-133 (0 .. 127) */
        return (uint16_t)(sign | (uint16_t)(v / 0x1p-133));
    }
    int ev;
    double fr = frexp(v, &ev); /* v = fr * 2^ev, fr in [0.5, 1) */
    unsigned biased = (unsigned)(ev - 1 + 127);
    unsigned mant = (unsigned)((fr * 2.0 - 1.0) * 128.0); /* exact */
    return (uint16_t)(sign | (biased << 7) | mant);
}

/* Element k of a canonical code row. */
static unsigned code_at(const uint8_t* row, int64_t k) {
    uint8_t byte = row[k / 2];
#if ORACLE_MUTANT == 1
    return (k & 1) ? (byte & 0xFu) : (byte >> 4); /* nibble order swapped */
#else
    return (k & 1) ? (byte >> 4) : (byte & 0xFu);
#endif
}

/* Scale of element k of a canonical scale row. */
static unsigned scale_at(const uint8_t* srow, int64_t k) {
#if ORACLE_MUTANT == 4
    return srow[k / 32]; /* wrong block size */
#else
    return srow[k / 16];
#endif
}

/* Decoded element k of row r of an operand (codes [rows][K/2], scales
 * [rows][K/16], canonical layout). */
static double operand_at(const uint8_t* codes, const uint8_t* scales, int64_t K, int64_t r,
                         int64_t k) {
    const uint8_t* crow = codes + r * (K / 2);
    const uint8_t* srow = scales + r * (K / 16);
    return oracle_e2m1(code_at(crow, k)) * oracle_e4m3(scale_at(srow, k));
}

/* Decoded element (r, k) of an operand in canonical layout; exported so the
 * element-order convention (element 2j in bits 3:0 of byte j) can be checked
 * on its own: the GEMM result does not depend on it when both operands share
 * it. */
double oracle_element(const uint8_t* codes, const uint8_t* scales, int64_t K, int64_t r,
                      int64_t k) {
    return operand_at(codes, scales, K, r, k);
}

/* B operand: row n of the N x K matrix.  The transposed-operand mutant reads
 * the code bytes as if they were stored (K/2) x N instead. */
static double b_at(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, int64_t n,
                   int64_t k) {
#if ORACLE_MUTANT == 5
    uint8_t byte = codes[(k / 2) * N + n];
    unsigned c = (k & 1) ? (byte >> 4) : (byte & 0xFu);
    return oracle_e2m1(c) * oracle_e4m3(scales[n * (K / 16) + k / 16]);
#else
    (void)N;
    return operand_at(codes, scales, K, n, k);
#endif
}

/* One output element: exact sum S, sum of magnitudes T, rounded result. */
static void one_element(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                        const uint8_t* b_scales, const double* b_row_decoded, float alpha,
                        int64_t N, int64_t K, int64_t m, int64_t n, const double* a_row_decoded,
                        uint16_t* out, double* exact, double* mag) {
    double S = 0.0, T = 0.0;
#if ORACLE_MUTANT == 9
    float Sf = 0.0f; /* fp32 accumulation instead of fp64 */
#endif
    for (int64_t k = 0; k < K; ++k) {
        double a = a_row_decoded ? a_row_decoded[k] : operand_at(a_codes, a_scales, K, m, k);
        double b = b_row_decoded ? b_row_decoded[k] : b_at(b_codes, b_scales, N, K, n, k);
        double p = a * b;
#if ORACLE_MUTANT == 9
        Sf += (float)p;
#endif
        S += p;
#if ORACLE_MUTANT == 11
        T += p; /* magnitude sum without the absolute value */
#else
        T += fabs(p);
#endif
    }
#if ORACLE_MUTANT == 9
    S = (double)Sf;
#endif
#if ORACLE_MUTANT == 6
    double y = S; /* alpha ignored */
#else
    double y = (double)alpha * S;
#endif
    if (out) *out = oracle_bf16(y);
    if (exact) *exact = y;
    if (mag) *mag = T;
}

/* Full GEMM on canonical operands.
 *   a_codes  [M][K/2], a_scales [M][K/16], b_codes [N][K/2], b_scales [N][K/16]
 *   out      [M][N] bfloat16 bit patterns (required)
 *   exact    [M][N] alpha*S in fp64 (optional, may be NULL)
 *   mag      [M][N] T = sum_k |a'_k b'_k| (optional, may be NULL)
 * Returns 0, or -1 when M, N or K is negative or K is not a multiple of 16
 * (the pages require K to be a whole number of scale blocks, and so of code
 * pairs: "The SM120 FP4 Kernel Disaster", section "The Bash Command").
 * Work is spread over the host threads by output element, so a product with
 * a single row uses every thread as well; each element is still the same
 * plain sum over k in increasing order. */
int oracle_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                const uint8_t* b_scales, float alpha, int64_t M, int64_t N, int64_t K,
                uint16_t* out, double* exact, double* mag) {
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0) return -1;
    if (M == 0 || N == 0) return 0;
    const size_t kk = (size_t)(K > 0 ? K : 1);
    /* Step 1: decode every row of A and of B once to fp64 (exact). */
    double* adec = (double*)malloc((size_t)M * kk * sizeof(double));
    double* bdec = (double*)malloc((size_t)N * kk * sizeof(double));
    if (!adec || !bdec) {
        free(adec);
        free(bdec);
        return -2;
    }
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) adec[m * K + k] = operand_at(a_codes, a_scales, K, m, k);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) bdec[n * K + k] = b_at(b_codes, b_scales, N, K, n, k);
    /* Step 2: every output element is the contraction of its two rows. */
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < M * N; ++i) {
        const int64_t m = i / N, n = i % N;
        one_element(a_codes, a_scales, b_codes, b_scales, bdec + n * K, alpha, N, K, m, n,
                    adec + m * K, out + i, exact ? exact + i : NULL, mag ? mag + i : NULL);
    }
    free(adec);
    free(bdec);
    return 0;
}

/* Selected output elements only, each computed on its own from the packed
 * canonical bytes: element p is (ms[p], ns[p]).  Same operands and rules as
 * oracle_gemm; used to check very large problems at sampled positions. */
int oracle_gemm_points(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                       const uint8_t* b_scales, float alpha, int64_t M, int64_t N, int64_t K,
                       const int64_t* ms, const int64_t* ns, int64_t P, uint16_t* out,
                       double* exact, double* mag) {
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0 || P < 0) return -1;
    for (int64_t p = 0; p < P; ++p)
        if (ms[p] < 0 || ms[p] >= M || ns[p] < 0 || ns[p] >= N) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < P; ++p) {
        one_element(a_codes, a_scales, b_codes, b_scales, NULL, alpha, N, K, ms[p], ns[p], NULL,
                    out + p, exact ? exact + p : NULL, mag ? mag + p : NULL);
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * NVFP4 quantisation of fp32 rows: the step before the GEMM, activations
 * quantised per 16-element block along K into E2M1 codes and one E4M3 scale
 * per block (format: "Peeling the Kernel Onion", section "The Benchmark
 * Design"; the recipe is the plainest reading of "scale = E4M3(amax / 6),
 * codes = round-to-nearest-even E2M1").  Readings:
 *   - amax / 6 and x / scale are single fp32 operations (correctly rounded);
 *   - the scale byte is the non-negative finite E4M3 value nearest to
 *     amax / 6, ties to the even byte; past 448 it saturates to 448;
 *   - a block whose scale is 0 (all zeros, or amax / 6 below half the
 *     smallest E4M3 subnormal) gets magnitude-0 codes;
 *   - a code is the E2M1 magnitude nearest to |x / scale|, ties to the even
 *     code, past 6 saturating to 6, with the sign bit of x (so -0.0 and
 *     negative values that round to 0 give code 0x8);
 *   - non-finite inputs are outside the contract (infinities saturate).
 * Both roundings pick the nearest entry of the value table by exhaustive
 * search, so the code states the definition directly.
 * ------------------------------------------------------------------------- */
static unsigned quant_scale_byte(float amax) {
    const float t = amax / 6.0f;
    if (t >= 448.0f) return 0x7E;     /* at or past the largest finite value */
    unsigned best = 0;
    double bestd = INFINITY;
    for (unsigned b = 0; b <= 0x7E; ++b) {
        const double v = oracle_e4m3(b);
#if ORACLE_MUTANT == 12
        /* planted mistake: truncation (largest value not above t) */
        if (v <= (double)t) best = b;
        continue;
#endif
        const double d = fabs(v - (double)t);
        if (d < bestd || (d == bestd && (b & 1u) == 0)) {
            best = b;
            bestd = d;
        }
    }
    return best;
}

static unsigned quant_code(float x, float s) {
    unsigned sign = signbit(x) ? 8u : 0u;
    if (s == 0.0f) return sign;
#if ORACLE_MUTANT == 15
    const float y = x * (1.0f / s);   /* planted mistake: reciprocal multiply */
#else
    const float y = x / s;
#endif
    const double ay = fabs((double)y);
    if (ay >= 6.0) return sign | 7u;  /* at or past the largest magnitude */
    unsigned best = 0;
    double bestd = INFINITY;
    for (unsigned c = 0; c < 8; ++c) {
        const double d = fabs(oracle_e2m1(c) - ay);
#if ORACLE_MUTANT == 13
        /* planted mistake: ties away from zero */
        if (d < bestd || d == bestd) {
#else
        if (d < bestd || (d == bestd && (c & 1u) == 0)) {
#endif
            best = c;
            bestd = d;
        }
    }
#if ORACLE_MUTANT == 14
    if (best == 0) sign = 0;          /* planted mistake: zero codes lose the sign */
#endif
    return sign | best;
}

/* x: rows x K fp32 values, row stride ld (>= K) elements; codes [rows][K/2]
 * (element 2j in bits 3:0 of byte j), scales [rows][K/16].  Returns 0, or -1
 * for bad sizes. */
int oracle_quantize(const float* x, int64_t rows, int64_t K, int64_t ld, uint8_t* codes,
                    uint8_t* scales) {
    if (rows < 0 || K < 0 || K % 16 != 0 || ld < K) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t blk = 0; blk < K / 16; ++blk) {
            const float* v = x + r * ld + blk * 16;
            float amax = 0.0f;
            for (int i = 0; i < 16; ++i) {
                const float a = fabsf(v[i]);
                if (a > amax) amax = a;
            }
            const unsigned sb = quant_scale_byte(amax);
            scales[r * (K / 16) + blk] = (uint8_t)sb;
            const float s = (float)oracle_e4m3(sb);
            for (int i = 0; i < 16; i += 2) {
                const unsigned c0 = quant_code(v[i], s), c1 = quant_code(v[i + 1], s);
                codes[r * (K / 2) + blk * 8 + i / 2] = (uint8_t)(c0 | (c1 << 4));
            }
        }
    }
    return 0;
}
