/*
 * Runs every function of the oracle (oracle/oracle.c) under AddressSanitizer
 * and UndefinedBehaviorSanitizer (float-cast-overflow included) on small
 * inputs with ragged row strides, each buffer allocated at exactly the size
 * its rows span, and checks properties that hold whatever the inputs:
 *  - H_G H_G^T = G I;
 *  - the rotation of a unit vector spreads it to +-1/sqrt(G) over its group
 *    and preserves the sum of squares of every row;
 *  - codes stay within +-qmax, the absmax element maps to +-qmax, zero rows
 *    get scale 1 and codes 0, non-finite rows are rejected;
 *  - weight quantisation + unpack yields codes in [-7, 7];
 *  - the grouped integer sums add up to the whole-row sum;
 *  - the epilogue is linear in the input scale;
 *  - the AWQ product equals the bf16 matmul of the dequantised weight to
 *    within the weight's bf16 rounding;
 *  - every invalid argument listed returns BAD_ARG without touching memory.
 * Prints "oracle driver: N checks, 0 failures" and exits 0 when all pass.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_hadamard(int64_t G, int8_t *H);
int oracle_rotate(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int64_t G, float *xr, int64_t ldr);
int oracle_quantize(const float *xr, int64_t M, int64_t K, int64_t ldr, int32_t qmax, int8_t *codes,
                    int64_t ldq, float *scales);
int oracle_quantize_weights(const float *wr, int64_t N, int64_t K, int64_t ldr, int32_t group, uint8_t *packed,
                            int64_t ldp, uint16_t *scales);
int oracle_unpack(const uint8_t *packed, int64_t N, int64_t K, int64_t ldw, int8_t *w);
int oracle_int_gemm(const int8_t *codes, int64_t ldq, int64_t M, int64_t K, const int8_t *w, int64_t N,
                    int64_t Gk, int64_t *acc);
int oracle_epilogue(const int64_t *acc, int64_t M, int64_t N, int64_t ng, const float *row_scales,
                    const uint16_t *w_scales, int32_t kind, const uint16_t *bias, double x_scale, double *out);
int oracle_awq_gemv(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const uint8_t *packed, int64_t ldw,
                    const uint16_t *scales, const uint16_t *zeros, int64_t Gw, int64_t N, const uint16_t *bias,
                    double *out);
int oracle_awq_dequantize(const uint8_t *packed, int64_t N, int64_t K, int64_t ldw, const uint16_t *scales,
                          const uint16_t *zeros, int64_t Gw, uint16_t *w);
int oracle_bf16_matmul(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const uint16_t *w, int64_t N,
                       int64_t ldw, const uint16_t *bias, double *out);

static int g_checks, g_failures;

#define EXPECT(cond)                                                                        \
    do {                                                                                    \
        ++g_checks;                                                                         \
        if (!(cond)) {                                                                      \
            ++g_failures;                                                                   \
            fprintf(stderr, "%s:%d: EXPECT(%s) failed\n", __FILE__, __LINE__, #cond);       \
        }                                                                                   \
    } while (0)

/* Exact-size allocation of `rows` rows of `cols` elements with stride ld. */
static void *rows_alloc(int64_t rows, int64_t cols, int64_t ld, size_t esize)
{
    const size_t n = rows <= 0 ? 1 : (size_t)((rows - 1) * ld + cols) * esize;
    void *p = malloc(n);
    if (!p) {
        fprintf(stderr, "allocation of %zu bytes failed\n", n);
        exit(2);
    }
    memset(p, 0x7f, n);
    return p;
}

static uint32_t g_rng = 12345u;
static uint32_t rnd(void)
{
    g_rng = g_rng * 1664525u + 1013904223u;
    return g_rng >> 8;
}

/* bf16 bits of a value in [-r, r) that is exactly representable. */
static uint16_t rnd_bf16(float r)
{
    float f = ((float)(rnd() % 65536) / 32768.0f - 1.0f) * r;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static double bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static void test_hadamard(void)
{
    const int64_t sizes[] = {1, 2, 16, 64, 256};
    for (int s = 0; s < 5; ++s) {
        const int64_t G = sizes[s];
        int8_t *H = malloc((size_t)(G * G));
        EXPECT(oracle_hadamard(G, H) == 0);
        int bad = 0;
        for (int64_t i = 0; i < G; ++i)
            for (int64_t j = 0; j < G; ++j) {
                int64_t d = 0;
                for (int64_t k = 0; k < G; ++k)
                    d += H[i * G + k] * H[j * G + k];
                bad += d != (i == j ? G : 0);
            }
        EXPECT(bad == 0);
        free(H);
    }
    int8_t h1[9];
    EXPECT(oracle_hadamard(3, h1) != 0);
    EXPECT(oracle_hadamard(0, h1) != 0);
    EXPECT(oracle_hadamard(16, NULL) != 0);
}

static void test_rotate(void)
{
    const int64_t Gs[] = {16, 64, 256};
    for (int gi = 0; gi < 3; ++gi) {
        const int64_t G = Gs[gi], M = 5, K = 2 * G, ldx = K + 8, ldr = K + 3;
        uint16_t *x = rows_alloc(M, K, ldx, 2);
        float *xr = rows_alloc(M, K, ldr, 4);
        for (int64_t m = 0; m < M; ++m)
            for (int64_t k = 0; k < K; ++k)
                x[m * ldx + k] = rnd_bf16(4.0f);
        /* row 0: the unit vector at column G + 3 */
        for (int64_t k = 0; k < K; ++k)
            x[k] = 0;
        x[G + 3] = 0x3f80; /* 1.0 */
        EXPECT(oracle_rotate(x, M, K, ldx, G, xr, ldr) == 0);
        int spread = 1;
        for (int64_t k = 0; k < K; ++k) {
            const double want = k < G ? 0.0 : 1.0 / sqrt((double)G);
            spread &= fabs(fabs(xr[k]) - want) < 1e-7;
        }
        EXPECT(spread);
        for (int64_t m = 1; m < M; ++m) {
            double e0 = 0, e1 = 0;
            for (int64_t k = 0; k < K; ++k) {
                const double v = bf16_to_double(x[m * ldx + k]);
                e0 += v * v;
                e1 += (double)xr[m * ldr + k] * xr[m * ldr + k];
            }
            EXPECT(fabs(e0 - e1) <= 1e-6 * e0);
        }
        EXPECT(oracle_rotate(x, M, K, ldx, G + 1, xr, ldr) != 0);
        EXPECT(oracle_rotate(x, M, K, K - 1, G, xr, ldr) != 0);
        EXPECT(oracle_rotate(x, M, K + G / 2, ldx, G, xr, ldr) != 0);
        EXPECT(oracle_rotate(NULL, M, K, ldx, G, xr, ldr) != 0);
        free(x);
        free(xr);
    }
}

static void test_quantize(void)
{
    const int32_t qmaxes[] = {127, 7};
    for (int qi = 0; qi < 2; ++qi) {
        const int32_t qmax = qmaxes[qi];
        const int64_t M = 6, K = 100, ldr = 103, ldq = 111;
        float *xr = rows_alloc(M, K, ldr, 4);
        int8_t *codes = rows_alloc(M, K, ldq, 1);
        float *sc = malloc(M * sizeof(float));
        for (int64_t m = 0; m < M; ++m)
            for (int64_t k = 0; k < K; ++k)
                xr[m * ldr + k] = m == 2 ? 0.0f : (float)((int)(rnd() % 20001) - 10000) * 1e-3f;
        xr[4 * ldr + 17] = -50.0f; /* the absmax of row 4, negative */
        EXPECT(oracle_quantize(xr, M, K, ldr, qmax, codes, ldq, sc) == 0);
        int range = 1;
        for (int64_t m = 0; m < M; ++m)
            for (int64_t k = 0; k < K; ++k)
                range &= codes[m * ldq + k] >= -qmax && codes[m * ldq + k] <= qmax;
        EXPECT(range);
        EXPECT(codes[4 * ldq + 17] == -qmax);
        EXPECT(fabsf(sc[4] * (float)qmax - 50.0f) <= 50.0f * 1e-6f);
        EXPECT(sc[2] == 1.0f);
        int zero = 1;
        for (int64_t k = 0; k < K; ++k)
            zero &= codes[2 * ldq + k] == 0;
        EXPECT(zero);
        /* every code is the rounding of its value / scale, to within rounding of the scale */
        int close = 1;
        for (int64_t m = 0; m < M; ++m)
            for (int64_t k = 0; k < K; ++k)
                close &= fabs(xr[m * ldr + k] / sc[m] - codes[m * ldq + k]) <= 0.5 + 1e-4;
        EXPECT(close);
        /* non-finite values are rejected */
        xr[1 * ldr + 5] = INFINITY;
        EXPECT(oracle_quantize(xr, M, K, ldr, qmax, codes, ldq, sc) != 0);
        xr[1 * ldr + 5] = NAN;
        EXPECT(oracle_quantize(xr, M, K, ldr, qmax, codes, ldq, sc) != 0);
        EXPECT(oracle_quantize(xr, M, K, ldr, 128, codes, ldq, sc) != 0);
        EXPECT(oracle_quantize(xr, M, K, ldr, 0, codes, ldq, sc) != 0);
        EXPECT(oracle_quantize(xr, M, K, K - 1, qmax, codes, ldq, sc) != 0);
        free(xr);
        free(codes);
        free(sc);
    }
}

static void test_weights_and_gemm(void)
{
    const int64_t N = 5, K = 192, ldr = 197, ldp = K / 2 + 7, M = 3, ldq = K + 5;
    float *wr = rows_alloc(N, K, ldr, 4);
    uint8_t *packed = rows_alloc(N, K / 2, ldp, 1);
    uint16_t *sc_g = malloc((size_t)(K / 64) * N * 2), *sc_c = malloc((size_t)N * 2);
    int8_t *w = malloc((size_t)(N * K));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            wr[n * ldr + k] = n == 3 ? 0.0f : (float)((int)(rnd() % 2001) - 1000) * 1e-3f;
    const int32_t groups[] = {0, 64};
    for (int gi = 0; gi < 2; ++gi) {
        uint16_t *sc = groups[gi] ? sc_g : sc_c;
        EXPECT(oracle_quantize_weights(wr, N, K, ldr, groups[gi], packed, ldp, sc) == 0);
        EXPECT(oracle_unpack(packed, N, K, ldp, w) == 0);
        int range = 1;
        for (int64_t i = 0; i < N * K; ++i)
            range &= w[i] >= -7 && w[i] <= 7;
        EXPECT(range);
        int zero = 1;
        for (int64_t k = 0; k < K; ++k)
            zero &= w[3 * K + k] == 0;
        EXPECT(zero && sc[3] == 0);
    }
    wr[7] = NAN;
    EXPECT(oracle_quantize_weights(wr, N, K, ldr, 64, packed, ldp, sc_g) != 0);
    EXPECT(oracle_quantize_weights(wr, N, K, ldr, 63, packed, ldp, sc_g) != 0);
    EXPECT(oracle_quantize_weights(wr, N, K, ldr, 0, packed, K / 2 - 1, sc_c) != 0);
    EXPECT(oracle_unpack(packed, N, K + 1, ldp, w) != 0);

    int8_t *codes = rows_alloc(M, K, ldq, 1);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            codes[m * ldq + k] = (int8_t)((int)(rnd() % 255) - 127);
    int64_t *whole = malloc((size_t)(M * N) * 8), *grouped = malloc((size_t)(M * N * (K / 64)) * 8);
    EXPECT(oracle_int_gemm(codes, ldq, M, K, w, N, K, whole) == 0);
    EXPECT(oracle_int_gemm(codes, ldq, M, K, w, N, 64, grouped) == 0);
    int sums = 1;
    for (int64_t i = 0; i < M * N; ++i)
        sums &= whole[i] == grouped[3 * i] + grouped[3 * i + 1] + grouped[3 * i + 2];
    EXPECT(sums);
    EXPECT(oracle_int_gemm(codes, ldq, M, K, w, N, 50, grouped) != 0);
    EXPECT(oracle_int_gemm(codes, K - 1, M, K, w, N, 64, grouped) != 0);

    /* epilogue: linear in the input scale (bias absent), bias adds once */
    float rs[3] = {0.5f, 0.25f, 3.0f};
    uint16_t bias[5];
    for (int n = 0; n < 5; ++n)
        bias[n] = rnd_bf16(2.0f);
    double *o1 = malloc((size_t)(M * N) * 8), *o2 = malloc((size_t)(M * N) * 8), *o3 = malloc((size_t)(M * N) * 8);
    EXPECT(oracle_epilogue(grouped, M, N, K / 64, rs, sc_g, 1, NULL, 1.0, o1) == 0);
    EXPECT(oracle_epilogue(grouped, M, N, K / 64, rs, sc_g, 1, NULL, 0.375, o2) == 0);
    EXPECT(oracle_epilogue(grouped, M, N, K / 64, rs, sc_g, 1, bias, 0.375, o3) == 0);
    int lin = 1;
    for (int64_t i = 0; i < M * N; ++i) {
        lin &= fabs(o2[i] - 0.375 * o1[i]) <= 1e-12 * (1 + fabs(o1[i]));
        lin &= fabs(o3[i] - o2[i] - bf16_to_double(bias[i % N])) <= 1e-12 * (1 + fabs(o2[i]));
    }
    EXPECT(lin);
    EXPECT(oracle_epilogue(whole, M, N, 1, rs, sc_c, 0, NULL, 1.0, o1) == 0);
    EXPECT(oracle_epilogue(whole, M, N, 2, rs, sc_c, 0, NULL, 1.0, o1) != 0);
    EXPECT(oracle_epilogue(whole, M, N, 1, rs, sc_c, 2, NULL, 1.0, o1) != 0);
    EXPECT(oracle_epilogue(whole, M, N, 1, rs, sc_c, 0, NULL, 0.0, o1) != 0);
    EXPECT(oracle_epilogue(whole, M, N, 1, rs, sc_c, 0, NULL, NAN, o1) != 0);
    EXPECT(oracle_epilogue(whole, M, N, 1, rs, sc_c, 0, NULL, INFINITY, o1) != 0);
    free(wr), free(packed), free(sc_g), free(sc_c), free(w), free(codes), free(whole), free(grouped);
    free(o1), free(o2), free(o3);
}

static void test_awq(void)
{
    const int64_t M = 3, K = 128, N = 6, ldx = K + 8, ldw = K / 2 + 5, Gw = 64;
    uint16_t *x = rows_alloc(M, K, ldx, 2);
    uint8_t *packed = rows_alloc(N, K / 2, ldw, 1);
    uint16_t *sc = malloc((size_t)(K / Gw) * N * 2), *zp = malloc((size_t)(K / Gw) * N * 2);
    uint16_t *bias = malloc((size_t)N * 2), *wd = malloc((size_t)(N * K) * 2);
    double *o1 = malloc((size_t)(M * N) * 8), *o2 = malloc((size_t)(M * N) * 8);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            x[m * ldx + k] = rnd_bf16(1.0f);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j)
            packed[n * ldw + j] = (uint8_t)rnd();
    for (int64_t i = 0; i < (K / Gw) * N; ++i) {
        sc[i] = rnd_bf16(0.05f);
        zp[i] = rnd_bf16(0.1f);
    }
    for (int64_t n = 0; n < N; ++n)
        bias[n] = rnd_bf16(1.0f);
    EXPECT(oracle_awq_gemv(x, M, K, ldx, packed, ldw, sc, zp, Gw, N, bias, o1) == 0);
    EXPECT(oracle_awq_dequantize(packed, N, K, ldw, sc, zp, Gw, wd) == 0);
    EXPECT(oracle_bf16_matmul(x, M, K, ldx, wd, N, K, bias, o2) == 0);
    /* The two differ only by the two bf16 roundings of the rebuilt weight
     * (of (q - 8) s and of the sum with z), each within 2^-9 of its operand:
     * |dW| <= 2^-8 (|(q - 8) s| + |z|) per element, summed against |x|.  The
     * bound is far below the size of any dropped or misplaced term. */
    int near = 1, differs = 0;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double bound = 0;
            for (int64_t k = 0; k < K; ++k) {
                const uint8_t b = packed[n * ldw + k / 2];
                const int q = k % 2 ? b >> 4 : b & 15;
                const double s = bf16_to_double(sc[(k / Gw) * N + n]), z = bf16_to_double(zp[(k / Gw) * N + n]);
                bound += fabs(bf16_to_double(x[m * ldx + k])) * (fabs((q - 8) * s) + fabs(z)) / 256.0;
            }
            near &= fabs(o1[m * N + n] - o2[m * N + n]) <= bound + 1e-12;
            differs |= o1[m * N + n] != o2[m * N + n];
        }
    EXPECT(near);
    EXPECT(differs); /* the rounding of W is visible at these sizes */
    EXPECT(oracle_awq_gemv(x, M, K, ldx, packed, ldw, sc, zp, 48, N, bias, o1) != 0);
    EXPECT(oracle_awq_gemv(x, M, K, K - 2, packed, ldw, sc, zp, Gw, N, bias, o1) != 0);
    EXPECT(oracle_awq_dequantize(packed, N, K, K / 2 - 1, sc, zp, Gw, wd) != 0);
    EXPECT(oracle_bf16_matmul(x, M, K, ldx, wd, N, K - 1, bias, o2) != 0);
    free(x), free(packed), free(sc), free(zp), free(bias), free(wd), free(o1), free(o2);
}

int main(void)
{
    test_hadamard();
    test_rotate();
    test_quantize();
    test_weights_and_gemm();
    test_awq();
    printf("oracle driver: %d checks, %d failures\n", g_checks, g_failures);
    return g_failures == 0 ? 0 : 1;
}
