/*
 * Reference oracle for the ConvRot packed-INT4 quantized linear.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library under
 * packed_int4_convrot_amd/ may link, import or call this file; only the
 * tests, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * It is deliberately plain: single-threaded loops, no blocking, no fast
 * transform, no vectorisation.  Real-valued sums are taken in fp64.  The one
 * place where floating point decides an integer (the activation codes) is
 * done in fp32, the precision the GPU kernels use for the same decision.
 * Compile with -O2 -ffp-contract=off so that no multiply-add is fused.
 *
 * Sources, by page title:
 *  - "[PR #155] [Feat][Ascend] Add fused RotateQuant backend" (comfy-kitchen),
 *    section "What this PR does": the fused operator replaces a rotation
 *    matmul followed by a dynamic rowwise quantisation; group sizes 16, 64
 *    and 256; zero rows must keep a positive scale.
 *  - "comfy_kitchen/tensor/awq_w4a16.py", module docstring and dequantize():
 *    the packed uint4 layout (bits 0..3 = column 2j, bits 4..7 = column
 *    2j+1, stored code q means q-8) and the AWQ dequantisation
 *    W[n,k] = (q-8)*s[k/G,n] + z[k/G,n].
 *  - "[PR #182] HIP port of #176: W4A8 decode GEMV ..." (comfy-kitchen),
 *    description: integer dot products of int8 activations with decoded
 *    int4 weights, then a rowwise-times-weight-scale epilogue.
 *  - "feat: support packed INT4 convrot models" (stable-diffusion.cpp),
 *    summary: 64-element ConvRot quantisation groups ("H64").
 *
 * Readings where the pages are silent (each is listed in the design doc):
 *  - H_G is the Sylvester Hadamard matrix in natural order,
 *    H[i][j] = (-1)^popcount(i & j), applied as x_g . H_G / sqrt(G) to each
 *    contiguous block of G columns.
 *  - Codes are symmetric: qmax = 127 (int8) or 7 (int4); scale = absmax/qmax;
 *    code = round-half-even(fp32(xr * fp32(qmax/absmax))), clamped to
 *    [-qmax, qmax].  An all-zero row gets codes 0 and scale 1.0.
 *  - The input scale a of the packed matmul is the linear of a * x: the
 *    codes of x with the row scale multiplied by a (see oracle_epilogue).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define OK 0
#define BAD_ARG 1

/* bf16 bit pattern -> exact double (bf16 is the top half of an fp32). */
static double bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

/* Sylvester Hadamard entry in natural order. */
static int hadamard_entry(int64_t i, int64_t j)
{
    uint64_t v = (uint64_t)(i & j);
    int parity = 0;
    while (v) {
        parity ^= (int)(v & 1u);
        v >>= 1;
    }
    return parity ? -1 : 1;
}

/* H[i*G + j] = (-1)^popcount(i & j), i, j < G. */
int oracle_hadamard(int64_t G, int8_t *H)
{
    if (!is_pow2(G) || !H)
        return BAD_ARG;
    for (int64_t i = 0; i < G; ++i)
        for (int64_t j = 0; j < G; ++j)
            H[i * G + j] = (int8_t)hadamard_entry(i, j);
    return OK;
}

/*
 * Group-wise rotation by explicit matrix product:
 *   xr[m, g*G + j] = fp32( (sum_i x[m, g*G + i] * H[i][j]) / sqrt(G) ).
 * The sum runs in fp64 and is rounded to fp32 once.  x is bf16 with row
 * stride ldx (elements); xr is fp32 with row stride ldr.
 */
int oracle_rotate(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                  int64_t G, float *xr, int64_t ldr)
{
    if (!x || !xr || M < 0 || K < 0 || !is_pow2(G) || K % G != 0 ||
        ldx < K || ldr < K)
        return BAD_ARG;
    const double norm = sqrt((double)G);
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t g = 0; g < K / G; ++g) {
            const uint16_t *xg = x + m * ldx + g * G;
            for (int64_t j = 0; j < G; ++j) {
                double s = 0.0;
                for (int64_t i = 0; i < G; ++i)
                    s += bf16_value(xg[i]) * (double)hadamard_entry(i, j);
                xr[m * ldr + g * G + j] = (float)(s / norm);
            }
        }
    }
    return OK;
}

/*
 * Dynamic rowwise symmetric quantisation of already rotated values.
 *   a = max_k |xr[m,k]|
 *   a > 0 : s = fp32(a / qmax), inv = fp32(qmax / a),
 *           code = clamp(rne(fp32(xr * inv)), -qmax, qmax)
 *   a == 0: code = 0, s = 1.0
 * Defined for finite values only: a row holding Inf or NaN is BAD_ARG (the
 * pages give no rule for it, and a NaN code has no integer value).
 */
int oracle_quantize(const float *xr, int64_t M, int64_t K, int64_t ldr,
                    int32_t qmax, int8_t *codes, int64_t ldq, float *scales)
{
    if (!xr || !codes || !scales || M < 0 || K < 0 || ldr < K || ldq < K ||
        qmax < 1 || qmax > 127)
        return BAD_ARG;
    const float fq = (float)qmax;
    for (int64_t m = 0; m < M; ++m) {
        const float *row = xr + m * ldr;
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            if (!isfinite(row[k]))
                return BAD_ARG;
            float v = fabsf(row[k]);
            if (v > a)
                a = v;
        }
        if (a > 0.0f) {
            const float s = a / fq;
            const float inv = fq / a;
            for (int64_t k = 0; k < K; ++k) {
                float t = row[k] * inv;
                float r = nearbyintf(t); /* default rounding: half to even */
                if (r > fq)
                    r = fq;
                if (r < -fq)
                    r = -fq;
                codes[m * ldq + k] = (int8_t)r;
            }
            scales[m] = s;
        } else {
            for (int64_t k = 0; k < K; ++k)
                codes[m * ldq + k] = 0;
            scales[m] = 1.0f;
        }
    }
    return OK;
}

/* fp32 -> bf16 bit pattern, round to nearest even on the 16 dropped bits
 * (finite values only). */
static uint16_t bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint32_t lower = u & 0xFFFFu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

/*
 * Weight quantisation of already rotated weight rows (the producer of the
 * packed format; the pages hold packed checkpoints but no formula, so this is
 * the plain symmetric reading, listed in the design doc):
 *   a = max |wr| over the row (group == 0) or over each run of `group`
 *       columns (group == 64);
 *   s = bf16(fp32(a / 7)) and, where s > 0,
 *   code = clamp(rne(fp32(wr * fp32(1 / s))), -7, 7), else code = 0;
 *   stored q = code + 8, byte j of a row = q[2j] | q[2j + 1] << 4.
 * scales: bf16 bits, [N] (group == 0) or [K/group, N] (N contiguous).
 * Finite weights only (BAD_ARG otherwise), as in oracle_quantize.
 */
int oracle_quantize_weights(const float *wr, int64_t N, int64_t K, int64_t ldr, int32_t group,
                            uint8_t *packed, int64_t ldp, uint16_t *scales)
{
    if (!wr || !packed || !scales || N < 0 || K <= 0 || K % 2 != 0 || ldr < K || ldp < K / 2 ||
        group < 0 || (group > 0 && (group % 2 != 0 || K % group != 0)))
        return BAD_ARG;
    const int64_t glen = group > 0 ? group : K;
    for (int64_t n = 0; n < N; ++n) {
        const float *row = wr + n * ldr;
        uint8_t *prow = packed + n * ldp;
        for (int64_t g0 = 0; g0 < K; g0 += glen) {
            float a = 0.0f;
            for (int64_t k = g0; k < g0 + glen; ++k) {
                if (!isfinite(row[k]))
                    return BAD_ARG;
                float v = fabsf(row[k]);
                if (v > a)
                    a = v;
            }
            const uint16_t sb = bf16_round(a / 7.0f);
            const float sf = (float)bf16_value(sb);
            const float inv = sf > 0.0f ? 1.0f / sf : 0.0f;
            for (int64_t k = g0; k < g0 + glen; k += 2) {
                int q[2];
                for (int e = 0; e < 2; ++e) {
                    float r = nearbyintf(row[k + e] * inv);
                    if (r > 7.0f)
                        r = 7.0f;
                    if (r < -7.0f)
                        r = -7.0f;
                    q[e] = (int)r + 8;
                }
                prow[k / 2] = (uint8_t)(q[0] | (q[1] << 4));
            }
            if (group > 0)
                scales[(g0 / glen) * N + n] = sb;
            else
                scales[n] = sb;
        }
    }
    return OK;
}

/*
 * Packed uint4 weight decode: byte j of row n holds column 2j in bits 0..3
 * and column 2j+1 in bits 4..7; the stored code q stands for q - 8.
 * packed has row stride ldw (bytes); w is [N, K] int8, row stride K.
 */
int oracle_unpack(const uint8_t *packed, int64_t N, int64_t K, int64_t ldw,
                  int8_t *w)
{
    if (!packed || !w || N < 0 || K < 0 || K % 2 != 0 || ldw < K / 2)
        return BAD_ARG;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < K / 2; ++j) {
            const uint8_t b = packed[n * ldw + j];
            w[n * K + 2 * j] = (int8_t)((int)(b & 0x0F) - 8);
            w[n * K + 2 * j + 1] = (int8_t)((int)(b >> 4) - 8);
        }
    }
    return OK;
}

/*
 * Integer matmul with exact accumulation, split into K-groups of Gk columns
 * (Gk == K gives one sum per output):
 *   acc[(m*N + n)*(K/Gk) + g] = sum_{k in group g} codes[m,k] * w[n,k]
 * The sums are taken in int64; the caller checks the int32 range.
 */
int oracle_int_gemm(const int8_t *codes, int64_t ldq, int64_t M, int64_t K,
                    const int8_t *w, int64_t N, int64_t Gk, int64_t *acc)
{
    if (!codes || !w || !acc || M < 0 || N < 0 || K < 0 || ldq < K ||
        Gk <= 0 || K % Gk != 0)
        return BAD_ARG;
    const int64_t ng = K / Gk;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t g = 0; g < ng; ++g) {
                int64_t s = 0;
                for (int64_t k = g * Gk; k < (g + 1) * Gk; ++k)
                    s += (int64_t)codes[m * ldq + k] * (int64_t)w[n * K + k];
                acc[(m * N + n) * ng + g] = s;
            }
    return OK;
}

/*
 * Scale epilogue in fp64.
 *   per channel (kind 0, ng == 1): out = a * s_x[m] * s_w[n] * acc[m,n]
 *   per group   (kind 1):          out = a * s_x[m] * sum_g s_w[g,n] * acc_g[m,n]
 * plus bias[n] when bias is not NULL.  w_scales is bf16: [N] for kind 0,
 * [ng, N] (N contiguous) for kind 1.  out is [M, N] fp64.
 *
 * a is the input scale of "feat: support packed INT4 convrot models"
 * (summary: the packed matmul takes an optional bias and input scale; the
 * review text on its ConvRot notes says inputs of other scales are scaled
 * and quantised inside the matmul).  Reading: the result is the linear of
 * a * x.  In exact arithmetic the rotation and the absmax are both linear in
 * x, so a * x has the codes of x and the row scale a * s_x; the oracle
 * therefore multiplies the row scale by a (in fp64) and leaves the bias
 * unscaled.  a = 1 is the plain linear; a must be positive and finite.
 */
int oracle_epilogue(const int64_t *acc, int64_t M, int64_t N, int64_t ng,
                    const float *row_scales, const uint16_t *w_scales,
                    int32_t kind, const uint16_t *bias, double x_scale,
                    double *out)
{
    if (!acc || !row_scales || !w_scales || !out || M < 0 || N < 0 ||
        ng <= 0 || (kind != 0 && kind != 1) || (kind == 0 && ng != 1) ||
        !(x_scale > 0.0) || !isfinite(x_scale))
        return BAD_ARG;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double t = 0.0;
            if (kind == 0) {
                t = bf16_value(w_scales[n]) * (double)acc[m * N + n];
            } else {
                for (int64_t g = 0; g < ng; ++g)
                    t += bf16_value(w_scales[g * N + n]) *
                         (double)acc[(m * N + n) * ng + g];
            }
            t *= (double)row_scales[m] * x_scale;
            if (bias)
                t += bf16_value(bias[n]);
            out[m * N + n] = t;
        }
    }
    return OK;
}

/*
 * AWQ W4A16 product, fp64 throughout:
 *   W[n,k] = (q[n,k] - 8) * s[k/Gw, n] + z[k/Gw, n]
 *   out[m,n] = sum_k x[m,k] * W[n,k]  (+ bias[n])
 * The weight is not rounded to bf16 before the product.
 */
int oracle_awq_gemv(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                    const uint8_t *packed, int64_t ldw, const uint16_t *scales,
                    const uint16_t *zeros, int64_t Gw, int64_t N,
                    const uint16_t *bias, double *out)
{
    if (!x || !packed || !scales || !zeros || !out || M < 0 || N < 0 ||
        K < 0 || K % 2 != 0 || ldx < K || ldw < K / 2 || Gw <= 0 ||
        K % Gw != 0)
        return BAD_ARG;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double t = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const uint8_t b = packed[n * ldw + k / 2];
                const int q = (k % 2 == 0) ? (b & 0x0F) : (b >> 4);
                const double wv = (double)(q - 8) *
                                      bf16_value(scales[(k / Gw) * N + n]) +
                                  bf16_value(zeros[(k / Gw) * N + n]);
                t += bf16_value(x[m * ldx + k]) * wv;
            }
            if (bias)
                t += bf16_value(bias[n]);
            out[m * N + n] = t;
        }
    }
    return OK;
}

/*
 * The dequantise path of "comfy_kitchen/tensor/awq_w4a16.py", dequantize():
 * the weight is rebuilt in the bf16 compute dtype, one tensor operation at a
 * time, so each product and each sum is rounded to bf16 (nearest even):
 *   W[n, k] = bf16( bf16((q - 8) * s[k/Gw, n]) + z[k/Gw, n] )
 * (each operation computed in fp32 first, as a bf16 tensor operation does;
 * (q - 8) * s is exact in fp32).  W is written as bf16 bits [N, K].
 */
int oracle_awq_dequantize(const uint8_t *packed, int64_t N, int64_t K, int64_t ldw,
                          const uint16_t *scales, const uint16_t *zeros, int64_t Gw,
                          uint16_t *w)
{
    if (!packed || !scales || !zeros || !w || N < 0 || K < 0 || K % 2 != 0 ||
        ldw < K / 2 || Gw <= 0 || K % Gw != 0)
        return BAD_ARG;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const uint8_t b = packed[n * ldw + k / 2];
            const int q = (k % 2 == 0) ? (b & 0x0F) : (b >> 4);
            const float sc = (float)bf16_value(scales[(k / Gw) * N + n]);
            const float zp = (float)bf16_value(zeros[(k / Gw) * N + n]);
            const float prod = (float)(q - 8) * sc;
            const float sum = (float)bf16_value(bf16_round(prod)) + zp;
            w[n * K + k] = bf16_round(sum);
        }
    return OK;
}

/* out[m, n] = sum_k x[m, k] * w[n, k] (+ bias[n]) in fp64, x and w bf16. */
int oracle_bf16_matmul(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                       const uint16_t *w, int64_t N, int64_t ldw, const uint16_t *bias,
                       double *out)
{
    if (!x || !w || !out || M < 0 || N < 0 || K < 0 || ldx < K || ldw < K)
        return BAD_ARG;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double t = 0.0;
            for (int64_t k = 0; k < K; ++k)
                t += bf16_value(x[m * ldx + k]) * bf16_value(w[n * ldw + k]);
            if (bias)
                t += bf16_value(bias[n]);
            out[m * N + n] = t;
        }
    return OK;
}
