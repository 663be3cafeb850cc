// Decode GEMV for 1 <= M <= 8 activation rows on given int8 codes.
//
// Prior art: the W4A8 decode GEMV of "[PR #182] HIP port of #176: W4A8 decode
// GEMV and fused GatedDeltaNet decode" (description): register-side int4
// decode feeding v_dot4 integer dot products and a rowwise x weight-scale
// epilogue, with no decoded weight copy in memory.  (The whole decode linear
// from bf16 rows, with the rotate-quant in the same launch, is
// w4_gemv_fused.hip; it keeps this kernel's per-wave layout and arithmetic.)
//
// Layout (built for HBM streaming, one K slice per wave):
//   * wave w of a block owns columns k in [2048 w, 2048 w + 2048); lane l owns
//     the 32 columns starting at 2048 w + 32 l, i.e. 16 packed bytes of every
//     weight row, so one load instruction reads 1 KiB of contiguous weights;
//   * a block handles R consecutive weight rows; each lane issues its
//     activation-code loads, then its R 16-byte weight loads, then splits its
//     32 codes into even / odd k to match the nibble decode;
//   * per weight row: unsigned nibbles (0..15) times codes with v_dot4_i32_i8,
//     then subtract 8 * sum(codes) (the code-8 offset), then the per-group
//     scale for the lane's group;
//   * the R per-row partials of all 64 lanes are summed by a transposed
//     reduction (permlane32/16 swaps, DPP, swizzle), then across waves through
//     LDS in a fixed order.
#include "ck_device.h"
#include "gemv_reduce.h"
#include "launch.h"

namespace ck {
namespace {

constexpr int kMaxWaves = kGemvMaxWaves;  // K <= 16384
#ifndef CK_GEMV_ROWS
#define CK_GEMV_ROWS 8  // weight rows per block (8, 16 or 32)
#endif
template <int M, int R, bool PER_GROUP, bool OUT_I32>
__global__ __launch_bounds__(kMaxWaves * kWave) void w4_gemv_kernel(
    const int8_t *__restrict__ codes, int64_t ldq, const float *__restrict__ row_scales, int K,
    const uint8_t *__restrict__ packed, int64_t ldw, const uint16_t *__restrict__ w_scales, int N,
    const uint16_t *__restrict__ bias, float x_scale, uint16_t *__restrict__ out, int64_t ldo,
    int32_t *__restrict__ acc_out, int64_t lda)
{
    constexpr bool FSUM = PER_GROUP && !OUT_I32;  // partials are fp32 (scaled) or exact int32
    __shared__ uint32_t s_red[kMaxWaves][R][M];

    const int nw = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int n0 = xcd_block(blockIdx.x, gridDim.x) * R;
    const int kbase = 2048 * wave + 32 * lane;
    const bool active = kbase < K;
    const int kc = active ? kbase : K - 32;  // clamped: every address stays inside the row

    // 1. Loads, in this order: the activation codes (small, usually
    //    L2-resident), the weight scales, then the R weight rows.  Loads retire
    //    in issue order, so the activation work below waits only for the
    //    codes, and row r's dot products only for rows 0..r, while the
    //    remaining weight rows are still streaming in.
    u32x4 araw[M][2];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int c = 0; c < 2; ++c)
            araw[m][c] = *reinterpret_cast<const u32x4 *>(codes + (int64_t)m * ldq + kc + 16 * c);
    // The R scales of the lane's group are contiguous: R / 8 16-byte loads.
    // (Eight 2-byte loads per row block were measured ~0.5 us slower.)
    u32x4 sv[PER_GROUP ? R / 8 : 1];
    if constexpr (PER_GROUP) {
#pragma unroll
        for (int q = 0; q < R / 8; ++q)
            sv[q] = *reinterpret_cast<const u32x4 *>(w_scales + (int64_t)(kc / 64) * N + n0 + 8 * q);
    }
    u32x4 wv[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        wv[r] = load_nt16(packed + (int64_t)(n0 + r) * ldw + kc / 2);
    // Keep the compiler from moving these loads below the activation work.
    __builtin_amdgcn_sched_barrier(0);

    // 2. activation codes for this lane's 32 columns: even k in alo, odd k in ahi.
    uint32_t alo[M][4], ahi[M][4];
    float sx[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const u32x4 c0 = araw[m][0];
        const u32x4 c1 = araw[m][1];
        const v4i p0 = act_perm16(c0[0], c0[1], c0[2], c0[3]);
        const v4i p1 = act_perm16(c1[0], c1[1], c1[2], c1[3]);
        const uint32_t q[8] = {(uint32_t)p0[0], (uint32_t)p0[1], (uint32_t)p0[2], (uint32_t)p0[3],
                               (uint32_t)p1[0], (uint32_t)p1[1], (uint32_t)p1[2], (uint32_t)p1[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            alo[m][i] = active ? q[2 * i] : 0u;
            ahi[m][i] = active ? q[2 * i + 1] : 0u;
        }
        sx[m] = OUT_I32 ? 1.f : row_scales[m];
    }
    int asum8[M];  // 8 * sum of this lane's codes (the code - 8 offset)
#pragma unroll
    for (int m = 0; m < M; ++m) {
        int s = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s = __builtin_amdgcn_sdot4((int)alo[m][i], 0x01010101, s, false);
            s = __builtin_amdgcn_sdot4((int)ahi[m][i], 0x01010101, s, false);
        }
        asum8[m] = 8 * s;
    }

    // 3. dot products, one partial per (row, activation row) and lane.
    uint32_t part[M][R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo[i] = wv[r][i] & 0x0f0f0f0fu;
            hi[i] = (wv[r][i] >> 4) & 0x0f0f0f0fu;
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            int acc = -asum8[m];  // the code - 8 offset, subtracted up front
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc = __builtin_amdgcn_sdot4((int)lo[i], (int)alo[m][i], acc, false);
                acc = __builtin_amdgcn_sdot4((int)hi[i], (int)ahi[m][i], acc, false);
            }
            if constexpr (FSUM)
                part[m][r] = __float_as_uint(__uint_as_float(r % 2 ? sv[r / 8][(r % 8) / 2] & 0xffff0000u
                                                                   : sv[r / 8][(r % 8) / 2] << 16) *
                                             (float)acc);
            else
                part[m][r] = (uint32_t)acc;
        }
    }

    // 4. sum over the lanes of the wave, then over the waves (fixed order).
    //    The (activation row, weight row) partials go through transposed lane
    //    reductions of up to 32 values at once (4, 2 or 1 activation rows of
    //    8 weight rows), which take fewer lane exchanges than one reduction
    //    per activation row; each is the same binary tree over the lanes, so
    //    the sums are the same bit for bit.
    reduce_rows<M, R, FSUM, 0>(part, lane, s_red[wave]);
    __syncthreads();
    for (int e = threadIdx.x; e < R * M; e += blockDim.x) {
        const int r = e / M, m = e % M;
        const int n = n0 + r;
        uint32_t t = s_red[0][r][m];
        for (int w = 1; w < nw; ++w)
            t = add32<FSUM>(t, s_red[w][r][m]);
        if constexpr (OUT_I32) {
            acc_out[(int64_t)m * lda + n] = (int32_t)t;
        } else {
            float y;
            if constexpr (FSUM) {
                y = __uint_as_float(t) * (sx[m] * x_scale);
                if (bias)
                    y += bf16_to_f32(bias[n]);
            } else {
                y = epilogue_channel((float)(int32_t)t, bf16_to_f32(w_scales[n]), sx[m] * x_scale,
                                     bias ? bf16_to_f32(bias[n]) : 0.f);
            }
            out[(int64_t)m * ldo + n] = f32_to_bf16(y);
        }
    }
}

template <int M, int R>
hipError_t launch_m(bool pg, bool i32, const int8_t *codes, int64_t ldq, const float *rs, int K,
                    const uint8_t *packed, int64_t ldw, const uint16_t *ws, int N, const uint16_t *bias,
                    float xs, uint16_t *out, int64_t ldo, int32_t *acc, int64_t lda, hipStream_t s)
{
    const dim3 grid((unsigned)(N / R));
    const dim3 block((unsigned)(kWave * ((K + 2047) / 2048)));
    if (i32)
        hipLaunchKernelGGL((w4_gemv_kernel<M, R, false, true>), grid, block, 0, s, codes, ldq, rs, K, packed,
                           ldw, ws, N, bias, xs, out, ldo, acc, lda);
    else if (pg)
        hipLaunchKernelGGL((w4_gemv_kernel<M, R, true, false>), grid, block, 0, s, codes, ldq, rs, K, packed,
                           ldw, ws, N, bias, xs, out, ldo, acc, lda);
    else
        hipLaunchKernelGGL((w4_gemv_kernel<M, R, false, false>), grid, block, 0, s, codes, ldq, rs, K, packed,
                           ldw, ws, N, bias, xs, out, ldo, acc, lda);
    return hipGetLastError();
}

}  // namespace


int launch_w4_gemv(const int8_t *codes, int64_t ldq, const float *row_scales, int M, int K,
                   const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, bool per_group, int N,
                   const uint16_t *bias, float x_scale, uint16_t *out, int64_t ldo, int32_t *acc_out,
                   int64_t lda, void *stream)
{
    if (!w4_gemv_supports(M, K) || N % 16 != 0)
        return (int)hipErrorInvalidValue;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool i32 = acc_out != nullptr;
    constexpr int R = CK_GEMV_ROWS;
    hipError_t e;
#define CK_GEMV_M(MM)                                                                                       \
    case MM:                                                                                                \
        e = launch_m<MM, R>(per_group, i32, codes, ldq, row_scales, K, packed, ldw, w_scales, N, bias,     \
                            x_scale, out, ldo, acc_out, lda, s);                                            \
        break;
    switch (M) {
        CK_GEMV_M(1)
        CK_GEMV_M(2)
        CK_GEMV_M(3)
        CK_GEMV_M(4)
        CK_GEMV_M(5)
        CK_GEMV_M(6)
        CK_GEMV_M(7)
        CK_GEMV_M(8)
    default: e = hipErrorInvalidValue; break;
    }
#undef CK_GEMV_M
    return (int)e;
}

}  // namespace ck
