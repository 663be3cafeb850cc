// Decode GEMV for 1 <= M <= 8 activation rows, optionally (M = 1) fused with
// the rotate-quant of that row.
//
// Prior art: the W4A8 decode GEMV of "[PR #182] HIP port of #176: W4A8 decode
// GEMV and fused GatedDeltaNet decode" (description): register-side int4
// decode feeding v_dot4 integer dot products and a rowwise x weight-scale
// epilogue, with no decoded weight copy in memory.  The fused form follows the
// activation-side fusion of "[PR #155] [Feat][Ascend] Add fused RotateQuant
// backend" one step further: the rotate-quant of the few activation rows runs
// inside the GEMV launch, while the weights are already streaming in.
//
// Layout (built for HBM streaming, one K slice per wave):
//   * wave w of a block owns columns k in [2048 w, 2048 w + 2048); lane l owns
//     the 32 columns starting at 2048 w + 32 l, i.e. 16 packed bytes of every
//     weight row, so one load instruction reads 1 KiB of contiguous weights;
//   * a block handles R consecutive weight rows; each lane issues its R
//     16-byte weight loads first, then builds its activation operands (int8
//     codes for its 32 columns, split into even / odd k to match the nibble
//     decode) from either given codes or, fused, from bf16 x:
//       load 32 bf16 -> fp32 -> butterflies of H_G (in registers for strides
//       < 32, DPP / ds_swizzle across lanes above) -> row absmax over all lanes
//       and waves -> codes = rne(y * qmax / absmax) (the same arithmetic as the
//       rotate-quant kernel, so the codes are bit-identical to it);
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

constexpr int kMaxWaves = 8;  // K <= 16384
#ifndef CK_GEMV_ROWS
#define CK_GEMV_ROWS 8  // weight rows per block (8 or 16)
#endif
// The fused form pays the rotation once per block; measured on MI355X it is
// faster than a separate rotate-quant launch only for a single activation row.
constexpr int kMaxFusedRows = 1;
#ifndef CK_GEMV_MAX_M
#define CK_GEMV_MAX_M 8
#endif

// One cross-lane butterfly stage on 32 values per lane (fused rotation).
template <int MASK>
__device__ __forceinline__ void lane_stage32(float (&v)[32], int lane)
{
    const float sgn = (lane & MASK) ? -1.f : 1.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        const float p = __uint_as_float(lane_xor_u<MASK>(__float_as_uint(v[r])));
        v[r] = __builtin_fmaf(v[r], sgn, p);
    }
}

__device__ __forceinline__ uint32_t rne_byte(float t) { return __float_as_uint(t + 12582912.0f); }

__device__ __forceinline__ uint32_t pack4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3)
{
    const uint32_t p01 = perm(b1, b0, 0x0C0C0400u);
    const uint32_t p23 = perm(b3, b2, 0x0C0C0400u);
    return perm(p23, p01, 0x05040100u);
}

template <int M, int R, int G, bool PER_GROUP, bool OUT_I32>
__global__ __launch_bounds__(kMaxWaves * kWave) void w4_gemv_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, float qmax, const int8_t *__restrict__ codes,
    int64_t ldq, const float *__restrict__ row_scales, int K, const uint8_t *__restrict__ packed,
    int64_t ldw, const uint16_t *__restrict__ w_scales, int N, const uint16_t *__restrict__ bias,
    float x_scale, uint16_t *__restrict__ out, int64_t ldo, int32_t *__restrict__ acc_out, int64_t lda)
{
    constexpr bool FUSED = G != 0;
    constexpr bool FSUM = PER_GROUP && !OUT_I32;  // partials are fp32 (scaled) or exact int32
    __shared__ float s_am[kMaxWaves][M];
    __shared__ uint32_t s_red[kMaxWaves][R][M];

    const int nw = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int n0 = xcd_block(blockIdx.x, gridDim.x) * R;
    const int kbase = 2048 * wave + 32 * lane;
    const bool active = kbase < K;
    const int kc = active ? kbase : K - 32;  // clamped: every address stays inside the row

    // 1. Loads, in this order: the activations (small, usually L2-resident),
    //    the weight scales, then the R weight rows.  Loads retire in issue
    //    order, so the activation work below waits only for the activations,
    //    and row r's dot products only for rows 0..r, while the remaining
    //    weight rows are still streaming in.
    u32x4 araw[M][FUSED ? 4 : 2];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        if constexpr (FUSED) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                araw[m][c] = *reinterpret_cast<const u32x4 *>(x + (int64_t)m * ldx + kc + 8 * c);
        } else {
#pragma unroll
            for (int c = 0; c < 2; ++c)
                araw[m][c] = *reinterpret_cast<const u32x4 *>(codes + (int64_t)m * ldq + kc + 16 * c);
        }
    }
    uint16_t sv[PER_GROUP ? R : 1];
    if constexpr (PER_GROUP) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            sv[r] = w_scales[(int64_t)(kc / 64) * N + n0 + r];
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
    if constexpr (FUSED) {
        constexpr float kInvSqrtG = G == 16 ? 0.25f : G == 64 ? 0.125f : 0.0625f;
        float inv[M];
        float vv[M][32];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float(&v)[32] = vv[m];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4 w = araw[m][c];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[8 * c + 2 * j] = active ? __uint_as_float(w[j] << 16) : 0.f;
                    v[8 * c + 2 * j + 1] = active ? __uint_as_float(w[j] & 0xffff0000u) : 0.f;
                }
            }
            // Butterflies of H_G: strides 1 .. min(G/2, 16) in registers, then across lanes.
#pragma unroll
            for (int h = 1; h < 32 && h < G; h <<= 1)
#pragma unroll
                for (int r = 0; r < 32; ++r)
                    if ((r & h) == 0) {
                        const float a = v[r], b = v[r + h];
                        v[r] = a + b;
                        v[r + h] = a - b;
                    }
            if constexpr (G >= 64) lane_stage32<1>(v, lane);
            if constexpr (G >= 128) lane_stage32<2>(v, lane);
            if constexpr (G >= 256) lane_stage32<4>(v, lane);
            float am = 0.f;
#pragma unroll
            for (int r = 0; r < 32; ++r)
                am = fmaxf(am, fabsf(v[r]));
            am = fmaxf(am, __uint_as_float(lane_xor_u<1>(__float_as_uint(am))));
            am = fmaxf(am, __uint_as_float(lane_xor_u<2>(__float_as_uint(am))));
            am = fmaxf(am, __uint_as_float(lane_xor_u<4>(__float_as_uint(am))));
            am = fmaxf(am, __uint_as_float(lane_xor_u<8>(__float_as_uint(am))));
            am = fmaxf(am, __uint_as_float(lane_xor_u<16>(__float_as_uint(am))));
            am = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(am), 0)),
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(am), 32)));
            if (lane == 0)
                s_am[wave][m] = am;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float am = s_am[0][m];
            for (int w = 1; w < nw; ++w)
                am = fmaxf(am, s_am[w][m]);
            inv[m] = am > 0.f ? qmax / am : 0.f;
            sx[m] = am > 0.f ? (am / qmax) * kInvSqrtG : 1.0f;
            const float(&v)[32] = vv[m];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t b[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    b[j] = rne_byte(v[8 * i + j] * inv[m]);
                alo[m][i] = pack4(b[0], b[2], b[4], b[6]);
                ahi[m][i] = pack4(b[1], b[3], b[5], b[7]);
            }
        }
    } else {
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
            int acc = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc = __builtin_amdgcn_sdot4((int)lo[i], (int)alo[m][i], acc, false);
                acc = __builtin_amdgcn_sdot4((int)hi[i], (int)ahi[m][i], acc, false);
            }
            acc -= asum8[m];
            if constexpr (FSUM)
                part[m][r] = __float_as_uint(bf16_to_f32(sv[r]) * (float)acc);
            else
                part[m][r] = (uint32_t)acc;
        }
    }

    // 4. sum over the lanes of the wave, then over the waves (fixed order).
    constexpr int kShift = R == 16 ? 2 : 3;
    const int row = lane >> kShift;
    const bool owner = (lane & ((1 << kShift) - 1)) == 0;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const uint32_t t = transposed_row_sum<R, FSUM>(part[m], lane);
        if (owner)
            s_red[wave][row][m] = t;
    }
    __syncthreads();
    if (threadIdx.x < R * M) {
        const int r = threadIdx.x / M, m = threadIdx.x % M;
        const int n = n0 + r;
        uint32_t t = s_red[0][r][m];
        for (int w = 1; w < nw; ++w)
            t = add32<FSUM>(t, s_red[w][r][m]);
        if constexpr (OUT_I32) {
            acc_out[(int64_t)m * lda + n] = (int32_t)t;
        } else {
            float y = FSUM ? __uint_as_float(t) : bf16_to_f32(w_scales[n]) * (float)(int32_t)t;
            y *= sx[m] * x_scale;
            if (bias)
                y += bf16_to_f32(bias[n]);
            out[(int64_t)m * ldo + n] = f32_to_bf16(y);
        }
    }
}

template <int M, int R, int G>
hipError_t launch_mg(bool pg, bool i32, const uint16_t *x, int64_t ldx, float qmax, const int8_t *codes,
                     int64_t ldq, const float *rs, int K, const uint8_t *packed, int64_t ldw,
                     const uint16_t *ws, int N, const uint16_t *bias, float xs, uint16_t *out, int64_t ldo,
                     int32_t *acc, int64_t lda, hipStream_t s)
{
    const dim3 grid((unsigned)(N / R));
    const dim3 block((unsigned)(kWave * ((K + 2047) / 2048)));
    if (i32) {
        if constexpr (G == 0)
            hipLaunchKernelGGL((w4_gemv_kernel<M, R, G, false, true>), grid, block, 0, s, x, ldx, qmax, codes,
                               ldq, rs, K, packed, ldw, ws, N, bias, xs, out, ldo, acc, lda);
    } else if (pg) {
        hipLaunchKernelGGL((w4_gemv_kernel<M, R, G, true, false>), grid, block, 0, s, x, ldx, qmax, codes,
                           ldq, rs, K, packed, ldw, ws, N, bias, xs, out, ldo, acc, lda);
    } else {
        hipLaunchKernelGGL((w4_gemv_kernel<M, R, G, false, false>), grid, block, 0, s, x, ldx, qmax, codes,
                           ldq, rs, K, packed, ldw, ws, N, bias, xs, out, ldo, acc, lda);
    }
    return hipGetLastError();
}

template <int M, int R>
hipError_t launch_m(int G, bool pg, bool i32, const uint16_t *x, int64_t ldx, float qmax,
                    const int8_t *codes, int64_t ldq, const float *rs, int K, const uint8_t *packed,
                    int64_t ldw, const uint16_t *ws, int N, const uint16_t *bias, float xs,
                    uint16_t *out, int64_t ldo, int32_t *acc, int64_t lda, hipStream_t s)
{
    if (G == 0)
        return launch_mg<M, R, 0>(pg, i32, x, ldx, qmax, codes, ldq, rs, K, packed, ldw, ws, N, bias, xs, out, ldo, acc, lda, s);
    if constexpr (M <= kMaxFusedRows) {
        switch (G) {
        case 16: return launch_mg<M, R, 16>(pg, false, x, ldx, qmax, codes, ldq, rs, K, packed, ldw, ws, N, bias, xs, out, ldo, acc, lda, s);
        case 64: return launch_mg<M, R, 64>(pg, false, x, ldx, qmax, codes, ldq, rs, K, packed, ldw, ws, N, bias, xs, out, ldo, acc, lda, s);
        case 256: return launch_mg<M, R, 256>(pg, false, x, ldx, qmax, codes, ldq, rs, K, packed, ldw, ws, N, bias, xs, out, ldo, acc, lda, s);
        default: break;
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool w4_gemv_supports(int64_t M, int64_t K) { return M >= 1 && M <= CK_GEMV_MAX_M && K <= 2048 * kMaxWaves; }
bool w4_gemv_fused_supports(int64_t M, int64_t K) { return w4_gemv_supports(M, K) && M <= kMaxFusedRows; }

int launch_w4_gemv(const uint16_t *x, int64_t ldx, int G, int qmax, const int8_t *codes, int64_t ldq,
                   const float *row_scales, int M, int K, const uint8_t *packed, int64_t ldw,
                   const uint16_t *w_scales, bool per_group, int N, const uint16_t *bias, float x_scale,
                   uint16_t *out, int64_t ldo, int32_t *acc_out, int64_t lda, void *stream)
{
    if (!w4_gemv_supports(M, K) || N % 16 != 0)
        return (int)hipErrorInvalidValue;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool i32 = acc_out != nullptr;
    const float q = (float)qmax;
    constexpr int R = CK_GEMV_ROWS;
    hipError_t e;
    switch (M) {
    case 1: e = launch_m<1, R>(G, per_group, i32, x, ldx, q, codes, ldq, row_scales, K, packed, ldw, w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s); break;
    case 2: e = launch_m<2, R>(G, per_group, i32, x, ldx, q, codes, ldq, row_scales, K, packed, ldw, w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s); break;
    case 3: e = launch_m<3, R>(G, per_group, i32, x, ldx, q, codes, ldq, row_scales, K, packed, ldw, w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s); break;
    case 4: e = launch_m<4, R>(G, per_group, i32, x, ldx, q, codes, ldq, row_scales, K, packed, ldw, w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s); break;
#if CK_GEMV_MAX_M > 4
    case 5: e = launch_m<5, R>(G, per_group, i32, x, ldx, q, codes, ldq, row_scales, K, packed, ldw, w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s); break;
    case 6: e = launch_m<6, R>(G, per_group, i32, x, ldx, q, codes, ldq, row_scales, K, packed, ldw, w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s); break;
    case 7: e = launch_m<7, R>(G, per_group, i32, x, ldx, q, codes, ldq, row_scales, K, packed, ldw, w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s); break;
    case 8: e = launch_m<8, R>(G, per_group, i32, x, ldx, q, codes, ldq, row_scales, K, packed, ldw, w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s); break;
#endif
    default: e = hipErrorInvalidValue; break;
    }
    return (int)e;
}

}  // namespace ck
