// Rotate-quant of a few bf16 rows inside one workgroup, shared by the
// one-launch decode kernels (w4_gemv_fused.hip, w4_skinny_fused.hip).
//
// The group-wise Hadamard rotation and per-row absmax quantisation of the
// ConvRot method ("feat: support packed INT4 convrot models", Summary; the
// fused operator of "[PR #155] [Feat][Ascend] Add fused RotateQuant backend",
// "What this PR does"), in 8-column chunks: butterfly strides 1, 2, 4 in
// registers, the larger strides across lanes, the absmax by DPP within a wave
// and an LDS atomic maximum across the rotation waves.  The fp32 operations
// and their order are those of the rotate-quant kernel, so the codes match it
// bit for bit.
#pragma once
#include "ck_device.h"
#include "gemv_reduce.h"

namespace ck {

__device__ __forceinline__ uint32_t rne_byte(float t) { return __float_as_uint(t + 12582912.0f); }

__device__ __forceinline__ uint32_t pack4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3)
{
    const uint32_t p01 = perm(b1, b0, 0x0C0C0400u);
    const uint32_t p23 = perm(b3, b2, 0x0C0C0400u);
    return perm(p23, p01, 0x05040100u);
}

// Cross-lane butterfly on U chunks of 8 values: the lower lane of a pair keeps
// a + b, the upper one a - b (fma(b, -1, a), one rounding).  SWIZZLE: the
// partner's value through ds_swizzle (the LDS pipe) for every lane distance,
// one VALU operation per value; otherwise DPP for distances 1 and 2 (a VALU
// move each, but shorter latency).
template <int MASK, int U, bool SWIZZLE>
__device__ __forceinline__ void lane_stage8(float (&v)[U][8], int lane)
{
    const float sgn = (lane & MASK) ? -1.f : 1.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float p = SWIZZLE ? __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v[u][r]), 0x1F | (MASK << 10)))
                                    : __uint_as_float(lane_xor_u<MASK>(__float_as_uint(v[u][r])));
            v[u][r] = __builtin_fmaf(v[u][r], sgn, p);
        }
}

__device__ __forceinline__ float wave_max(float am)
{
    am = fmaxf(am, __uint_as_float(lane_xor_u<1>(__float_as_uint(am))));
    am = fmaxf(am, __uint_as_float(lane_xor_u<2>(__float_as_uint(am))));
    am = fmaxf(am, __uint_as_float(lane_mirror8_u(__float_as_uint(am))));
    am = fmaxf(am, __uint_as_float(lane_mirror16_u(__float_as_uint(am))));
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(am), 0)),
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(am), 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(am), 32)),
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(am), 48))));
}

// Maximum over the rotation waves of the per-wave maxima of row m (fp32 bits
// of non-negative values, so the unsigned order is the float order).
__device__ __forceinline__ uint32_t row_max_bits(const uint32_t *wave_max_bits, int m, int M, int nwr)
{
    uint32_t a = 0;
    for (int w = 0; w < nwr; ++w)
        a = max(a, wave_max_bits[w * M + m]);
    return a;
}

// The same maximum formed by a whole wave (every lane active, nwr <= 8): lane l
// reads wave l % 8's maximum, three lane exchanges combine the 8, and the result
// is wave-uniform.  One LDS read per row instead of nwr.
__device__ __forceinline__ uint32_t row_max_bits_wave(const uint32_t *wave_max_bits, int m, int M, int nwr,
                                                      int lane)
{
    uint32_t a = (lane & 7) < nwr ? wave_max_bits[(lane & 7) * M + m] : 0u;
    a = max(a, lane_xor_u<1>(a));
    a = max(a, lane_xor_u<2>(a));
    a = max(a, lane_mirror8_u(a));
    return __builtin_amdgcn_readfirstlane(a);
}

// Rotation waves of a one-launch decode kernel: thread rt of the rstride
// rotation threads holds chunks rt + j * rstride (j < CPR) of every row.  A
// G-column group is G / 8 consecutive chunks on neighbouring lanes of one wave
// (rstride and nchunk are multiples of G / 8).  The row maxima are combined
// across the rotation waves in one of two ways:
//   WAVE_MAXIMA false: amax[M] and *arrived are LDS words that this function
//     zeroes before the workgroup's first barrier; each wave posts its maxima
//     by an LDS atomic maximum and waits on the arrival count; the row maxima
//     stay in amax for the epilogue;
//   WAVE_MAXIMA true: wave w of the rotation waves stores its maxima to
//     amax[w * M + m] (nwr * M LDS words, nothing to zero), the workgroup's
//     first barrier publishes them, and every reader takes the maximum over
//     the waves (as unsigned integers, which orders non-negative floats; at
//     most 8 waves); the other waves may then meet the first barrier whenever
//     they like.
// SWIZZLE: every cross-lane butterfly stage through ds_swizzle (lane_stage8),
// one VALU operation fewer per value at lane distances 1 and 2 (for a rotation
// bounded by its VALU work rather than its latency).  Each chunk's 8 codes go
// out through store(m, c, even, odd): even holds the codes of columns 8c + 0,
// 2, 4, 6 (bytes 0..3), odd those of 8c + 1, 3, 5, 7.  Barriers: the
// workgroup's two (counters published or maxima published; codes stored), met
// by every other wave in the same order.
template <int M, int G, int CPR, bool WAVE_MAXIMA, bool SWIZZLE, typename Store>
__device__ __forceinline__ void rotate_rows(const uint16_t *__restrict__ x, int64_t ldx, float qmax, int K,
                                            int rt, int rstride, int nwr, int lane, uint32_t *amax,
                                            uint32_t *arrived, Store store)
{
    const int nchunk = K / 8;
    u32x4 xraw[M][CPR];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < CPR; ++j) {
            const int c = rt + j * rstride;
            xraw[m][j] = *reinterpret_cast<const u32x4 *>(x + (int64_t)m * ldx + 8 * (c < nchunk ? c : nchunk - 1));
        }
    if constexpr (!WAVE_MAXIMA) {
        if (rt == 0) {
            *arrived = 0;
#pragma unroll
            for (int m = 0; m < M; ++m)
                amax[m] = 0;
        }
        __syncthreads();  // the counters are published
    }

    float v[M * CPR][8];
#pragma unroll
    for (int u = 0; u < M * CPR; ++u) {
        const bool live = rt + (u % CPR) * rstride < nchunk;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w = live ? xraw[u / CPR][u % CPR][j] : 0u;
            v[u][2 * j] = __uint_as_float(w << 16);
            v[u][2 * j + 1] = __uint_as_float(w & 0xffff0000u);
        }
    }
#pragma unroll
    for (int h = 1; h < 8 && h < G; h <<= 1)
#pragma unroll
        for (int u = 0; u < M * CPR; ++u)
#pragma unroll
            for (int r = 0; r < 8; ++r)
                if ((r & h) == 0) {
                    const float a = v[u][r], b = v[u][r + h];
                    v[u][r] = a + b;
                    v[u][r + h] = a - b;
                }
    if constexpr (G >= 16) lane_stage8<1, M * CPR, SWIZZLE>(v, lane);
    if constexpr (G >= 32) lane_stage8<2, M * CPR, SWIZZLE>(v, lane);
    if constexpr (G >= 64) lane_stage8<4, M * CPR, SWIZZLE>(v, lane);
    if constexpr (G >= 128) lane_stage8<8, M * CPR, SWIZZLE>(v, lane);
    if constexpr (G >= 256) lane_stage8<16, M * CPR, SWIZZLE>(v, lane);
    // Row absmax over the rotation waves.  Atomic form: LDS atomic maximum, then
    // an arrival count that every rotation wave waits on (they are all resident
    // in this workgroup, so the wait ends).  Per-wave form: each wave's maxima,
    // then the workgroup's first barrier.
#pragma unroll
    for (int m = 0; m < M; ++m) {
        float am = 0.f;
#pragma unroll
        for (int j = 0; j < CPR; ++j)
#pragma unroll
            for (int r = 0; r < 8; ++r)
                am = fmaxf(am, fabsf(v[m * CPR + j][r]));
        am = wave_max(am);
        if (lane == 0) {
            if constexpr (WAVE_MAXIMA)
                amax[(rt / kWave) * M + m] = __float_as_uint(am);
            else
                atomicMax(&amax[m], __float_as_uint(am));
        }
    }
    if constexpr (WAVE_MAXIMA) {
        __syncthreads();  // the per-wave maxima are published
    } else {
        if (lane == 0)
            __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        while (__builtin_amdgcn_readfirstlane(
                   __hip_atomic_load(arrived, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) < (uint32_t)nwr)
            __builtin_amdgcn_s_sleep(1);
    }
    // Quantise: rne(y * qmax / absmax), the codes of the rotate-quant kernel
    // bit for bit.
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float am = __uint_as_float(WAVE_MAXIMA ? row_max_bits_wave(amax, m, M, nwr, lane) : amax[m]);
        const float inv = am > 0.f ? qmax / am : 0.f;
#pragma unroll
        for (int j = 0; j < CPR; ++j) {
            const int c = rt + j * rstride;
            const float(&y)[8] = v[m * CPR + j];
            uint32_t b[8];
#pragma unroll
            for (int r = 0; r < 8; ++r)
                b[r] = rne_byte(y[r] * inv);
            if (c < nchunk)
                store(m, c, pack4(b[0], b[2], b[4], b[6]), pack4(b[1], b[3], b[5], b[7]));
        }
    }
    __syncthreads();  // the codes are in LDS
}

}  // namespace ck
