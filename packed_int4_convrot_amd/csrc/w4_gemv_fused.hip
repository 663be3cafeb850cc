// Whole W4A8/W4A4 decode linear for 1 <= M <= 4 activation rows in one launch:
// rotate-quant of the bf16 rows and the packed-int4 GEMV, with one workgroup
// per compute unit.
//
// Prior art: the fused RotateQuant operator of "[PR #155] [Feat][Ascend] Add
// fused RotateQuant backend" ("What this PR does": the group-wise Hadamard
// rotation and the per-row quantisation in one pass) and the register-side
// int4 decode + v_dot4 + rowwise-scale epilogue of "[PR #182] HIP port of
// #176: W4A8 decode GEMV and fused GatedDeltaNet decode" (description).
//
// Why one workgroup per CU.  A decode step is a single ~21 MB weight read, so
// the kernel must have nearly every weight byte in flight from its first
// microsecond.  Many small workgroups per CU do that well, but each then
// rotates the activation rows again (five times per CU for the GEMV on codes'
// 1280 workgroups).  Here a workgroup owns RB blocks of 8 consecutive weight
// rows (all the rows one CU streams) and rotates the rows once.
//
// Two kinds of waves:
//   * streaming waves keep the per-wave layout of the GEMV on codes (wave =
//     one 2048-column slice of one 8-row block, lane = 16 packed bytes of
//     each row, so one load instruction reads 1 KiB of one row).  They issue
//     all their weight loads at once, which stalls their issue while the
//     CU's memory pipeline is full (1.6 us median at the decode workload);
//   * rotation waves (a multiple of 4, one per SIMD each) load the bf16 rows
//     first, rotate them in 8-column chunks (butterfly strides 1, 2, 4 in
//     registers, the rest across lanes), take the row absmax (DPP within a
//     wave, an LDS atomic maximum and arrival count across the rotation
//     waves), quantise with rne(y * qmax / absmax) -- the same fp32
//     operations in the same order as the rotate-quant kernel, so the codes
//     are bit-identical to it -- and write the codes to LDS, even and odd
//     columns of each 32-column piece apart (the order of the nibble decode).
// Two barriers: the first publishes the LDS counters (after the rotation
// waves' activation loads, before any weight load); the second hands the
// codes to the streaming waves.  Each streaming wave then forms dot products
// (unsigned nibbles x codes, v_dot4_i32_i8, minus 8 * sum(codes)), applies
// the per-group scale and sums over its lanes by the transposed reduction;
// the last of the S slices of a row block to finish (an LDS arrival count)
// sums the slices in slice order and writes the outputs.  These are the
// operations of the GEMV on codes, so the outputs equal rotate-quant + GEMV
// bit for bit.
// LDS: M * K bytes of codes; just over 80 KiB is requested whenever the grid
// fits the chip, so that no CU receives two workgroups.
#include <mutex>

#include "ck_device.h"
#include "gemv_reduce.h"
#include "launch.h"
#include "rotate_rows.h"

namespace ck {
namespace {

constexpr int kRows = 8;  // weight rows per wave

// LDS of a workgroup besides the codes.
template <int M>
struct FusedShared {
    uint32_t red[kFusedMaxStreamWaves][kRows][M];  // per-wave lane sums of the streaming waves
    uint32_t amax[M];                                // row absmax (fp32 bits; non-negative, so ordered as integers)
    uint32_t arrived;                                // rotation waves whose maxima are in amax
    uint32_t done[kFusedMaxStreamWaves];             // slices of each row block summed into red
};

// Streaming waves: an 8-row block n0 .. n0 + 7 and the 2048-column slice of
// wave % S; lane l owns columns kbase = 2048 (wave % S) + 32 l .. + 31.
template <int M, int G, bool PER_GROUP>
__device__ __forceinline__ void stream_role(float qmax, int K, const uint8_t *__restrict__ packed, int64_t ldw,
                                            const uint16_t *__restrict__ w_scales, int N,
                                            const uint16_t *__restrict__ bias, float x_scale,
                                            uint16_t *__restrict__ out, int64_t ldo, int S, int wave, int lane,
                                            int n0, bool has_rows, const uint8_t *s_codes, FusedShared<M> &sh)
{
    constexpr float kInvSqrtG = G == 16 ? 0.25f : G == 64 ? 0.125f : 0.0625f;
    constexpr bool FSUM = PER_GROUP;  // partials are fp32 (scaled) or exact int32
    const int kbase = 2048 * (wave % S) + 32 * lane;
    const bool active = has_rows && kbase < K;
    const int kc = kbase < K ? kbase : K - 32;  // every address stays inside the row

    // The weight scales and the 8 weight rows go out right after the first
    // barrier, all in flight at once.  Their issue stalls while the CU's
    // memory pipeline is full, which is why the rotation runs in other waves.
    // (Issuing some of them before the first barrier measured slower: the
    // barrier, and with it the rotation, then waits for their issue.)
    if (threadIdx.x < kFusedMaxStreamWaves)
        sh.done[threadIdx.x] = 0;
    __syncthreads();  // the counters are published
    u32x4 sv = {0u, 0u, 0u, 0u};
    if constexpr (PER_GROUP)
        sv = *reinterpret_cast<const u32x4 *>(w_scales + (int64_t)(kc / 64) * N + n0);
    u32x4 wv[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
        wv[r] = load_nt16(packed + (int64_t)(n0 + r) * ldw + kc / 2);
    __syncthreads();  // the codes are in LDS

    // Every path below uses the weights (waves without rows compute on rows
    // 0 .. 7 and drop the result), so the compiler cannot sink the loads
    // into a conditional block after the barriers.
    // This lane's codes: even columns in alo, odd ones in ahi.
    uint32_t alo[M][4], ahi[M][4];
    int asum8[M];  // 8 * sum of the lane's codes (the code - 8 offset)
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const u32x4 e = active ? *reinterpret_cast<const u32x4 *>(s_codes + m * K + kbase) : u32x4{0u, 0u, 0u, 0u};
        const u32x4 o = active ? *reinterpret_cast<const u32x4 *>(s_codes + m * K + kbase + 16)
                               : u32x4{0u, 0u, 0u, 0u};
        int s = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            alo[m][i] = e[i];
            ahi[m][i] = o[i];
            s = __builtin_amdgcn_sdot4((int)alo[m][i], 0x01010101, s, false);
            s = __builtin_amdgcn_sdot4((int)ahi[m][i], 0x01010101, s, false);
        }
        asum8[m] = 8 * s;
    }

    // Dot products, one partial per (activation row, weight row) and lane.
    uint32_t part[M][kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
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
                part[m][r] = __float_as_uint(
                    __uint_as_float(r % 2 ? sv[r / 2] & 0xffff0000u : sv[r / 2] << 16) * (float)acc);
            else
                part[m][r] = (uint32_t)acc;
        }
    }

    // Sum over the lanes of the wave, then over the S slices of the row
    // block: the last slice to finish sums them in slice order and writes the
    // outputs.
    reduce_rows<M, kRows, FSUM, 0>(part, lane, sh.red[wave]);
    if (!has_rows)
        return;
    const int rbl = wave / S;
    uint32_t prior = 0;
    if (lane == 0)
        prior = __hip_atomic_fetch_add(&sh.done[rbl], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__builtin_amdgcn_readfirstlane(prior) != (uint32_t)(S - 1))
        return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (lane < kRows * M) {
        const int r = lane / M, m = lane % M;
        const int n = n0 + r;
        uint32_t t = sh.red[rbl * S][r][m];
        for (int k = 1; k < S; ++k)
            t = add32<FSUM>(t, sh.red[rbl * S + k][r][m]);
        const float am = __uint_as_float(sh.amax[m]);
        const float sx = am > 0.f ? (am / qmax) * kInvSqrtG : 1.0f;
        float y;
        if constexpr (FSUM) {
            y = __uint_as_float(t) * (sx * x_scale);
            if (bias)
                y += bf16_to_f32(bias[n]);
        } else {
            y = epilogue_channel((float)(int32_t)t, bf16_to_f32(w_scales[n]), sx * x_scale,
                                 bias ? bf16_to_f32(bias[n]) : 0.f);
        }
        out[(int64_t)m * ldo + n] = f32_to_bf16(y);
    }
}

// CPR: 8-column rotation chunks per rotation thread and row.  Workgroup
// (blockDim.x = 64 * (NWS + nwr)): streaming wave w < NWS serves row block
// lb * RB + w / S, columns [2048 (w % S), 2048 (w % S) + 2048); the nwr
// rotation waves after them rotate and quantise the M rows.  Every wave meets
// the same two barriers.
template <int M, int G, bool PER_GROUP, int CPR>
__global__ __launch_bounds__(1024) void w4_gemv_fused_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, float qmax, int K, const uint8_t *__restrict__ packed,
    int64_t ldw, const uint16_t *__restrict__ w_scales, int N, const uint16_t *__restrict__ bias,
    float x_scale, uint16_t *__restrict__ out, int64_t ldo, int S, int RB, int NWS)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t s_codes[];  // [M][K]
    __shared__ FusedShared<M> sh;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (wave >= NWS) {
        const int nwr = (int)blockDim.x / kWave - NWS;
        // Chunk c is columns 8 (c % 4) .. + 7 of 32-column piece c / 4: its even
        // columns go to bytes 4 (c % 4) .. + 3 of the piece's first 16 bytes, its
        // odd columns to the same bytes of the next 16.
        rotate_rows<M, G, CPR, false, false>(x, ldx, qmax, K, (int)threadIdx.x - kWave * NWS, kWave * nwr, nwr, lane, sh.amax,
                               &sh.arrived, [&](int m, int c, uint32_t even, uint32_t odd) {
                                   uint8_t *piece = s_codes + m * K + 32 * (c >> 2) + 4 * (c & 3);
                                   *reinterpret_cast<uint32_t *>(piece) = even;
                                   *reinterpret_cast<uint32_t *>(piece + 16) = odd;
                               });
    } else {
        const int rb = xcd_block(blockIdx.x, gridDim.x) * RB + wave / S;
        const bool has_rows = rb < N / kRows;
        // a wave past the last row block loads (and drops) rows 0 .. 7
        stream_role<M, G, PER_GROUP>(qmax, K, packed, ldw, w_scales, N, bias, x_scale, out, ldo, S, wave, lane,
                                     has_rows ? rb * kRows : 0, has_rows, s_codes, sh);
    }
}

template <int M, int G, bool PG, int CPR>
hipError_t launch_k(const FusedGemvShape &sh, const uint16_t *x, int64_t ldx, float qmax, int K,
                    const uint8_t *packed, int64_t ldw, const uint16_t *ws, int N, const uint16_t *bias,
                    float xs, uint16_t *out, int64_t ldo, hipStream_t s)
{
    // Only the shapes w4_gemv_fused_shape() allows are instantiated.
    if constexpr (M * CPR > kFusedMaxChunks) {
        return hipErrorInvalidValue;
    } else {
        auto kern = w4_gemv_fused_kernel<M, G, PG, CPR>;
        // The largest request of any shape: M * K codes, or just over 80 KiB.
        constexpr int kMaxLds = M * 2048 * kGemvMaxWaves > 81 * 1024 ? M * 2048 * kGemvMaxWaves : 81 * 1024;
        static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
        if (attr != hipSuccess)
            return attr;
        hipLaunchKernelGGL(kern, dim3((unsigned)sh.nb), dim3((unsigned)((sh.nws + sh.nwr) * kWave)),
                           (size_t)sh.lds, s, x, ldx, qmax, K, packed, ldw, ws, N, bias, xs, out, ldo, sh.s,
                           sh.rb, sh.nws);
        return hipGetLastError();
    }
}

template <int M, int G, bool PG>
hipError_t launch_mg(const FusedGemvShape &sh, const uint16_t *x, int64_t ldx, float qmax, int K,
                     const uint8_t *packed, int64_t ldw, const uint16_t *ws, int N, const uint16_t *bias,
                     float xs, uint16_t *out, int64_t ldo, hipStream_t s)
{
    switch (sh.cpr) {
    case 1: return launch_k<M, G, PG, 1>(sh, x, ldx, qmax, K, packed, ldw, ws, N, bias, xs, out, ldo, s);
    case 2: return launch_k<M, G, PG, 2>(sh, x, ldx, qmax, K, packed, ldw, ws, N, bias, xs, out, ldo, s);
    case 4: return launch_k<M, G, PG, 4>(sh, x, ldx, qmax, K, packed, ldw, ws, N, bias, xs, out, ldo, s);
    case 8: return launch_k<M, G, PG, 8>(sh, x, ldx, qmax, K, packed, ldw, ws, N, bias, xs, out, ldo, s);
    default: return hipErrorInvalidValue;
    }
}

template <int M>
hipError_t launch_m(const FusedGemvShape &sh, int G, bool pg, const uint16_t *x, int64_t ldx, float qmax, int K,
                    const uint8_t *packed, int64_t ldw, const uint16_t *ws, int N, const uint16_t *bias,
                    float xs, uint16_t *out, int64_t ldo, hipStream_t s)
{
#define CK_FG_G(GG)                                                                                              \
    return pg ? launch_mg<M, GG, true>(sh, x, ldx, qmax, K, packed, ldw, ws, N, bias, xs, out, ldo, s)          \
              : launch_mg<M, GG, false>(sh, x, ldx, qmax, K, packed, ldw, ws, N, bias, xs, out, ldo, s);
    switch (G) {
    case 16: CK_FG_G(16)
    case 64: CK_FG_G(64)
    case 256: CK_FG_G(256)
    default: return hipErrorInvalidValue;
    }
#undef CK_FG_G
}

}  // namespace

int device_cu_count()
{
    constexpr int kMaxDevices = 64;
    static std::once_flag once[kMaxDevices];
    static int counts[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 256;
    std::call_once(once[dev], [dev] {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        counts[dev] = n;
    });
    return counts[dev];
}

int launch_w4_gemv_fused(const uint16_t *x, int64_t ldx, int G, int qmax, int M, int K, const uint8_t *packed,
                         int64_t ldw, const uint16_t *w_scales, bool per_group, int N, const uint16_t *bias,
                         float x_scale, uint16_t *out, int64_t ldo, void *stream)
{
    FusedGemvShape sh;
    if (!w4_gemv_fused_shape(M, K, N, device_cu_count(), sh))
        return (int)hipErrorInvalidValue;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const float q = (float)qmax;
    switch (M) {
    case 1: return (int)launch_m<1>(sh, G, per_group, x, ldx, q, K, packed, ldw, w_scales, N, bias, x_scale, out, ldo, s);
    case 2: return (int)launch_m<2>(sh, G, per_group, x, ldx, q, K, packed, ldw, w_scales, N, bias, x_scale, out, ldo, s);
    case 3: return (int)launch_m<3>(sh, G, per_group, x, ldx, q, K, packed, ldw, w_scales, N, bias, x_scale, out, ldo, s);
    case 4: return (int)launch_m<4>(sh, G, per_group, x, ldx, q, K, packed, ldw, w_scales, N, bias, x_scale, out, ldo, s);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace ck
