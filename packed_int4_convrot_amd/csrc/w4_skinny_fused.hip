// Whole W4A8/W4A4 linear for 1 <= M <= 8 activation rows in one launch: the
// rotate-quant of the bf16 rows and the packed-int4 matmul on int8 MFMA, one
// workgroup per compute unit.  The linear takes it for 5 to 8 rows when the
// weights span at least 8192 rows; every shape is reachable through a test
// entry point.
//
// Prior art: the fused RotateQuant operator of "[PR #155] [Feat][Ascend] Add
// fused RotateQuant backend" ("What this PR does") and the register-side int4
// decode + rowwise-scale epilogue of "[PR #182] HIP port of #176: W4A8 decode
// GEMV and fused GatedDeltaNet decode" (description).
//
// The one-launch decode GEMV (w4_gemv_fused.hip) forms its dot products on the
// VALU, whose work grows with the row count (and its rotation threads hold at
// most 4 rows).  Here the products run on v_mfma_i32_16x16x64_i8 as in the
// few-row kernel (w4_skinny.hip).  The group loop still costs about 15 VALU
// instructions per MFMA (nibble decode, int -> fp32, the per-group scale fold),
// so below 5 rows the VALU GEMV, which folds one scale per 32 weights, stays
// faster; and every CU rotates all M rows, which is what bounds the kernel at
// 8 rows once a CU's share of the weights is small.
//
// Workgroup: kSfRotWaves rotation waves first, then nws = T * S streaming waves.
//   * rotation waves: rotate_rows() with one 8-column chunk per thread and row
//     (K <= 4096); each wave posts its row maxima to LDS, the first barrier
//     publishes them, and the codes go to LDS in the MFMA operand order below
//     before the second barrier.  Being first in the workgroup, their x loads
//     enter the CU's memory pipeline ahead of the weight stream;
//   * the workgroup owns `rows` consecutive weight rows (a multiple of 8): T
//     tiles of 16 rows, the last possibly of 8; streaming wave (t, s) streams
//     K-groups 32 s .. 32 s + 31 of tile t from its first instructions on: the
//     per-group weight scales, then one global_load_lds_dwordx4 per tile row,
//     each a contiguous 1 KiB of that row, to LDS rows 1040 bytes apart (so the
//     8-byte fragment reads of 16 rows hit 16 bank groups).  It meets the two
//     barriers without waiting for that DMA (barrier_lds_only), then waits for
//     its own loads and copies its scales to LDS;
//   * after a third barrier (every slice and its scales in LDS) every wave,
//     the rotation waves included, multiplies units of 16 K-groups of one
//     tile, A = codes (rows M .. 15 are whatever LDS holds there: MFMA rows are
//     independent and those outputs are never stored; groups past K are zero
//     codes), B = decoded weights.  A per-group scale is folded in right after
//     the MFMA of its group: a unit's fp32 sum is one wave's sum of the
//     few-row kernel (16 groups per wave there), in the same order;
//   * the last unit of a tile to finish (an LDS arrival count) adds the units'
//     sums in group order, applies the row scale, x_scale and bias and stores
//     bf16, so the outputs equal rotate-quant + few-row kernel bit for bit.
// Codes in LDS: the 16 codes of row r (< 8) and k-block kb of 64-column group
// g (columns 64 g + 16 kb .. + 15, in the nibble decode's order 0,2,4,6,
// 1,3,5,7, 8,10,12,14, 9,11,13,15) sit at 576 g + 144 kb + 16 r.  A rotation
// wave's 8-byte stores (64 consecutive chunks of one row) then hit 32 distinct
// bank pairs per half-wave, a streaming wave's 16-byte operand reads (8 rows of
// one k-block per quarter-wave) are 128 contiguous bytes, and every LDS
// address in the group loop is one per-lane register plus an immediate offset
// (XOR swizzles that depend on the group need a register per group: measured
// 64 spilled registers, and the spill reloads serialised the weight loads).
#include "ck_device.h"
#include "launch.h"
#include "rotate_rows.h"

namespace ck {
namespace {

typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kGpw = kSfGroupsPerWave;  // K-groups per streaming wave
constexpr int kP = 32 * kGpw;           // bytes of one tile row in a slice (1 KiB)
constexpr int kPitch = kSfSlicePitch;   // LDS bytes between slice rows
constexpr int kSlice = 16 * kPitch;     // LDS bytes of one wave's slice
constexpr int kHalf = 16;               // groups per fp32 partial sum
static_assert(kP == 64 * 16 && kGpw == 2 * kHalf, "one DMA instruction per tile row, two partial sums per wave");

template <int M>
struct SfShared {
    uint32_t wmax[kSfRotWaves][M];     // each rotation wave's row absmax (fp32 bits)
    uint32_t done[kSfMaxStreamWaves];  // units of each tile whose partial sums are in LDS
};
static_assert(sizeof(SfShared<kSfMaxRows>) + kSfMaxLds <= 160 * 1024, "static and dynamic LDS fit the CU");

// s_barrier for the streaming waves: their own LDS stores complete first, but
// not their weight DMA (a workgroup fence before the barrier would wait for
// it); the "memory" clobber keeps the compiler's LDS accesses on their side.
__device__ __forceinline__ void barrier_lds_only() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ int code_offset(int g, int kb, int r) { return kSfCodeGroup * g + 144 * kb + 16 * r; }

template <int M, int G, bool PER_GROUP>
__global__ __launch_bounds__(1024) void w4_skinny_fused_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, float qmax, int K, const uint8_t *__restrict__ packed,
    int64_t ldw, const uint16_t *__restrict__ w_scales, int N, const uint16_t *__restrict__ bias,
    float x_scale, uint16_t *__restrict__ out, int64_t ldo, int rows, int S, int NWS)
{
    constexpr float kInvSqrtG = G == 16 ? 0.25f : G == 64 ? 0.125f : 0.0625f;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_generic[];
    __shared__ SfShared<M> sh;
    lds_u8 *smem = (lds_u8 *)smem_generic;
    const int ng = K / 64;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    lds_u8 *codes = smem + NWS * kSlice;  // [32 S groups][576]
    // [NWS][kSwLd][64] scale dwords, then [units][64][4] partial sums
    constexpr int kSwLd = PER_GROUP ? kGpw / 8 : 1;
    uint32_t *scl = reinterpret_cast<uint32_t *>(smem_generic + NWS * kSlice + kSfCodeGroup * kGpw * S);
    uint32_t *red = scl + NWS * kSfScaleDwords;
    const int n0 = xcd_block(blockIdx.x, gridDim.x) * rows;
    const int nrows = min(rows, N - n0);

    if (wave < kSfRotWaves) {
        // Chunks past K up to the last slice's end hold zero codes, so that
        // the groups past K multiply zero activations.
        const int rt = (int)threadIdx.x;
        if (rt >= K / 8 && rt < 8 * kGpw * S) {
#pragma unroll
            for (int m = 0; m < M; ++m)
                *(__attribute__((address_space(3))) u32x2 *)(codes + code_offset(rt >> 3, (rt >> 1) & 3, m) +
                                                             8 * (rt & 1)) = u32x2{0u, 0u};
        }
        rotate_rows<M, G, 1, true, true>(x, ldx, qmax, K, rt, kWave * kSfRotWaves, kSfRotWaves, lane, &sh.wmax[0][0],
                                         nullptr, [&](int m, int c, uint32_t even, uint32_t odd) {
                                             *(__attribute__((address_space(3))) u32x2 *)(
                                                 codes + code_offset(c >> 3, (c >> 1) & 3, m) + 8 * (c & 1)) =
                                                 u32x2{even, odd};
                                         });
        barrier_lds_only();  // every slice and its scales are in LDS
    } else {
        const int sw = wave - kSfRotWaves;  // streaming wave: tile sw / S, K-slice sw % S
        const int t = sw / S, g0 = (sw % S) * kGpw, tr0 = 16 * t;
        const int cnt = max(0, min(kGpw, ng - g0));
        lds_u8 *slice = smem + sw * kSlice;
        if (sw == 0 && lane < kSfMaxStreamWaves)
            sh.done[lane] = 0;  // read after the workgroup's last barrier
        // Per-group weight scales, one dword per lane and 8 groups: lane l holds
        // the scales of columns 2 (l % 8) and + 1 of the tile in group g0 + l / 8
        // (+ 8 q); they go to LDS for whichever wave multiplies these groups.
        uint32_t swd[kSwLd];
        if constexpr (PER_GROUP) {
            const int cs = min(n0 + tr0 + 2 * (lane % 8), N - 2);  // a half tile at the end of N reads column N - 2
#pragma unroll
            for (int q = 0; q < kSwLd; ++q)
                swd[q] = *reinterpret_cast<const uint32_t *>(w_scales + (int64_t)min(g0 + 8 * q + lane / 8, ng - 1) * N +
                                                             cs);
        }
        // The weight slice: instruction r copies row r's 1 KiB (lane l: chunk l).
        // Rows past the workgroup's end are not loaded (their outputs are not stored).
        const uint8_t *wrow = packed + (int64_t)(n0 + tr0) * ldw + 32 * g0 + 16 * lane;
        const bool wlive = lane < 2 * cnt;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (wlive && tr0 + r < nrows)
                __builtin_amdgcn_global_load_lds(wrow + r * ldw, slice + kPitch * r, 16, 0, 0);
        // The weights are requested from the first instructions on; the rotation
        // waves' two barriers (maxima published, codes stored) are met here
        // without waiting for them.
        barrier_lds_only();
        barrier_lds_only();
        wait_vmcnt0();  // this wave's scales and slice have landed
        if constexpr (PER_GROUP) {
#pragma unroll
            for (int q = 0; q < kSwLd; ++q)
                scl[(sw * kSwLd + q) * kWave + lane] = swd[q];
        }
        barrier_lds_only();  // every slice and its scales are in LDS
    }

    // Every wave now multiplies: unit u = (tile u / nh, block u % nh) covers 16
    // K-groups of one tile, the groups of one wave of the few-row kernel, so its
    // fp32 partial sum (per-group scales folded in group order) is one of that
    // kernel's, and the last unit of a tile to finish adds them in block order.
    // Groups past K multiply zero codes.  Rows M .. 15 of the activation operand
    // hold whatever the LDS holds there: MFMA rows are independent, and those
    // rows' outputs are never stored.
    const int nh = (ng + kHalf - 1) / kHalf, units = (NWS / S) * nh;
    for (int u = wave; u < units; u += (int)blockDim.x / kWave) {
        // The lane's role, derived here rather than kept live through the
        // rotation above (at 8 rows that spilled a register).
        int tid = (int)threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int col = tid % 16, kb = (tid % kWave) / 16;
        // This lane's bf16 scale from a pair of columns, into the high half.
        const uint32_t ssel = (col & 1) ? 0x03020C0Cu : 0x01000C0Cu;
        const int t = u / nh, h = u % nh, tr0 = 16 * t;
        const int sl = t * S + h / 2;                 // the slice (streaming wave) holding these groups
        const int jo = (h % 2) * kHalf;               // their first group within the slice
        const lds_u8 *abase = codes + code_offset(kGpw * (h / 2) + jo, kb, col & 7);
        const lds_u8 *bbase = smem + sl * kSlice + col * kPitch + 32 * jo + 16 * (kb >> 1) + 8 * (kb & 1);
        const uint32_t *sbase = scl + sl * kSwLd * kWave + col / 2;
        float y[4] = {0.f, 0.f, 0.f, 0.f};
        v4i acc = v4i{0, 0, 0, 0};
        constexpr int kBatch = 4, kNb = kHalf / kBatch;
        u32x4 ar[2][kBatch];
        u32x2 wq[2][kBatch];
        uint32_t pair[2][kBatch];
        // Software pipelined: the LDS reads of batch b + 1 are issued before the
        // MFMAs and scale folds of batch b.
        auto read_batch = [&](int b) {
#pragma unroll
            for (int e = 0; e < kBatch; ++e) {
                const int j = b * kBatch + e;         // group jo + j of the slice
                ar[b & 1][e] = *(const __attribute__((address_space(3))) u32x4 *)(abase + kSfCodeGroup * j);
                wq[b & 1][e] = *(const __attribute__((address_space(3))) u32x2 *)(bbase + 32 * j);
                if constexpr (PER_GROUP) {
                    const int js = jo + j;             // lane (js % 8) * 8 + col / 2 of dword js / 8 holds the pair
                    pair[b & 1][e] = sbase[(js / 8) * kWave + (js % 8) * 8];
                }
            }
        };
        read_batch(0);
#pragma unroll
        for (int b = 0; b < kNb; ++b) {
            if (b + 1 < kNb)
                read_batch(b + 1);
            v4i d[kBatch];
#pragma unroll
            for (int e = 0; e < kBatch; ++e) {
                const u32x4 &ra = ar[b & 1][e];
                const v4i a = v4i{(int)ra[0], (int)ra[1], (int)ra[2], (int)ra[3]};
                const v4i bw = w4_operand_x16(wq[b & 1][e][0], wq[b & 1][e][1]);
                if constexpr (PER_GROUP)
                    d[e] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bw, v4i{0, 0, 0, 0}, 0, 0, 0);
                else
                    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bw, acc, 0, 0, 0);
            }
            if constexpr (PER_GROUP) {
#pragma unroll
                for (int e = 0; e < kBatch; ++e) {
                    const float sc = __uint_as_float(perm(0u, pair[b & 1][e], ssel));
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        y[i] = __builtin_fmaf(sc, (float)d[e][i], y[i]);
                }
                // Keep each batch's scale folds with its MFMAs: left alone, the
                // compiler issued all the MFMAs first and folded afterwards, which
                // needs more registers than 16 waves per CU leave.
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    asm volatile("" : "+v"(y[i]));
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // The partial to LDS; the last of the tile's nh units adds them in block order.
        uint32_t *mine = red + (u * kWave + lane) * 4;
        if constexpr (PER_GROUP)
            *reinterpret_cast<float4 *>(mine) = make_float4(y[0], y[1], y[2], y[3]);
        else
            *reinterpret_cast<int4 *>(mine) = make_int4(acc[0], acc[1], acc[2], acc[3]);
        uint32_t prior = 0;
        if (lane == 0)
            prior = __hip_atomic_fetch_add(&sh.done[t], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (__builtin_amdgcn_readfirstlane(prior) != (uint32_t)(nh - 1))
            continue;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        // Lane (col, kb) holds D[4 kb + i][col]: activation rows 4 kb + i, weight row col.
        if (tr0 + col < nrows) {
            const int n = n0 + tr0 + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * kb + i;
                if (m >= M)
                    break;
                const float am = __uint_as_float(row_max_bits(&sh.wmax[0][0], m, M, kSfRotWaves));
                const float sx = am > 0.f ? (am / qmax) * kInvSqrtG : 1.0f;  // the rotate-quant kernel's row scale
                float yv;
                if constexpr (PER_GROUP) {
                    float sum = 0.f;
                    for (int hh = 0; hh < nh; ++hh)
                        sum += __uint_as_float(red[((t * nh + hh) * kWave + lane) * 4 + i]);
                    yv = sum * 0.0625f * (sx * x_scale);
                    if (bias)
                        yv += bf16_to_f32(bias[n]);
                } else {
                    int sum = 0;
                    for (int hh = 0; hh < nh; ++hh)
                        sum += (int)red[((t * nh + hh) * kWave + lane) * 4 + i];
                    yv = epilogue_channel((float)sum, 0.0625f * bf16_to_f32(w_scales[n]), sx * x_scale,
                                          bias ? bf16_to_f32(bias[n]) : 0.f);  // sum = 16 * dot
                }
                out[(int64_t)m * ldo + n] = f32_to_bf16(yv);
            }
        }
    }
}

template <int M, int G, bool PG>
hipError_t launch_k(const SkinnyFusedShape &sh, const uint16_t *x, int64_t ldx, float qmax, int K,
                    const uint8_t *packed, int64_t ldw, const uint16_t *ws, int N, const uint16_t *bias, float xs,
                    uint16_t *out, int64_t ldo, hipStream_t s)
{
    auto kern = w4_skinny_fused_kernel<M, G, PG>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kSfMaxLds);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL(kern, dim3((unsigned)sh.nb), dim3((unsigned)((sh.nws + kSfRotWaves) * kWave)),
                       (size_t)sh.lds, s, x, ldx, qmax, K, packed, ldw, ws, N, bias, xs, out, ldo, sh.rows, sh.s,
                       sh.nws);
    return hipGetLastError();
}

template <int M>
hipError_t launch_m(const SkinnyFusedShape &sh, int G, bool pg, const uint16_t *x, int64_t ldx, float qmax, int K,
                    const uint8_t *packed, int64_t ldw, const uint16_t *ws, int N, const uint16_t *bias, float xs,
                    uint16_t *out, int64_t ldo, hipStream_t s)
{
#define CK_SF_G(GG)                                                                                     \
    return pg ? launch_k<M, GG, true>(sh, x, ldx, qmax, K, packed, ldw, ws, N, bias, xs, out, ldo, s)  \
              : launch_k<M, GG, false>(sh, x, ldx, qmax, K, packed, ldw, ws, N, bias, xs, out, ldo, s);
    switch (G) {
    case 16: CK_SF_G(16)
    case 64: CK_SF_G(64)
    case 256: CK_SF_G(256)
    default: return hipErrorInvalidValue;
    }
#undef CK_SF_G
}

}  // namespace

int launch_w4_skinny_fused(const uint16_t *x, int64_t ldx, int G, int qmax, int M, int K, const uint8_t *packed,
                           int64_t ldw, const uint16_t *w_scales, bool per_group, int N, const uint16_t *bias,
                           float x_scale, uint16_t *out, int64_t ldo, void *stream)
{
    SkinnyFusedShape sh;
    if (!w4_skinny_fused_shape(M, K, N, device_cu_count(), sh))
        return (int)hipErrorInvalidValue;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const float q = (float)qmax;
#define CK_SF_M(MM) \
    case MM: return (int)launch_m<MM>(sh, G, per_group, x, ldx, q, K, packed, ldw, w_scales, N, bias, x_scale, out, ldo, s);
    switch (M) {
        CK_SF_M(1) CK_SF_M(2) CK_SF_M(3) CK_SF_M(4) CK_SF_M(5) CK_SF_M(6) CK_SF_M(7) CK_SF_M(8)
    default: return (int)hipErrorInvalidValue;
    }
#undef CK_SF_M
}

}  // namespace ck
