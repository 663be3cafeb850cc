// Fused group-wise Walsh-Hadamard rotation + rowwise absmax quantisation.
//
// Follows the fused RotateQuant operator of "[PR #155] [Feat][Ascend] Add
// fused RotateQuant backend" (section "What this PR does"): the rotation
// x_g . H_G / sqrt(G) of every contiguous G-column group (G = 16, 64, 256) and
// the dynamic per-row quantisation happen in one pass over x, so the rotated
// tensor is never written out.
//
// Work layout (one workgroup per row of 128, 256 or 1024 threads, by K):
//   * thread t owns chunks c = t, t + BLOCK, ... of CW consecutive bf16
//     (CW = 8: one coalesced 16-byte load; CW = 16, used for activation codes
//     from G = 64 on: two);
//   * a group of G columns is G/CW chunks held by G/CW neighbouring lanes of
//     one wave (groups never straddle a wave or a chunk round);
//   * the first log2(CW) butterfly stages (strides 1 .. CW/2) run inside the
//     thread's registers, the remaining log2(G/CW) stages across lanes
//     (ds_swizzle from G = 64 on, which keeps the exchange off the VALU,
//     except the lane-distance-1 stage of 8-column chunks at G = 16 and 256:
//     DPP quad permute);
//   * the fp32 values stay in registers until the row absmax is known
//     (wave reduction, then LDS across waves); then every thread quantises and
//     stores its own CW codes with one store.
// The transform is kept unnormalised (y = sqrt(G) * xr).  Because sqrt(G) is a
// power of two, fp32(qmax / max|y|) * y equals fp32(qmax / max|xr|) * xr
// exactly, so the codes match the normalised definition bit for bit; the row
// scale is max|y| / qmax divided by sqrt(G) (also exact).
#include "ck_device.h"
#include "launch.h"

namespace ck {
namespace {

// Value held by the lane whose index differs in bit log2(MASK).  DPP moves
// are VALU instructions, ds_swizzle runs on the LDS pipe; SWZ selects the
// swizzle for every distance (see fht() for where each is used).
template <int MASK, bool SWZ = false>
__device__ __forceinline__ float lane_xor(float v)
{
    int i = __float_as_int(v);
    if constexpr (SWZ)
        i = __builtin_amdgcn_ds_swizzle(i, 0x1F | (MASK << 10));      // bitmask mode: lane ^ MASK
    else if constexpr (MASK == 1)
        i = __builtin_amdgcn_update_dpp(0, i, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
    else if constexpr (MASK == 2)
        i = __builtin_amdgcn_update_dpp(0, i, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
    else
        i = __builtin_amdgcn_ds_swizzle(i, 0x1F | (MASK << 10));      // bitmask mode: lane ^ MASK
    return __int_as_float(i);
}

// One cross-lane butterfly stage: the lower lane of each pair keeps u + v,
// the upper lane v' = u - v (written as fma(v, -1, u), same rounding).
template <int MASK, int CPT, int CW, bool SWZ>
__device__ __forceinline__ void lane_stage(float (&v)[CPT][CW], float sgn)
{
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int r = 0; r < CW; ++r) {
            const float p = lane_xor<MASK, SWZ>(v[i][r]);
            v[i][r] = __builtin_fmaf(v[i][r], sgn, p);
        }
}

template <int G, int CPT, int CW>
__device__ __forceinline__ void fht(float (&v)[CPT][CW], int lane)
{
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
#pragma unroll
        for (int h = 1; h < CW && h < G; h <<= 1)
#pragma unroll
            for (int r = 0; r < CW; ++r)
                if ((r & h) == 0) {
                    const float a = v[i][r], b = v[i][r + h];
                    v[i][r] = a + b;
                    v[i][r + h] = a - b;
                }
    }
    // From G = 64 on, the kernel issues about as many VALU cycles as its HBM
    // traffic takes, so it turns VALU-bound wherever the clock drops.  A DPP
    // exchange costs a VALU move besides the fma; ds_swizzle runs on the LDS
    // pipe instead.  At G = 64 all three exchanges use it (12.8 rather than
    // 14.8 VALU instructions per element).  At G = 256 five swizzles per
    // element overload the LDS pipe (wave-cycles waiting to issue LDS
    // instructions: 11.5 M per launch, against 1.6 M at G = 64), so the
    // distance-1 stage goes through DPP: 4 swizzles and about 15 VALU
    // instructions per element, measured 6% faster than all-swizzle (these
    // figures are for 8-column chunks).  With 16-column chunks the stride-8
    // stage is in registers and every remaining exchange goes through
    // ds_swizzle (at most 4 per element at G = 256).
    constexpr int L = G / CW;  // lanes per group
    constexpr bool SWZ = G >= 64 || CW == 16;
    constexpr bool SWZ1 = CW == 16 || (G >= 64 && G < 256);
    if constexpr (L >= 2) lane_stage<1, CPT, CW, SWZ1>(v, (lane & 1) ? -1.f : 1.f);
    if constexpr (L >= 4) lane_stage<2, CPT, CW, SWZ>(v, (lane & 2) ? -1.f : 1.f);
    if constexpr (L >= 8) lane_stage<4, CPT, CW, SWZ>(v, (lane & 4) ? -1.f : 1.f);
    if constexpr (L >= 16) lane_stage<8, CPT, CW, SWZ>(v, (lane & 8) ? -1.f : 1.f);
    if constexpr (L >= 32) lane_stage<16, CPT, CW, SWZ>(v, (lane & 16) ? -1.f : 1.f);
}

// Maximum over the wave: over each 16-lane row by DPP alone (quad permutes,
// then row_half_mirror and row_mirror, which pair lanes across bits 2 and 3),
// then over the four rows' first lanes.
__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, lane_xor<1>(v));
    v = fmaxf(v, lane_xor<2>(v));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true)));
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Low byte of fp32(t) + 1.5 * 2^23 is the two's-complement of rne(t) for
// |t| < 2^22 (the add rounds to an integer, ties to even).
__device__ __forceinline__ uint32_t rne_byte(float t) { return __float_as_uint(t + 12582912.0f); }

__device__ __forceinline__ uint32_t pack4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3)
{
    const uint32_t p01 = perm(b1, b0, 0x0C0C0400u);
    const uint32_t p23 = perm(b3, b2, 0x0C0C0400u);
    return perm(p23, p01, 0x05040100u);
}

// Output of the kernel: int8 codes (one per byte), the rotated fp32 values
// (test hook), W4A4 codes packed two per byte (4-bit two's complement,
// column 2j in bits 0..3), which halves the codes traffic of the W4A4 GEMM,
// or packed weights (stored code q = value + 8) with bf16 scales per row or
// per 64-column group.
// kTiled16 writes int8 codes in the few-row kernel's operand layout
// (CodesLayout::kTiled16 in launch.h).
enum OutMode { kCodes8 = 0, kF32 = 1, kPacked4 = 2, kWeightRow = 3, kWeightGroup = 4, kTiled16 = 5 };

// Weight quantisation of rotated values y = sqrt(G) * wr (see the launcher):
// scale s = bf16(fp32(a / 7)) for the absmax a of wr over the scale group,
// code = clamp(rne(fp32(wr * fp32(1 / s))), -7, 7).  am is max|y|.
struct WeightScale {
    float inv_y;     // fp32(1 / s) / sqrt(G): y * inv_y == wr * fp32(1 / s) exactly
    uint16_t bits;   // s as bf16
};
template <int G>
__device__ __forceinline__ WeightScale weight_scale(float am)
{
    constexpr float kInvSqrtG = G == 16 ? 0.25f : G == 64 ? 0.125f : 0.0625f;
    const float a = am * kInvSqrtG;
    const uint16_t sb = f32_to_bf16(a / 7.0f);
    const float sf = bf16_to_f32(sb);
    return WeightScale{sf > 0.f ? (1.0f / sf) * kInvSqrtG : 0.f, sb};
}

// FULL: every thread's CPT chunks lie inside the row (K = 8 * BLOCK * CPT),
// so the loads and stores need no bounds test (the test and the zero fill
// cost 5-6% of the kernel's VALU instructions).
template <int G, int BLOCK, int CPT, int MODE, bool FULL, int CW>
__global__ __launch_bounds__(BLOCK) void rotate_quant_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int K, float qmax, int8_t *__restrict__ codes,
    int64_t ldq, float *__restrict__ row_scales, float *__restrict__ xr, int64_t ldr,
    uint16_t *__restrict__ wscales, int64_t ldsc)
{
    constexpr float kInvSqrtG = G == 16 ? 0.25f : G == 64 ? 0.125f : 0.0625f;
    static_assert(G == 16 || G == 64 || G == 256, "G");
    static_assert(CW == 8 || (CW == 16 && (MODE == kCodes8 || MODE == kPacked4 || MODE == kF32 ||
                                           MODE == kTiled16)),
                  "chunk width");
    __shared__ float wmax[BLOCK / kWave];

    const int64_t m = blockIdx.x;
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int nchunk = K / CW;
    const uint16_t *xrow = x + m * ldx;

    constexpr int LD = CW / 8;  // 16-byte loads per chunk
    u32x4 raw[CPT][LD];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = t + i * BLOCK;
#pragma unroll
        for (int q = 0; q < LD; ++q)
            raw[i][q] = FULL || c < nchunk ? load_nt16(xrow + CW * c + 8 * q) : u32x4{0u, 0u, 0u, 0u};
    }
    float v[CPT][CW];
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int q = 0; q < LD; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[i][8 * q + 2 * j] = __uint_as_float(raw[i][q][j] << 16);
                v[i][8 * q + 2 * j + 1] = __uint_as_float(raw[i][q][j] & 0xffff0000u);
            }

    fht<G, CPT, CW>(v, lane);

    float am = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int r = 0; r < CW; ++r)
            am = fmaxf(am, fabsf(v[i][r]));
    am = wave_max(am);
    if (lane == 0)
        wmax[t / kWave] = am;
    __syncthreads();
    am = wmax[0];
#pragma unroll
    for (int w = 1; w < BLOCK / kWave; ++w)
        am = fmaxf(am, wmax[w]);

    if constexpr (MODE == kWeightRow || MODE == kWeightGroup) {
        // Packed weights: byte j of a row = q(2j) | q(2j + 1) << 4, q = code + 8.
        WeightScale ws = weight_scale<G>(am);
        uint8_t *prow = reinterpret_cast<uint8_t *>(codes) + m * ldq;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = t + i * BLOCK;
            if constexpr (MODE == kWeightGroup) {
                // A 64-column group is 8 chunks held by 8 neighbouring lanes.
                float gm = 0.f;
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    gm = fmaxf(gm, fabsf(v[i][r]));
                gm = fmaxf(gm, lane_xor<1>(gm));
                gm = fmaxf(gm, lane_xor<2>(gm));
                gm = fmaxf(gm, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(gm), 0x141, 0xF, 0xF,
                                                                          true)));  // row_half_mirror
                ws = weight_scale<G>(gm);
                if ((FULL || c < nchunk) && (c & 7) == 0)
                    wscales[(int64_t)(c >> 3) * ldsc + m] = ws.bits;
            }
            uint32_t b[8];
#pragma unroll
            for (int r = 0; r < 8; ++r)
                b[r] = rne_byte(fminf(fmaxf(v[i][r] * ws.inv_y, -7.f), 7.f));
            if (FULL || c < nchunk) {
                const uint32_t ev = pack4(b[0], b[2], b[4], b[6]);
                const uint32_t od = pack4(b[1], b[3], b[5], b[7]);
                // two's-complement nibble ^ 8 = value + 8
                reinterpret_cast<uint32_t *>(prow)[c] =
                    ((ev & 0x0f0f0f0fu) | ((od << 4) & 0xf0f0f0f0u)) ^ 0x88888888u;
            }
        }
        if constexpr (MODE == kWeightRow)
            if (t == 0)
                wscales[m] = ws.bits;
    } else if constexpr (MODE == kF32) {
        float *orow = xr + m * ldr;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = t + i * BLOCK;
            if (FULL || c < nchunk) {
                float4 *o = reinterpret_cast<float4 *>(orow + CW * c);
#pragma unroll
                for (int q = 0; q < CW / 4; ++q)
                    o[q] = make_float4(v[i][4 * q] * kInvSqrtG, v[i][4 * q + 1] * kInvSqrtG,
                                       v[i][4 * q + 2] * kInvSqrtG, v[i][4 * q + 3] * kInvSqrtG);
            }
        }
    } else if constexpr (MODE == kTiled16) {
        // Each 8 columns become 8 bytes of a 16-byte operand chunk: the even
        // columns, then the odd ones.  Row m is row m % 16 of tile m / 16.
        const float inv = am > 0.f ? qmax / am : 0.f;
        int8_t *trow = codes + (m >> 4) * (int64_t)K * 16 + (m & 15) * 16;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = t + i * BLOCK;
            uint32_t b[CW];
#pragma unroll
            for (int r = 0; r < CW; ++r)
                b[r] = rne_byte(v[i][r] * inv);
            if (FULL || c < nchunk) {
#pragma unroll
                for (int q = 0; q < CW / 8; ++q) {
                    const uint32_t *bq = b + 8 * q;
                    const int c8 = (CW / 8) * c + q;  // 8-column unit of the row
                    const int c16 = c8 >> 1;          // 16-column chunk: group c16 / 4, kb = c16 % 4
                    int8_t *dst = trow + (c16 >> 2) * 1024 + (c16 & 3) * 256 + 8 * (c8 & 1);
                    *reinterpret_cast<uint2 *>(dst) =
                        uint2{pack4(bq[0], bq[2], bq[4], bq[6]), pack4(bq[1], bq[3], bq[5], bq[7])};
                }
            }
        }
        if (t == 0)
            row_scales[m] = am > 0.f ? (am / qmax) * kInvSqrtG : 1.0f;
    } else {
        // am == 0 (all-zero row): inv = 0 makes every code 0; the scale is 1.
        const float inv = am > 0.f ? qmax / am : 0.f;
        int8_t *crow = codes + m * ldq;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = t + i * BLOCK;
            uint32_t b[CW];
#pragma unroll
            for (int r = 0; r < CW; ++r)
                b[r] = rne_byte(v[i][r] * inv);
            // Per 8 columns: one dword of packed nibbles (byte j = nibble of
            // column 2j | nibble of column 2j + 1 << 4) or two dwords of bytes.
            uint32_t o[MODE == kPacked4 ? CW / 8 : CW / 4];
#pragma unroll
            for (int q = 0; q < CW / 8; ++q) {
                const uint32_t *bq = b + 8 * q;
                if constexpr (MODE == kPacked4) {
                    const uint32_t ev = pack4(bq[0], bq[2], bq[4], bq[6]);
                    const uint32_t od = pack4(bq[1], bq[3], bq[5], bq[7]);
                    o[q] = (ev & 0x0f0f0f0fu) | ((od << 4) & 0xf0f0f0f0u);
                } else {
                    o[2 * q] = pack4(bq[0], bq[1], bq[2], bq[3]);
                    o[2 * q + 1] = pack4(bq[4], bq[5], bq[6], bq[7]);
                }
            }
            if (FULL || c < nchunk) {
                constexpr int NO = sizeof(o) / sizeof(o[0]);
                if constexpr (NO == 1)
                    reinterpret_cast<uint32_t *>(crow)[c] = o[0];
                else if constexpr (NO == 2)
                    reinterpret_cast<uint2 *>(crow)[c] = uint2{o[0], o[1]};
                else
                    reinterpret_cast<uint4 *>(crow)[c] = uint4{o[0], o[1], o[2], o[3]};
            }
        }
        if (t == 0)
            row_scales[m] = am > 0.f ? (am / qmax) * kInvSqrtG : 1.0f;
    }
}

// BLOCK threads, CPT chunks of CW columns per thread.  CPT is capped so that
// the row stays in VGPRs without spilling: 64 columns per thread up to 256
// threads (80 with 16-column chunks), 32 at 1024.
template <int G, int BLOCK, int MODE, int CW>
hipError_t launch_g(int cpt, dim3 grid, hipStream_t s, const uint16_t *x, int64_t ldx, int K,
                    float qmax, int8_t *codes, int64_t ldq, float *rs, float *xr, int64_t ldr,
                    uint16_t *wsc, int64_t ldsc)
{
    constexpr int kMaxCpt = BLOCK >= 1024 ? 32 / CW : CW == 16 ? 5 : 8;
    if (cpt < 1 || cpt > kMaxCpt)
        return hipErrorInvalidValue;
    const bool full = K == CW * BLOCK * cpt;
#define CK_RQ_CASE(C)                                                                           \
    case C:                                                                                     \
        if constexpr (C <= kMaxCpt) {                                                           \
            if (full)                                                                           \
                hipLaunchKernelGGL((rotate_quant_kernel<G, BLOCK, C, MODE, true, CW>), grid,    \
                                   dim3(BLOCK), 0, s, x, ldx, K, qmax, codes, ldq, rs, xr, ldr,  \
                                   wsc, ldsc);                                                  \
            else                                                                                \
                hipLaunchKernelGGL((rotate_quant_kernel<G, BLOCK, C, MODE, false, CW>), grid,   \
                                   dim3(BLOCK), 0, s, x, ldx, K, qmax, codes, ldq, rs, xr, ldr, \
                                   wsc, ldsc);                                                  \
        }                                                                                       \
        break;
    switch (cpt) {
        CK_RQ_CASE(1)
        CK_RQ_CASE(2)
        CK_RQ_CASE(3)
        CK_RQ_CASE(4)
        CK_RQ_CASE(5)
        CK_RQ_CASE(6)
        CK_RQ_CASE(7)
        CK_RQ_CASE(8)
    default:
        return hipErrorInvalidValue;
    }
#undef CK_RQ_CASE
    return hipGetLastError();
}

// Up to this many rows the kernel is latency-bound (a few workgroups on an
// otherwise idle chip): rows of up to 4096 columns then run 512 threads of
// one 8-column chunk each, so that each thread's serial chain is shortest.
// Measured on MI355X (K = 3840, G = 64) in the whole W4A8 linear: M = 32
// 10.36 us with 128 threads of two 16-column chunks, 9.51 with 256 threads of
// one, 9.37 with 512 threads of one 8-column chunk, 11.75 with one wave of
// four 16-column chunks; M = 4 11.91 / 10.94 / 10.74 / 13.29 us.
constexpr int64_t kFewRows = 64;

template <int G, int MODE>
hipError_t launch_rq(int64_t M, int K, hipStream_t s, const uint16_t *x, int64_t ldx, float qmax,
                     int8_t *codes, int64_t ldq, float *rs, float *xr, int64_t ldr,
                     uint16_t *wsc = nullptr, int64_t ldsc = 0)
{
    const dim3 grid((unsigned)M);
    if constexpr ((MODE == kCodes8 || MODE == kPacked4 || MODE == kF32 || MODE == kTiled16) && G >= 64) {
        // Activation codes from G = 64 on: 16-column chunks (K is a multiple
        // of G), except for the few-row shapes above.  The fp32 test output
        // takes the same instantiation for the same M, K and G, so the
        // rotation it exposes is the one the activation codes are made from.
        // Up to 10240 columns 128 threads of up to 5 chunks, then 256, then
        // 1024 threads of up to 2.  The in-register distance-8 stage and
        // the longer rows per thread take 1-2 VALU instructions per element
        // off (13.3 instead of 15.3 at G = 256, K = 10240), which is what
        // sets the time here: 5-10% faster at G = 64 and 256.  At G = 16 the
        // kernel is HBM-bound and the 8-column layout, whose loads fill whole
        // cache lines per instruction (a 16-column chunk is two 16-byte loads
        // 32 bytes apart), measured 8% faster.
        const int nchunk = K / 16;
        if (M <= kFewRows && K / 8 <= 512)
            return launch_g<G, 512, MODE, 8>(1, grid, s, x, ldx, K, qmax, codes, ldq, rs, xr, ldr, wsc, ldsc);
        if (nchunk <= 128 * 5)
            return launch_g<G, 128, MODE, 16>((nchunk + 127) / 128, grid, s, x, ldx, K, qmax, codes, ldq, rs, xr,
                                              ldr, wsc, ldsc);
        if (nchunk <= 256 * 5)
            return launch_g<G, 256, MODE, 16>((nchunk + 255) / 256, grid, s, x, ldx, K, qmax, codes, ldq, rs, xr,
                                              ldr, wsc, ldsc);
        return launch_g<G, 1024, MODE, 16>((nchunk + 1023) / 1024, grid, s, x, ldx, K, qmax, codes, ldq, rs, xr,
                                           ldr, wsc, ldsc);
    } else {
        const int nchunk = K / 8;
        if (M <= kFewRows && nchunk <= 512)
            return launch_g<G, 512, MODE, 8>(1, grid, s, x, ldx, K, qmax, codes, ldq, rs, xr, ldr, wsc, ldsc);
        // Rows of up to 8192 columns: 128 threads with up to 8 chunks each, which
        // measured 3-10% faster than 256 threads at K = 2048 and 3840 (more loads
        // in flight per thread, more resident rows per CU).
        if (nchunk <= 128 * 8) {
            const int cpt = (nchunk + 127) / 128;
            return launch_g<G, 128, MODE, 8>(cpt, grid, s, x, ldx, K, qmax, codes, ldq, rs, xr, ldr, wsc, ldsc);
        }
        if (nchunk <= 256 * 8) {
            const int cpt = (nchunk + 255) / 256;
            return launch_g<G, 256, MODE, 8>(cpt, grid, s, x, ldx, K, qmax, codes, ldq, rs, xr, ldr, wsc, ldsc);
        }
        const int cpt = (nchunk + 1023) / 1024;
        return launch_g<G, 1024, MODE, 8>(cpt, grid, s, x, ldx, K, qmax, codes, ldq, rs, xr, ldr, wsc, ldsc);
    }
}

}  // namespace

int launch_rotate_quant(const uint16_t *x, int64_t M, int K, int64_t ldx, int G, int qmax,
                        int8_t *codes, int64_t ldq, float *row_scales, float *xr, int64_t ldr,
                        CodesLayout layout, void *stream)
{
    if (M <= 0)
        return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const float q = (float)qmax;
    const int mode = xr ? kF32
                        : layout == CodesLayout::kPacked4 ? kPacked4
                        : layout == CodesLayout::kTiled16 ? kTiled16
                                                          : kCodes8;
#define CK_RQ_G(MODE)                                                                                  \
    switch (G) {                                                                                     \
    case 16: return (int)launch_rq<16, MODE>(M, K, s, x, ldx, q, codes, ldq, row_scales, xr, ldr);   \
    case 64: return (int)launch_rq<64, MODE>(M, K, s, x, ldx, q, codes, ldq, row_scales, xr, ldr);   \
    default: return (int)launch_rq<256, MODE>(M, K, s, x, ldx, q, codes, ldq, row_scales, xr, ldr);  \
    }
    if (mode == kF32) {
        CK_RQ_G(kF32)
    } else if (mode == kPacked4) {
        CK_RQ_G(kPacked4)
    } else if (mode == kTiled16) {
        CK_RQ_G(kTiled16)
    } else {
        CK_RQ_G(kCodes8)
    }
#undef CK_RQ_G
}

int launch_quantize_weights(const uint16_t *w, int64_t N, int K, int64_t ldw_in, int G, bool per_group,
                            uint8_t *packed, int64_t ldp, uint16_t *scales, void *stream)
{
    if (N <= 0)
        return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int8_t *dst = reinterpret_cast<int8_t *>(packed);
#define CK_WQ_G(MODE)                                                                                     \
    switch (G) {                                                                                        \
    case 16: return (int)launch_rq<16, MODE>(N, K, s, w, ldw_in, 7.f, dst, ldp, nullptr, nullptr, 0, scales, N);  \
    case 64: return (int)launch_rq<64, MODE>(N, K, s, w, ldw_in, 7.f, dst, ldp, nullptr, nullptr, 0, scales, N);  \
    default: return (int)launch_rq<256, MODE>(N, K, s, w, ldw_in, 7.f, dst, ldp, nullptr, nullptr, 0, scales, N); \
    }
    if (per_group) {
        CK_WQ_G(kWeightGroup)
    } else {
        CK_WQ_G(kWeightRow)
    }
#undef CK_WQ_G
}

}  // namespace ck
