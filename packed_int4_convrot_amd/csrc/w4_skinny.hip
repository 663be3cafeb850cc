// Weight-streaming W4 matmul for few activation rows (decode GEMV, M <= 64).
//
// Prior art: the W4A8 decode GEMV of "[PR #182] HIP port of #176: W4A8 decode
// GEMV and fused GatedDeltaNet decode" (description): int4 weights are decoded
// in registers and fed straight to integer dot products, then a rowwise x
// weight-scale epilogue ("EpiRowwise") is applied; no decoded copy of the
// weights ever exists in memory.  Here the integer products run on CDNA4 int8
// MFMA (v_mfma_i32_16x16x64_i8): one instruction covers 16 output columns x
// one 64-wide K group x up to 16 activation rows, so a per-group weight scale
// is applied right after the instruction that produced that group's sum.
//
// Operand layouts of v_mfma_i32_16x16x64_i8 (16 x 64 x 16):
//   A (activations): lane l holds 16 int8 of row m = l % 16, k-block l / 16
//   B (weights):     lane l holds 16 int8 of column n = l % 16, k-block l / 16
//   D:               lane l holds D[4 * (l / 16) + i][l % 16], i = 0..3
// A and B share the (lane, byte) -> k assignment, so the even/odd k order that
// the nibble decode produces on B is matched by permuting A once (act_perm16).
//
// Work split:
//   * a workgroup has KS waves; wave w owns a contiguous range of at most GPW
//     K-groups and keeps the activation operands of that range in VGPRs for
//     the whole kernel (loaded and permuted once);
//   * the workgroup walks 16-column tiles of the output; for each tile every
//     wave issues all its weight loads (8 bytes per lane per group, i.e. 32
//     contiguous bytes per weight row per group) before the first MFMA;
//   * per-wave partial results are summed across waves through LDS in a fixed
//     order (deterministic), then scaled, biased and stored as bf16.
#include "ck_device.h"
#include "launch.h"

namespace ck {
namespace {

constexpr int kMaxWaves = 8;  // 512 threads: up to 256 VGPRs per lane

template <int MT, int GPW, bool PER_GROUP, bool OUT_I32>
__global__ __launch_bounds__(kMaxWaves * kWave) void w4_skinny_kernel(
    const int8_t *__restrict__ codes, int64_t ldq, const float *__restrict__ row_scales, int M,
    int K, const uint8_t *__restrict__ packed, int64_t ldw, const uint16_t *__restrict__ w_scales,
    int N, const uint16_t *__restrict__ bias, float x_scale, uint16_t *__restrict__ out,
    int64_t ldo, int32_t *__restrict__ acc_out, int64_t lda, int gpw)
{
    extern __shared__ int red_smem[];  // [KS][MT][64][4] partials
    const int ks = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int ng = K / 64;
    const int g0 = wave * gpw;
    const int cnt = max(0, min(gpw, ng - g0));
    const int col = lane % 16;
    const int kb = lane / 16;

    // Issue the activation loads of this wave's groups and the first tile's
    // weight loads before any of them is used, so that all of them are in
    // flight together.  Addresses are clamped into the matrices; the values
    // of out-of-range rows / groups are replaced by zero afterwards.
    const int ntiles = N / 16;
    int tile = blockIdx.x;
    u32x4 raw[GPW][MT];
#pragma unroll
    for (int j = 0; j < GPW; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = min(mt * 16 + col, M - 1);
            const int g = min(g0 + j, ng - 1);
            raw[j][mt] = *reinterpret_cast<const u32x4 *>(codes + (int64_t)m * ldq + 64 * g + 16 * kb);
        }
    u32x2 bw[GPW];
    uint16_t sw[GPW];
    auto load_tile = [&](int t) {
        const int n = t * 16 + col;
        const uint8_t *wrow = packed + (int64_t)n * ldw + 8 * kb + 32 * g0;
#pragma unroll
        for (int j = 0; j < GPW; ++j)
            if (j < cnt) {
                bw[j] = load_nt8(wrow + 32 * j);
                if constexpr (PER_GROUP)
                    sw[j] = w_scales[(int64_t)(g0 + j) * N + n];
            }
    };
    if (tile < ntiles)
        load_tile(tile);

    // Activation operands, permuted to the decode order.
    v4i a[GPW][MT];
#pragma unroll
    for (int j = 0; j < GPW; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const bool live = j < cnt && mt * 16 + col < M;
            const v4i p = act_perm16(raw[j][mt][0], raw[j][mt][1], raw[j][mt][2], raw[j][mt][3]);
            a[j][mt] = live ? p : v4i{0, 0, 0, 0};
        }

    for (; tile < ntiles; tile += gridDim.x) {

        float y[MT][4];
        v4i acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            acc[mt] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                y[mt][i] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < GPW; ++j)
            if (j < cnt) {
                const v4i b = w4_operand_x16(bw[j][0], bw[j][1]);
                if constexpr (PER_GROUP) {
                    const float s = bf16_to_f32(sw[j]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j][mt], b,
                                                                           v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            y[mt][i] = __builtin_fmaf(s, (float)d[i], y[mt][i]);
                    }
                } else {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j][mt], b, acc[mt], 0, 0, 0);
                }
            }

        if (tile + (int)gridDim.x < ntiles)
            load_tile(tile + gridDim.x);  // next tile's weights fly during the reduction

        // Cross-wave reduction: red[w][mt][lane][i].
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            int *dst = red_smem + ((wave * MT + mt) * kWave + lane) * 4;
            if constexpr (PER_GROUP)
                *reinterpret_cast<float4 *>(dst) = make_float4(y[mt][0], y[mt][1], y[mt][2], y[mt][3]);
            else
                *reinterpret_cast<int4 *>(dst) = make_int4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
        }
        __syncthreads();
        for (int e = threadIdx.x; e < MT * kWave * 4; e += blockDim.x) {
            const int mt = e / (kWave * 4);
            const int l = (e / 4) % kWave;
            const int i = e % 4;
            const int m = mt * 16 + 4 * (l / 16) + i;
            const int nn = tile * 16 + l % 16;
            if (m < M) {
                if constexpr (OUT_I32) {
                    int s = 0;
                    for (int w = 0; w < ks; ++w)
                        s += red_smem[w * MT * kWave * 4 + e];
                    acc_out[(int64_t)m * lda + nn] = s >> 4;  // exact: s = 16 * sum
                } else {
                    float yv;
                    if constexpr (PER_GROUP) {
                        float s = 0.f;
                        for (int w = 0; w < ks; ++w)
                            s += __int_as_float(red_smem[w * MT * kWave * 4 + e]);
                        yv = s * 0.0625f;
                    } else {
                        int s = 0;
                        for (int w = 0; w < ks; ++w)
                            s += red_smem[w * MT * kWave * 4 + e];
                        yv = bf16_to_f32(w_scales[nn]) * ((float)s * 0.0625f);
                    }
                    yv *= row_scales[m] * x_scale;
                    if (bias)
                        yv += bf16_to_f32(bias[nn]);
                    out[(int64_t)m * ldo + nn] = f32_to_bf16(yv);
                }
            }
        }
        __syncthreads();
    }
}

struct SkinnyShape {
    int mt, ks, gpw;
};

// MT = ceil(M / 16) m-tiles; GPW groups per wave (capped so that the register
// copy of the activations stays <= 64 VGPRs per m-tile); KS waves.
bool skinny_shape(int64_t M, int64_t K, SkinnyShape &s)
{
    if (M < 1 || M > 64)
        return false;
    const int ng = (int)(K / 64);
    s.mt = M <= 16 ? 1 : M <= 32 ? 2 : 4;
    const int gmax = s.mt == 1 ? 16 : s.mt == 2 ? 8 : 4;
    s.ks = (ng + gmax - 1) / gmax;
    if (s.ks < 4)
        s.ks = ng < 4 ? ng : 4;
    if (s.ks > kMaxWaves)
        return false;
    s.gpw = (ng + s.ks - 1) / s.ks;
    return true;
}

template <int MT, int GPW, bool PG, bool I32>
hipError_t launch_t(const SkinnyShape &sh, const int8_t *codes, int64_t ldq, const float *rs, int M,
                    int K, const uint8_t *packed, int64_t ldw, const uint16_t *ws, int N,
                    const uint16_t *bias, float xs, uint16_t *out, int64_t ldo, int32_t *acc,
                    int64_t lda, hipStream_t s)
{
    const int ntiles = N / 16;
    const size_t smem = (size_t)sh.ks * MT * kWave * 4 * sizeof(int);
    const dim3 grid((unsigned)ntiles);
    hipLaunchKernelGGL((w4_skinny_kernel<MT, GPW, PG, I32>), grid, dim3(sh.ks * kWave), smem, s,
                       codes, ldq, rs, M, K, packed, ldw, ws, N, bias, xs, out, ldo, acc, lda,
                       sh.gpw);
    return hipGetLastError();
}

template <int MT, int GPW>
hipError_t launch_mt(const SkinnyShape &sh, bool pg, bool i32, const int8_t *codes, int64_t ldq,
                     const float *rs, int M, int K, const uint8_t *packed, int64_t ldw,
                     const uint16_t *ws, int N, const uint16_t *bias, float xs, uint16_t *out,
                     int64_t ldo, int32_t *acc, int64_t lda, hipStream_t s)
{
    if (i32)
        return launch_t<MT, GPW, false, true>(sh, codes, ldq, rs, M, K, packed, ldw, ws, N, bias,
                                              xs, out, ldo, acc, lda, s);
    if (pg)
        return launch_t<MT, GPW, true, false>(sh, codes, ldq, rs, M, K, packed, ldw, ws, N, bias,
                                              xs, out, ldo, acc, lda, s);
    return launch_t<MT, GPW, false, false>(sh, codes, ldq, rs, M, K, packed, ldw, ws, N, bias, xs,
                                           out, ldo, acc, lda, s);
}

}  // namespace

bool w4_skinny_supports(int64_t M, int64_t K)
{
    SkinnyShape s;
    return skinny_shape(M, K, s);
}

int launch_w4_skinny(const int8_t *codes, int64_t ldq, const float *row_scales, int M, int K,
                     const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, bool per_group,
                     int N, const uint16_t *bias, float x_scale, uint16_t *out, int64_t ldo,
                     int32_t *acc_out, int64_t lda, void *stream)
{
    SkinnyShape sh;
    if (!skinny_shape(M, K, sh))
        return (int)hipErrorInvalidValue;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool i32 = acc_out != nullptr;
    hipError_t e;
    switch (sh.mt) {
    case 1:
        e = launch_mt<1, 16>(sh, per_group, i32, codes, ldq, row_scales, M, K, packed, ldw,
                             w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s);
        break;
    case 2:
        e = launch_mt<2, 8>(sh, per_group, i32, codes, ldq, row_scales, M, K, packed, ldw,
                            w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s);
        break;
    default:
        e = launch_mt<4, 4>(sh, per_group, i32, codes, ldq, row_scales, M, K, packed, ldw,
                            w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s);
        break;
    }
    return (int)e;
}

}  // namespace ck
