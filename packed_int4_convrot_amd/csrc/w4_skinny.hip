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
//   * a workgroup computes 16 output columns (weight rows n0 .. n0 + 15) for
//     all M activation rows; it has KS waves, and wave w owns a contiguous
//     range of GPW K-groups;
//   * each wave loads the activation operands of its groups into VGPRs and
//     streams its slice of the 16 weight rows (GPW * 32 bytes per row) into
//     its own LDS region with global_load_lds_dwordx4: every 1 KiB
//     instruction covers whole 16-byte chunks of at most 8 rows, at least 128
//     contiguous bytes of each, which HBM serves at full rate (8-byte fragment
//     loads straight from global memory would touch 16 rows x 32 bytes per
//     instruction);
//   * activation codes come either row-major (permuted in registers) or, from
//     the whole linear's own rotate-quant, in the tiled operand layout
//     (CodesLayout::kTiled16), where each operand is one contiguous 1 KiB
//     block: row-major operand loads touch 16 rows x 64 bytes per instruction,
//     which the memory pipeline serves as 64 separate requests, and every
//     workgroup reads all the codes (measured on MI355X at M = 32, N = 3840:
//     7.3 us per launch row-major, 5.4 us tiled);
//   * chunk slots inside an LDS row are XOR-swizzled by row, so the 8-byte
//     fragment reads of 16 rows hit 16 different bank groups; a wave reads
//     only its own region, so its own vmcnt wait is the only synchronisation;
//   * per-wave partial results are summed across waves through LDS in a fixed
//     order (deterministic), then scaled, biased and stored as bf16.
#include "ck_device.h"
#include "launch.h"

namespace ck {
namespace {

constexpr int kMaxWaves = kSkinnyMaxWaves;  // 512 threads: up to 256 VGPRs per lane

typedef __attribute__((address_space(3))) uint8_t lds_u8;

template <int MT, int GPW, bool PER_GROUP, bool OUT_I32, bool TILED>
__global__ __launch_bounds__(kMaxWaves * kWave) void w4_skinny_kernel(
    const int8_t *__restrict__ codes, int64_t ldq, const float *__restrict__ row_scales, int M,
    int K, const uint8_t *__restrict__ packed, int64_t ldw, const uint16_t *__restrict__ w_scales,
    int N, const uint16_t *__restrict__ bias, float x_scale, uint16_t *__restrict__ out,
    int64_t ldo, int32_t *__restrict__ acc_out, int64_t lda)
{
    constexpr int P = 32 * GPW;        // bytes of one weight row in a wave's slice
    constexpr int CPR = P / 16;        // 16-byte chunks per slice row
    constexpr int SLICE = 16 * P;      // bytes of a wave's slice (16 rows)
    constexpr int NLD = SLICE / 1024;  // DMA instructions per wave
    // Slot swizzle: chunk c of row r sits in slot c ^ (r >> SH), which spreads
    // a column of 16 rows over the 16 bank groups of 16 bytes.
    constexpr int SH = CPR >= 16 ? 0 : CPR == 8 ? 1 : 2;
    static_assert(CPR >= 4 && NLD * 1024 == SLICE, "slice shape");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_generic[];
    lds_u8 *smem = (lds_u8 *)smem_generic;

    const int ks = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int ng = K / 64;
    const int g0 = wave * GPW;
    const int cnt = max(0, min(GPW, ng - g0));
    const int col = lane % 16;
    const int kb = lane / 16;
    const int n0 = xcd_block(blockIdx.x, gridDim.x) * 16;
    lds_u8 *slice = smem + wave * SLICE;
    int *red_smem = reinterpret_cast<int *>(smem_generic + ks * SLICE);  // [KS][MT][64][4]

    // 1. Loads.  Row-major codes: the activations of this wave's groups first
    //    (clamped addresses; out-of-range values are replaced by zero below),
    //    then the weight scales, then the weight slice into LDS.  Tiled codes
    //    (each 1 KiB block is one operand, so the loads are whole lines): the
    //    weight slice first, as it comes from HBM, then scales and codes.
    u32x4 raw[GPW][MT];
    // Per-group weight scales, one dword per lane and 8 groups: lane l holds
    // the scales of columns n0 + 2 (l % 8) and + 1 in group g0 + l / 8 (+ 8 q),
    // a coalesced 256-byte load instead of GPW two-byte loads per lane; each
    // lane picks its column's scale from the owning lane with ds_bpermute.
    constexpr int kSwLd = PER_GROUP ? (GPW + 7) / 8 : 1;
    uint32_t swd[kSwLd];
    auto load_weights = [&]() {
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int s = 64 * j + lane;  // slot in the slice
            const int r = s / CPR;
            const int c = (s % CPR) ^ (r >> SH);  // chunk of row r stored in that slot
            if (c < 2 * cnt)
                __builtin_amdgcn_global_load_lds(packed + (int64_t)(n0 + r) * ldw + 32 * g0 + 16 * c,
                                                 slice + 1024 * j, 16, 0, 0);
        }
    };
    auto load_scales = [&]() {
        if constexpr (PER_GROUP) {
#pragma unroll
            for (int q = 0; q < kSwLd; ++q)
                swd[q] = *reinterpret_cast<const uint32_t *>(
                    w_scales + (int64_t)min(g0 + 8 * q + lane / 8, ng - 1) * N + n0 + 2 * (lane % 8));
        }
    };
    if constexpr (TILED) {
        load_weights();
        load_scales();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int8_t *tile = codes + (int64_t)mt * K * 16 + 16 * lane;
            if (M >= 16 * (mt + 1)) {
#pragma unroll
                for (int j = 0; j < GPW; ++j)
                    raw[j][mt] = *reinterpret_cast<const u32x4 *>(tile + min(g0 + j, ng - 1) * 1024);
            } else {
                // Partial last tile: rows past M were never written; skip them.
#pragma unroll
                for (int j = 0; j < GPW; ++j) {
                    raw[j][mt] = u32x4{0u, 0u, 0u, 0u};
                    if (mt * 16 + col < M)
                        raw[j][mt] = *reinterpret_cast<const u32x4 *>(tile + min(g0 + j, ng - 1) * 1024);
                }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < GPW; ++j)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = min(mt * 16 + col, M - 1);
                const int g = min(g0 + j, ng - 1);
                raw[j][mt] = *reinterpret_cast<const u32x4 *>(codes + (int64_t)m * ldq + 64 * g + 16 * kb);
            }
        load_scales();
        load_weights();
    }

    // The epilogue factors of this thread's first output (row scale, weight
    // scale, bias), loaded after the operands and waited for with them, so
    // that their latency does not follow the reduction barrier.
    const int e0 = threadIdx.x;
    const int m_e0 = min((e0 / (kWave * 4)) * 16 + 4 * ((e0 / 4) % kWave / 16) + e0 % 4, M - 1);
    const int n_e0 = n0 + (e0 / 4) % kWave % 16;
    float rs_e0 = 0.f, sw_e0 = 0.f, b_e0 = 0.f;
    if constexpr (!OUT_I32) {
        rs_e0 = row_scales[m_e0];
        if constexpr (!PER_GROUP)
            sw_e0 = bf16_to_f32(w_scales[n_e0]);
        if (bias)
            b_e0 = bf16_to_f32(bias[n_e0]);
    }

    // 2. Activation operands in the decode order (tiled codes already are),
    //    zero for rows past M and groups past K.
    v4i a[GPW][MT];
#pragma unroll
    for (int j = 0; j < GPW; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const bool live = j < cnt && mt * 16 + col < M;
            const v4i p = TILED ? v4i{(int)raw[j][mt][0], (int)raw[j][mt][1], (int)raw[j][mt][2],
                                      (int)raw[j][mt][3]}
                                : act_perm16(raw[j][mt][0], raw[j][mt][1], raw[j][mt][2], raw[j][mt][3]);
            a[j][mt] = live ? p : v4i{0, 0, 0, 0};
        }

    // 3. This wave's slice has landed once its own loads have retired.  Every
    //    group runs, without a branch, so that the LDS reads issue together:
    //    past K the slice holds stale bytes, multiplied by zero activations.
    wait_vmcnt0();

    u32x2 wq[GPW];
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        // Lane (col, kb) holds k = 64 g + 16 kb .. + 15: bytes 32 j + 8 kb of row col.
        const int c = 2 * j + (kb >> 1);
        wq[j] = *(const __attribute__((address_space(3))) u32x2 *)(slice + col * P + 16 * (c ^ (col >> SH)) +
                                                                    8 * (kb & 1));
    }
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
    for (int j = 0; j < GPW; ++j) {
        const v4i b = w4_operand_x16(wq[j][0], wq[j][1]);
        if constexpr (PER_GROUP) {
            const uint32_t pair = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * ((j % 8) * 8 + col / 2),
                                                                        (int)swd[j / 8]);
            const float sc = __uint_as_float((col & 1) ? pair & 0xffff0000u : pair << 16);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j][mt], b, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    y[mt][i] = __builtin_fmaf(sc, (float)d[i], y[mt][i]);
            }
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j][mt], b, acc[mt], 0, 0, 0);
        }
    }

    // 4. Cross-wave reduction: red[w][mt][lane][i], summed in wave order.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        int *dst = red_smem + ((wave * MT + mt) * kWave + lane) * 4;
        if constexpr (PER_GROUP)
            *reinterpret_cast<float4 *>(dst) = make_float4(y[mt][0], y[mt][1], y[mt][2], y[mt][3]);
        else
            *reinterpret_cast<int4 *>(dst) = make_int4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
    }
    __syncthreads();
    // Output e = (mt, lane l, i): row mt * 16 + 4 (l / 16) + i, column n0 + l % 16.
    auto finish = [&](int e, float rsm, float swm, float bm) {
        const int mt = e / (kWave * 4);
        const int l = (e / 4) % kWave;
        const int i = e % 4;
        const int m = mt * 16 + 4 * (l / 16) + i;
        const int nn = n0 + l % 16;
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
                    yv = s * 0.0625f * (rsm * x_scale);
                    if (bias)
                        yv += bm;
                } else {
                    int s = 0;
                    for (int w = 0; w < ks; ++w)
                        s += red_smem[w * MT * kWave * 4 + e];
                    yv = epilogue_channel((float)s, 0.0625f * swm, rsm * x_scale, bm);  // s = 16 * sum
                }
                out[(int64_t)m * ldo + nn] = f32_to_bf16(yv);
            }
        }
    };
    if (e0 < MT * kWave * 4)
        finish(e0, rs_e0, sw_e0, b_e0);
    for (int e = e0 + blockDim.x; e < MT * kWave * 4; e += blockDim.x) {
        const int l = (e / 4) % kWave;
        const int m = min((e / (kWave * 4)) * 16 + 4 * (l / 16) + e % 4, M - 1);
        const int nn = n0 + l % 16;
        float rsm = 0.f, swm = 0.f, bm = 0.f;
        if constexpr (!OUT_I32) {
            rsm = row_scales[m];
            if constexpr (!PER_GROUP)
                swm = bf16_to_f32(w_scales[nn]);
            if (bias)
                bm = bf16_to_f32(bias[nn]);
        }
        finish(e, rsm, swm, bm);
    }
}

template <int MT, int GPW, bool PG, bool I32, bool TL>
hipError_t launch_t(const SkinnyShape &sh, const int8_t *codes, int64_t ldq, const float *rs, int M,
                    int K, const uint8_t *packed, int64_t ldw, const uint16_t *ws, int N,
                    const uint16_t *bias, float xs, uint16_t *out, int64_t ldo, int32_t *acc,
                    int64_t lda, hipStream_t s)
{
    const int ntiles = N / 16;
    const size_t smem = (size_t)sh.ks * (16 * 32 * GPW + MT * kWave * 4 * sizeof(int));
    auto kern = w4_skinny_kernel<MT, GPW, PG, I32, TL>;
    constexpr size_t smem_max = (size_t)kMaxWaves * (16 * 32 * GPW + MT * kWave * 4 * sizeof(int));
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem_max);
    if (attr != hipSuccess)
        return attr;
    const dim3 grid((unsigned)ntiles);
    hipLaunchKernelGGL(kern, grid, dim3(sh.ks * kWave), smem, s,
                       codes, ldq, rs, M, K, packed, ldw, ws, N, bias, xs, out, ldo, acc, lda);
    return hipGetLastError();
}

// The int32 test epilogue reads row-major codes only; tiled codes come from
// the linear's own rotate-quant.
template <int MT, int GPW>
hipError_t launch_mt(const SkinnyShape &sh, bool pg, bool i32, bool tiled, const int8_t *codes,
                     int64_t ldq, const float *rs, int M, int K, const uint8_t *packed, int64_t ldw,
                     const uint16_t *ws, int N, const uint16_t *bias, float xs, uint16_t *out,
                     int64_t ldo, int32_t *acc, int64_t lda, hipStream_t s)
{
    if (i32)
        return tiled ? hipErrorInvalidValue
                     : launch_t<MT, GPW, false, true, false>(sh, codes, ldq, rs, M, K, packed, ldw, ws, N,
                                                             bias, xs, out, ldo, acc, lda, s);
    if (tiled) {
        if (pg)
            return launch_t<MT, GPW, true, false, true>(sh, codes, ldq, rs, M, K, packed, ldw, ws, N, bias,
                                                        xs, out, ldo, acc, lda, s);
        return launch_t<MT, GPW, false, false, true>(sh, codes, ldq, rs, M, K, packed, ldw, ws, N, bias,
                                                     xs, out, ldo, acc, lda, s);
    }
    if (pg)
        return launch_t<MT, GPW, true, false, false>(sh, codes, ldq, rs, M, K, packed, ldw, ws, N, bias,
                                                     xs, out, ldo, acc, lda, s);
    return launch_t<MT, GPW, false, false, false>(sh, codes, ldq, rs, M, K, packed, ldw, ws, N, bias, xs,
                                                  out, ldo, acc, lda, s);
}

}  // namespace

int launch_w4_skinny(const int8_t *codes, int64_t ldq, bool tiled, const float *row_scales, int M,
                     int K, const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, bool per_group,
                     int N, const uint16_t *bias, float x_scale, uint16_t *out, int64_t ldo,
                     int32_t *acc_out, int64_t lda, void *stream)
{
    SkinnyShape sh;
    if (!skinny_shape(M, K, sh))
        return (int)hipErrorInvalidValue;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool i32 = acc_out != nullptr;
    hipError_t e;
    switch (sh.mt * 100 + sh.gpw) {
    case 116:
        e = launch_mt<1, 16>(sh, per_group, i32, tiled, codes, ldq, row_scales, M, K, packed, ldw,
                             w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s);
        break;
    case 208:
        e = launch_mt<2, 8>(sh, per_group, i32, tiled, codes, ldq, row_scales, M, K, packed, ldw,
                            w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s);
        break;
    case 216:
        e = launch_mt<2, 16>(sh, per_group, i32, tiled, codes, ldq, row_scales, M, K, packed, ldw,
                             w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s);
        break;
    case 408:
        e = launch_mt<4, 8>(sh, per_group, i32, tiled, codes, ldq, row_scales, M, K, packed, ldw,
                            w_scales, N, bias, x_scale, out, ldo, acc_out, lda, s);
        break;
    default:
        e = hipErrorInvalidValue;
        break;
    }
    return (int)e;
}

}  // namespace ck
