// Tiled int8-MFMA GEMM for the ConvRot packed-INT4 linear at large M.
//
// acc[m,n] = sum_k codes[m,k] * (q[n,k] - 8) in int32, then the scale
// epilogue (row scale x per-channel or per-group weight scale, optional bias)
// and a bf16 store.  The integer matmul with a rowwise x weight-scale epilogue
// follows the W4A8 path of "[PR #182] HIP port of #176 ..." (description) and
// the W4A4/W4A8 ConvRot matmul of "feat: support packed INT4 convrot models"
// (summary); the difference is that the int4 weights are decoded in VGPRs
// right before CDNA4 int8 MFMA instead of being unpacked to memory.
//
// Tiling (block = 4 waves as 2 x 2):
//   * block tile BM x BN = (2*WM*32) x (2*WN*32), K step BK = 64 (one group);
//   * v_mfma_i32_32x32x32_i8, each wave owns WM x WN 32x32 accumulator tiles;
//   * LDS holds two stages of [BM][64] activation bytes (rows padded to 80 B)
//     and [BN][32] packed weight bytes (rows padded to 40 B); the pads make
//     the 16-byte (A) and 8-byte (B) fragment reads bank-conflict free;
//   * activations are permuted to the nibble-decode k order while they are
//     staged (global -> VGPR -> LDS), once per block and K step;
//   * the next K step's global loads are issued before the current step's
//     MFMAs; one barrier per K step;
//   * blocks are renumbered so that each XCD (blocks are dealt to the 8 XCDs
//     round-robin) gets a contiguous run of tiles that share activation rows.
// Operand layouts of v_mfma_i32_32x32x32_i8: lane l holds 16 int8 of row
// (A) / column (B) l % 32, k-half l / 32; D lane l register r holds
// D[8*(r/4) + 4*(l/32) + r%4][l % 32].
#include "ck_device.h"
#include "launch.h"

namespace ck {
namespace {

constexpr int kAPitch = 80;  // bytes per staged activation row (64 + 16 pad)
constexpr int kBPitch = 40;  // bytes per staged packed-weight row (32 + 8 pad)
constexpr int kThreads = 256;
constexpr int kXcds = 8;

template <int WM, int WN, bool PER_GROUP, bool OUT_I32>
__global__ __launch_bounds__(kThreads) void w4_gemm_kernel(
    const int8_t *__restrict__ codes, int64_t ldq, const float *__restrict__ row_scales, int M,
    int K, const uint8_t *__restrict__ packed, int64_t ldw, const uint16_t *__restrict__ w_scales,
    int N, const uint16_t *__restrict__ bias, float x_scale, uint16_t *__restrict__ out,
    int64_t ldo, int32_t *__restrict__ acc_out, int64_t lda)
{
    constexpr int BM = 2 * WM * 32;
    constexpr int BN = 2 * WN * 32;
    constexpr int A_CHUNKS = BM * 4 / kThreads;  // 16-byte chunks per thread per K step
    constexpr int B_CHUNKS = BN * 2 / kThreads;
    static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small for the block");
    __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * kAPitch];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * kBPitch];

    // XCD-aware renumbering of the block index.
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    const int b = blockIdx.x;
    const int xcd = b % kXcds, local = b / kXcds;
    const int per = tiles / kXcds, rem = tiles % kXcds;
    const int tile = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
    const int m0 = (tile / tiles_n) * BM;
    const int n0 = (tile % tiles_n) * BN;

    const int t = threadIdx.x;
    const int wave = t / kWave, lane = t % kWave;
    const int wm = wave / 2, wn = wave % 2;
    const int l32 = lane % 32, h = lane / 32;
    const int ksteps = K / 64;

    // Global -> register staging.
    uint4 ra[A_CHUNKS], rb[B_CHUNKS];
    auto load_stage = [&](int kt) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int q = t + i * kThreads;
            const int row = q / 4, c = q % 4;
            const int m = m0 + row;
            ra[i] = m < M ? *reinterpret_cast<const uint4 *>(codes + (int64_t)m * ldq + kt * 64 + 16 * c)
                          : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) {
            const int q = t + i * kThreads;
            const int row = q / 2, c = q % 2;
            const int n = n0 + row;
            rb[i] = n < N ? *reinterpret_cast<const uint4 *>(packed + (int64_t)n * ldw + kt * 32 + 16 * c)
                          : make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
        }
    };
    auto store_stage = [&](int st) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int q = t + i * kThreads;
            const int row = q / 4, c = q % 4;
            const v4i p = act_perm16(ra[i].x, ra[i].y, ra[i].z, ra[i].w);
            *reinterpret_cast<v4i *>(&As[st][row * kAPitch + 16 * c]) = p;
        }
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) {
            const int q = t + i * kThreads;
            const int row = q / 2, c = q % 2;
            uint2 *dst = reinterpret_cast<uint2 *>(&Bs[st][row * kBPitch + 16 * c]);
            dst[0] = make_uint2(rb[i].x, rb[i].y);
            dst[1] = make_uint2(rb[i].z, rb[i].w);
        }
    };

    v16i acc[WM][WN];
    float y[PER_GROUP ? WM : 1][PER_GROUP ? WN : 1][PER_GROUP ? 16 : 1];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[i][j][r] = 0;
                if constexpr (PER_GROUP)
                    y[i][j][r] = 0.f;
            }

    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int kt = 0; kt < ksteps; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < ksteps)
            load_stage(kt + 1);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            v4i af[WM], bf[WN];
#pragma unroll
            for (int i = 0; i < WM; ++i)
                af[i] = *reinterpret_cast<const v4i *>(
                    &As[st][(wm * WM * 32 + i * 32 + l32) * kAPitch + 32 * s + 16 * h]);
#pragma unroll
            for (int j = 0; j < WN; ++j) {
                const uint2 p = *reinterpret_cast<const uint2 *>(
                    &Bs[st][(wn * WN * 32 + j * 32 + l32) * kBPitch + 16 * s + 8 * h]);
                bf[j] = w4_operand_x16(p.x, p.y);
            }
#pragma unroll
            for (int i = 0; i < WM; ++i)
#pragma unroll
                for (int j = 0; j < WN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if constexpr (PER_GROUP) {
#pragma unroll
            for (int j = 0; j < WN; ++j) {
                const int n = n0 + wn * WN * 32 + j * 32 + l32;
                const float sc = n < N ? bf16_to_f32(w_scales[(int64_t)kt * N + n]) : 0.f;
#pragma unroll
                for (int i = 0; i < WM; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        y[i][j][r] = __builtin_fmaf(sc, (float)acc[i][j][r], y[i][j][r]);
                        acc[i][j][r] = 0;
                    }
            }
        }
        if (kt + 1 < ksteps)
            store_stage(st ^ 1);
        __syncthreads();
    }

    // Epilogue.
#pragma unroll
    for (int j = 0; j < WN; ++j) {
        const int n = n0 + wn * WN * 32 + j * 32 + l32;
        if (n >= N)
            continue;
        float colscale = 0.0625f;
        if constexpr (!PER_GROUP && !OUT_I32)
            colscale *= bf16_to_f32(w_scales[n]);
        const float bn = (!OUT_I32 && bias) ? bf16_to_f32(bias[n]) : 0.f;
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * WM * 32 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                if (m < M) {
                    if constexpr (OUT_I32) {
                        acc_out[(int64_t)m * lda + n] = acc[i][j][r] >> 4;
                    } else {
                        float v;
                        if constexpr (PER_GROUP)
                            v = y[i][j][r] * colscale;
                        else
                            v = (float)acc[i][j][r] * colscale;
                        v = v * (row_scales[m] * x_scale) + bn;
                        out[(int64_t)m * ldo + n] = f32_to_bf16(v);
                    }
                }
            }
    }
}

template <int WM, int WN, bool PG, bool I32>
hipError_t launch_t(const int8_t *codes, int64_t ldq, const float *rs, int M, int K,
                    const uint8_t *packed, int64_t ldw, const uint16_t *ws, int N,
                    const uint16_t *bias, float xs, uint16_t *out, int64_t ldo, int32_t *acc,
                    int64_t lda, hipStream_t s)
{
    constexpr int BM = 2 * WM * 32, BN = 2 * WN * 32;
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL((w4_gemm_kernel<WM, WN, PG, I32>), dim3(tiles), dim3(kThreads), 0, s, codes,
                       ldq, rs, M, K, packed, ldw, ws, N, bias, xs, out, ldo, acc, lda);
    return hipGetLastError();
}

}  // namespace

int launch_w4_gemm(const int8_t *codes, int64_t ldq, const float *row_scales, int M, int K,
                   const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, bool per_group,
                   int N, const uint16_t *bias, float x_scale, uint16_t *out, int64_t ldo,
                   int32_t *acc_out, int64_t lda, void *stream)
{
    if (M <= 0)
        return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (acc_out)
        e = launch_t<4, 4, false, true>(codes, ldq, row_scales, M, K, packed, ldw, w_scales, N,
                                        bias, x_scale, out, ldo, acc_out, lda, s);
    else if (per_group)
        e = launch_t<2, 2, true, false>(codes, ldq, row_scales, M, K, packed, ldw, w_scales, N,
                                        bias, x_scale, out, ldo, acc_out, lda, s);
    else
        e = launch_t<4, 4, false, false>(codes, ldq, row_scales, M, K, packed, ldw, w_scales, N,
                                         bias, x_scale, out, ldo, acc_out, lda, s);
    return (int)e;
}

}  // namespace ck
