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
// Tiling (block = WGM x WGN waves):
//   * block tile BM x BN = (WGM*WM*32) x (WGN*WN*32), K step BK = 64 (one group);
//   * v_mfma_i32_32x32x32_i8, each wave owns WM x WN 32x32 accumulator tiles
//     (in AGPRs); the per-channel kernel runs 8 waves (two per SIMD) on a
//     256 x 256 tile, so one wave's LDS and barrier waits are covered by the
//     other wave's MFMAs;
//   * operands move global -> LDS directly (global_load_lds_dwordx4, no VGPR
//     staging) into a ring of NST stages, so the loads of K step t + NST - 1
//     are in flight while step t is multiplied;
//   * LDS rows are unpadded ([BM][64] activation bytes, [BN][32] packed weight
//     bytes); the 16-byte slots inside a row are XOR-swizzled by row so that
//     the 16-byte fragment reads are bank-conflict free; the DMA writes lanes
//     contiguously, so each lane loads the global chunk that belongs in its
//     slot;
//   * each lane reads one 16-byte weight fragment per K step (both 32-wide k
//     halves) and decodes it in VGPRs; activation fragments are permuted to
//     the decode's even/odd k order as they are read;
//   * blocks are renumbered so that each XCD (blocks are dealt to the 8 XCDs
//     round-robin) gets a contiguous run of tiles that share activation rows.
// Operand layouts of v_mfma_i32_32x32x32_i8: lane l holds 16 int8 of row
// (A) / column (B) l % 32, k-half l / 32; D lane l register r holds
// D[8*(r/4) + 4*(l/32) + r%4][l % 32].  Lane half h and K-half s select
// activation chunk 2h + s (codes k in [32h + 16s, +16)) and weight bytes
// [16h + 8s, +8) of the row's 32 bytes, i.e. the same 16 k values.
//
// A4 variant (W4A4): the activation codes arrive packed two per byte like the
// weights ([M][K/2] bytes, two's complement nibbles in [-7, 7]), so the
// activation stage, its DMA and its LDS reads are half as large, and both
// operands are decoded to 16 * value: the accumulator carries a factor 256.
#include "ck_device.h"
#include "launch.h"

namespace ck {
namespace {

constexpr int kStages = 4;

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Slot swizzles, chosen by measuring SQ_LDS_BANK_CONFLICT on gfx950 for the
// fragment read patterns: (r >> 2) & 3 for the 64-byte activation rows and
// ((n >> 2) ^ (n >> 3)) & 1 for the 32-byte weight rows read without conflicts
// (e.g. ((r >> 1) ^ (r >> 3)) & 3 gave 2-way conflicts).
__device__ __forceinline__ int swz_a(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swz_b(int n) { return ((n >> 2) ^ (n >> 3)) & 1; }

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int WGM, int WGN, int WM, int WN, int NST, bool PER_GROUP, bool OUT_I32, bool A4>
__global__ __launch_bounds__(WGM * WGN * kWave) void w4_gemm_kernel(
    const int8_t *__restrict__ codes, int64_t ldq, const float *__restrict__ row_scales, int M,
    int K, const uint8_t *__restrict__ packed, int64_t ldw, const uint16_t *__restrict__ w_scales,
    int N, const uint16_t *__restrict__ bias, float x_scale, uint16_t *__restrict__ out,
    int64_t ldo, int32_t *__restrict__ acc_out, int64_t lda)
{
    // Per-channel and int32 results are computed transposed (weights as the
    // MFMA A operand), so that a lane holds one output row and four
    // consecutive columns per register group; the per-group form keeps one
    // column per lane, which is what its per-K-step scale needs.
    constexpr bool TRANS = !PER_GROUP;
    constexpr int NWAVES = WGM * WGN;
    constexpr int BM = WGM * WM * 32;
    constexpr int BN = WGN * WN * 32;
    constexpr int A_ROW = A4 ? 32 : 64;            // activation bytes per row and K step
    constexpr int A_BYTES = BM * A_ROW;
    constexpr int STAGE = A_BYTES + BN * 32;
    // Activation DMA per wave and stage: A_LD instructions of A_LANES lanes
    // (a packed activation tile smaller than 1 KiB per wave leaves lanes idle).
    constexpr int A_PER = A_BYTES / NWAVES;
    constexpr int A_LANES = A_PER >= 1024 ? kWave : A_PER / 16;
    constexpr int A_LD = A_PER >= 1024 ? A_PER / 1024 : 1;
    constexpr int B_LD = BN * 32 / 1024 / NWAVES;  // 1 KiB DMA instructions per wave per stage
    static_assert(A_LD * NWAVES * A_LANES * 16 == A_BYTES && B_LD * NWAVES * 1024 == BN * 32, "DMA split");
    // Accumulator factor of the decoded operands: 16 (weights) or 256 (both).
    constexpr int ACC_SHIFT = A4 ? 8 : 4;
    constexpr float ACC_SCALE = A4 ? 1.f / 256.f : 1.f / 16.f;
    constexpr int L = A_LD + B_LD;
    static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for the block");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_generic[];
    lds_u8 *smem = (lds_u8 *)smem_generic;

    // XCD-aware renumbering of the block index.
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    const int tile = xcd_block(blockIdx.x, tiles);
    const int m0 = (tile / tiles_n) * BM;
    const int n0 = (tile % tiles_n) * BN;

    const int t = threadIdx.x;
    const int wave = t / kWave, lane = t % kWave;
    const int wm = wave / WGN, wn = wave % WGN;
    const int l32 = lane % 32, h = lane / 32;
    const int ksteps = K / 64;

    // Global -> LDS for K step kt into ring slot st.  Rows past M / N re-read
    // the last valid row; their results are never stored.
    auto issue_stage = [&](int kt, int st) {
        lds_u8 *sa = smem + st * STAGE;
#pragma unroll
        for (int j = 0; j < A_LD; ++j) {
            const int q = (wave * A_LD + j) * A_LANES + lane;
            if (A_LANES == kWave || lane < A_LANES) {
                int r, c;
                if constexpr (A4) {
                    r = q >> 1;
                    c = (q & 1) ^ swz_b(r);
                } else {
                    r = q >> 2;
                    c = (q & 3) ^ swz_a(r);
                }
                const int m = min(m0 + r, M - 1);
                __builtin_amdgcn_global_load_lds(codes + (int64_t)m * ldq + kt * A_ROW + 16 * c,
                                                 sa + (wave * A_LD + j) * A_LANES * 16, 16, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < B_LD; ++j) {
            const int q = (wave * B_LD + j) * kWave + lane;
            const int n = q >> 1, c = (q & 1) ^ swz_b(q >> 1);
            const int nn = min(n0 + n, N - 1);
            __builtin_amdgcn_global_load_lds(packed + (int64_t)nn * ldw + kt * 32 + 16 * c,
                                             sa + A_BYTES + (wave * B_LD + j) * 1024, 16, 0, 0);
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

#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < ksteps)
            issue_stage(s, s);

    for (int kt = 0; kt < ksteps; ++kt) {
        const int st = kt % NST;
        // This wave's DMA for step kt has landed once at most the later
        // stages' loads are outstanding; the barrier extends that to all
        // waves and also retires every read of the slot refilled below.
        if (kt + NST - 2 < ksteps)
            wait_vmcnt<(NST - 2) * L>();
        else
            wait_vmcnt<0>();
        // A bare barrier: __syncthreads() would also wait for every DMA still
        // in flight (vmcnt(0)) and drain the ring.  LDS reads of the previous
        // step were consumed by its MFMAs, so no LDS fence is needed.
        __builtin_amdgcn_s_barrier();
        uint16_t sc[PER_GROUP ? WN : 1];
        if constexpr (PER_GROUP) {
#pragma unroll
            for (int j = 0; j < WN; ++j)
                sc[j] = w_scales[(int64_t)kt * N + min(n0 + wn * WN * 32 + j * 32 + l32, N - 1)];
        }
        if (kt + NST - 1 < ksteps)
            issue_stage(kt + NST - 1, (kt + NST - 1) % NST);

        // All fragment reads of this K step are issued before the first MFMA,
        // so a single LDS latency is exposed per step instead of one per
        // fragment.
        const lds_u8 *sa = smem + st * STAGE;
        const lds_u8 *sb = sa + A_BYTES;
        u32x4 bq[WN];
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            const int n = wn * WN * 32 + j * 32 + l32;
            bq[j] = *(const __attribute__((address_space(3))) u32x4 *)(sb + n * 32 + 16 * (h ^ swz_b(n)));
        }
        u32x4 aq[A4 ? 1 : 2][WM];
#pragma unroll
        for (int s = 0; s < (A4 ? 1 : 2); ++s)
#pragma unroll
            for (int i = 0; i < WM; ++i) {
                const int r = wm * WM * 32 + i * 32 + l32;
                if constexpr (A4)  // the lane's 32 k values, like a weight fragment
                    aq[s][i] = *(const __attribute__((address_space(3))) u32x4 *)(
                        sa + r * 32 + 16 * (h ^ swz_b(r)));
                else
                    aq[s][i] = *(const __attribute__((address_space(3))) u32x4 *)(
                        sa + r * 64 + 16 * ((2 * h + s) ^ swz_a(r)));
            }
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            v4i bf[WN];
#pragma unroll
            for (int j = 0; j < WN; ++j)
                bf[j] = w4_operand_x16(bq[j][2 * s], bq[j][2 * s + 1]);
#pragma unroll
            for (int i = 0; i < WM; ++i) {
                v4i af;
                if constexpr (A4)
                    af = a4_operand_x16(aq[0][i][2 * s], aq[0][i][2 * s + 1]);
                else
                    af = act_perm16(aq[s][i][0], aq[s][i][1], aq[s][i][2], aq[s][i][3]);
#pragma unroll
                for (int j = 0; j < WN; ++j) {
                    if constexpr (TRANS)  // D^T[n][m]: lane = row m, registers = columns n
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[j], af, acc[i][j], 0, 0, 0);
                    else  // per group: the step's first product starts from zero
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                            af, bf[j], s == 0 ? v16i{} : acc[i][j], 0, 0, 0);
                }
            }
        }
        if constexpr (PER_GROUP) {
#pragma unroll
            for (int j = 0; j < WN; ++j) {
                const float scf = bf16_to_f32(sc[j]);
#pragma unroll
                for (int i = 0; i < WM; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        y[i][j][r] = __builtin_fmaf(scf, (float)acc[i][j][r], y[i][j][r]);
            }
        }
    }

    // Epilogue.
    if constexpr (TRANS) {
        // Lane l holds rows m = m0w + 32 i + l32 and, in register group q,
        // columns n = n0w + 32 j + 8 q + 4 h + (0..3).
        const int m0w = m0 + wm * WM * 32;
        const int n0w = n0 + wn * WN * 32;
        if constexpr (OUT_I32) {
#pragma unroll
            for (int i = 0; i < WM; ++i) {
                const int m = m0w + i * 32 + l32;
                if (m < M)
#pragma unroll
                    for (int j = 0; j < WN; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int n = n0w + j * 32 + 8 * q + 4 * h;
                            if (n < N) {
                                const v4i v = {acc[i][j][4 * q] >> ACC_SHIFT, acc[i][j][4 * q + 1] >> ACC_SHIFT,
                                               acc[i][j][4 * q + 2] >> ACC_SHIFT, acc[i][j][4 * q + 3] >> ACC_SHIFT};
                                *reinterpret_cast<v4i *>(acc_out + (int64_t)m * lda + n) = v;
                            }
                        }
            }
        } else {
            // Stage the wave's 32 WM x 32 WN bf16 tile in LDS (rows padded to
            // 16 bytes past the tile width) and write it back with 16-byte
            // row-contiguous stores.  Column factors (weight scale over the
            // accumulator factor) and
            // bias are loaded one 32-column tile at a time to bound registers.
            constexpr int TW = WN * 32;          // tile width (columns)
            constexpr int PITCH = TW * 2 + 16;   // bytes per staged row
            float rsc[WM];
#pragma unroll
            for (int i = 0; i < WM; ++i)
                rsc[i] = row_scales[min(m0w + i * 32 + l32, M - 1)] * x_scale;
            __builtin_amdgcn_s_barrier();        // every wave is done with the operand stages
            lds_u8 *wt = smem + wave * (WM * 32 * PITCH);
#pragma unroll
            for (int j = 0; j < WN; ++j) {
                float cs[4][4], bc[4][4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int n = min(n0w + j * 32 + 8 * q + 4 * h + t, N - 1);
                        cs[q][t] = ACC_SCALE * bf16_to_f32(w_scales[n]);
                        bc[q][t] = bias ? bf16_to_f32(bias[n]) : 0.f;
                    }
#pragma unroll
                for (int i = 0; i < WM; ++i) {
                    const int ml = i * 32 + l32;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            v[t] = __builtin_fmaf((float)acc[i][j][4 * q + t], cs[q][t] * rsc[i], bc[q][t]);
                        const u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                        *(__attribute__((address_space(3))) u32x2 *)(wt + ml * PITCH + (j * 32 + 8 * q + 4 * h) * 2) = pk;
                    }
                }
            }
            constexpr int CHUNKS = TW * 2 / 16;      // 16-byte chunks per row
            constexpr int ROWS = kWave / CHUNKS;     // rows per store instruction
#pragma unroll
            for (int it = 0; it < WM * 32 / ROWS; ++it) {
                const int ml = it * ROWS + lane / CHUNKS;
                const int c = lane % CHUNKS;
                const u32x4 v = *(const __attribute__((address_space(3))) u32x4 *)(wt + ml * PITCH + 16 * c);
                const int m = m0w + ml, n = n0w + 8 * c;
                if (m < M && n < N)
                    *reinterpret_cast<u32x4 *>(out + (int64_t)m * ldo + n) = v;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            const int n = n0 + wn * WN * 32 + j * 32 + l32;
            if (n >= N)
                continue;
            const float bn = bias ? bf16_to_f32(bias[n]) : 0.f;
#pragma unroll
            for (int i = 0; i < WM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * WM * 32 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                    if (m < M) {
                        const float v = y[i][j][r] * ACC_SCALE * (row_scales[m] * x_scale) + bn;
                        out[(int64_t)m * ldo + n] = f32_to_bf16(v);
                    }
                }
        }
    }
}

template <int WGM, int WGN, int WM, int WN, bool PG, bool I32, bool A4>
hipError_t launch_t(const int8_t *codes, int64_t ldq, const float *rs, int M, int K,
                    const uint8_t *packed, int64_t ldw, const uint16_t *ws, int N,
                    const uint16_t *bias, float xs, uint16_t *out, int64_t ldo, int32_t *acc,
                    int64_t lda, hipStream_t s)
{
    constexpr int BM = WGM * WM * 32, BN = WGN * WN * 32;
    constexpr size_t stages = (size_t)kStages * (BM * (A4 ? 32 : 64) + BN * 32);
    constexpr size_t staging = PG ? 0 : (size_t)WGM * WGN * (WM * 32) * (WN * 32 * 2 + 16);
    constexpr size_t smem = stages > staging ? stages : staging;
    auto kern = w4_gemm_kernel<WGM, WGN, WM, WN, kStages, PG, I32, A4>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (attr != hipSuccess)
        return attr;
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(WGM * WGN * kWave), smem, s, codes, ldq, rs, M, K, packed,
                       ldw, ws, N, bias, xs, out, ldo, acc, lda);
    return hipGetLastError();
}

}  // namespace

int launch_w4_gemm(const int8_t *codes, int64_t ldq, const float *row_scales, int M, int K,
                   const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, bool per_group,
                   int N, const uint16_t *bias, float x_scale, uint16_t *out, int64_t ldo,
                   int32_t *acc_out, int64_t lda, bool a4, void *stream)
{
    if (M <= 0)
        return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
#define CK_GEMM_LAUNCH(A4)                                                                              \
    if (acc_out)                                                                                        \
        return (int)launch_t<2, 4, 4, 2, false, true, A4>(codes, ldq, row_scales, M, K, packed, ldw,    \
                                                          w_scales, N, bias, x_scale, out, ldo,         \
                                                          acc_out, lda, s);                             \
    if (per_group)                                                                                      \
        return (int)launch_t<2, 4, 2, 2, true, false, A4>(codes, ldq, row_scales, M, K, packed, ldw,    \
                                                          w_scales, N, bias, x_scale, out, ldo,         \
                                                          acc_out, lda, s);                             \
    return (int)launch_t<2, 4, 4, 2, false, false, A4>(codes, ldq, row_scales, M, K, packed, ldw,       \
                                                       w_scales, N, bias, x_scale, out, ldo, acc_out,   \
                                                       lda, s);
    if (a4) {
        CK_GEMM_LAUNCH(true)
    }
    CK_GEMM_LAUNCH(false)
#undef CK_GEMM_LAUNCH
}

}  // namespace ck
