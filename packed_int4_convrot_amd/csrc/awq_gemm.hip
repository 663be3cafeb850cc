// AWQ W4A16 prefill GEMM (many activation rows) on bf16 MFMA.
//
// Computes out = x . W^T (+ bias) with the weight rebuilt as the dequantise
// path of "comfy_kitchen/tensor/awq_w4a16.py" (dequantize()) does it, in the
// bf16 compute dtype, one tensor operation at a time:
//   W[n, k] = bf16( bf16((q - 8) * s[k/64, n]) + z[k/64, n] )
// then a bf16 x bf16 product with fp32 accumulation and a bf16 store.  The
// rebuilt weight is never written to memory: each wave dequantises the
// fragments it multiplies, in VGPRs, once per K step.
//
// Tiling: 4 waves (one per SIMD), block tile 256 x 256, each wave 256 rows x
// 64 weight rows = 8 x 2 tiles of v_mfma_f32_32x32x16_bf16 (accumulators in
// AGPRs).  Weights are the MFMA A operand, so a lane holds one output row and
// four consecutive output columns per register group.  K step = 64 (one
// scale group); a stage holds two K steps of both operands (256-byte x rows,
// 64-byte weight rows), double-buffered and filled by buffer_load ... lds,
// one barrier per stage.  The activation fragments of sub-step v + 1 are
// read, and its weight fragments dequantised, while sub-step v multiplies.
// MFMA operand layout: lane l holds 8 consecutive k of row l % 32, k = 8 (l /
// 32) + e within a 16-wide sub-step; both operands use the same assignment,
// with sub-step u of a K step covering k = 16 u .. 16 u + 15.
#include <type_traits>

#include "ck_device.h"
#include "launch.h"

namespace ck {
namespace {

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) const uint32_t lds_u32;
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bfv __attribute__((ext_vector_type(8)));

constexpr int kNst = 2;                       // stage buffers
constexpr int kKS = 2;                        // K steps (64 wide) per stage
constexpr int kXRow = 128 * kKS;              // x bytes per row and stage (bf16)
constexpr int kWRow = 32 * kKS;               // packed weight bytes per row and stage
// Block shape: NW waves side by side over the weight rows, each wave WM x WN
// 32x32 tiles.
template <int WM, int WN, int NW>
struct Shape {
    static constexpr int kWaves = NW;
    static constexpr int BM = WM * 32;
    static constexpr int BN = kWaves * WN * 32;
    static constexpr int XBytes = BM * kXRow;
    static constexpr int Stage = XBytes + BN * kWRow;
    static constexpr int XLanes = XBytes / kWaves >= 1024 ? kWave : XBytes / kWaves / 16;
    static constexpr int XLd = XBytes / kWaves >= 1024 ? XBytes / kWaves / 1024 : 1;
    static constexpr int WLanes = BN * kWRow / kWaves >= 1024 ? kWave : BN * kWRow / kWaves / 16;
    static constexpr int WLd = BN * kWRow / kWaves >= 1024 ? BN * kWRow / kWaves / 1024 : 1;
    static constexpr int TW = WN * 32;         // output columns per wave
    static constexpr int Pitch = TW * 2 + 16;  // staged epilogue row, bytes
    static constexpr int Smem = kWaves * BM * Pitch > kNst * Stage ? kWaves * BM * Pitch : kNst * Stage;
    static_assert(XLd * kWaves * XLanes * 16 == XBytes && WLd * kWaves * WLanes * 16 == BN * kWRow, "DMA split");
    static_assert(Smem <= 160 * 1024, "LDS");
};

// Slot swizzles for 32 consecutive rows reading one 16-byte slot each (lane
// half in bit 0 of the slot): a 256-byte x row spans all 64 banks, so the
// 16 rows of a quarter-wave take 16 distinct slots (r & 15); 64-byte weight
// rows use (r >> 2) & 3, measured conflict-free for this pattern.
__device__ __forceinline__ int swz16(int r) { return r & 15; }
__device__ __forceinline__ int swz4(int r) { return (r >> 2) & 3; }

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Eight packed codes (one dword, byte j = column 2j | column 2j+1 << 4) to
// eight bf16 weights in column order, each rounded as the bf16 tensor
// operations round: bf16(bf16((q - 8) s) + z).  (q - 8) s is exact in fp32.
__device__ __forceinline__ v8bfv dequant8(uint32_t d, float s, float m8s, float z)
{
    uint32_t lo = d & 0x0f0f0f0fu, hi = (d >> 4) & 0x0f0f0f0fu;
    // Opaque to the compiler, so that each code converts straight from its
    // byte (v_cvt_f32_ubyte0..3) and each pair rounds to bf16 with one
    // v_cvt_pk_bf16_f32, instead of the per-element forms it would choose.
    asm("" : "+v"(lo), "+v"(hi));
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float q0 = (float)((lo >> (8 * i)) & 0xffu);
        const float q1 = (float)((hi >> (8 * i)) & 0xffu);
        uint32_t p = pack_bf16x2(__builtin_fmaf(q0, s, m8s), __builtin_fmaf(q1, s, m8s));
        asm("" : "+v"(p));
        r[i] = pack_bf16x2(__uint_as_float(p << 16) + z, __uint_as_float(p & 0xffff0000u) + z);
    }
    return __builtin_bit_cast(v8bfv, r);
}

template <int WM, int WN, int NW>
__global__ __launch_bounds__(NW * kWave) void awq_gemm_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int M, int K, const uint8_t *__restrict__ packed,
    int64_t ldw, const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros, int N,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ out, int64_t ldo)
{
    using S = Shape<WM, WN, NW>;
    constexpr int kWaves = NW;
    constexpr int kBM = S::BM, kBN = S::BN, kXBytes = S::XBytes, kStage = S::Stage, kTW = S::TW;
    constexpr int kPitch = S::Pitch;
    constexpr int kWM = WM, kWN = WN;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_generic[];
    lds_u8 *smem = (lds_u8 *)smem_generic;

    // XCD-aware renumbering, then a grouped raster (runs of kGroupM tile rows
    // walked column by column), so that the tiles an XCD runs at the same time
    // share a few activation and weight blocks.
    constexpr int kGroupM = 4;
    const int tiles_m = (M + kBM - 1) / kBM;
    const int tiles_n = (N + kBN - 1) / kBN;
    const int tile = xcd_block(blockIdx.x, tiles_m * tiles_n);
    const int group = tile / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int group_m = min(kGroupM, tiles_m - first_m);
    const int in_group = tile - group * kGroupM * tiles_n;
    const int m0 = (first_m + in_group % group_m) * kBM;
    const int n0 = (in_group / group_m) * kBN;

    const int t = threadIdx.x;
    const int wave = t / kWave, lane = t % kWave;
    const int l32 = lane % 32, h = lane / 32;
    const int ksteps = K / 64;

    // Buffer resources spanning exactly the block's rows: rows past M / N read
    // as zero and their results are never stored.
    const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(x + (int64_t)m0 * ldx), (short)0,
        (int)((int64_t)(min(M - m0, kBM) - 1) * ldx * 2 + (int64_t)K * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(packed + (int64_t)n0 * ldw), (short)0,
        (int)((int64_t)(min(N - n0, kBN) - 1) * ldw + K / 2), 0x00020000);

    // Global -> LDS for stage st (K steps kKS st ..) into buffer st % kNst.
    auto issue_stage = [&](int st) {
        lds_u8 *sa = smem + (st % kNst) * kStage;
#pragma unroll
        for (int j = 0; j < S::XLd; ++j) {
            const int q = (wave * S::XLd + j) * S::XLanes + lane;
            if (S::XLanes == kWave || lane < S::XLanes) {
                const int r = q / 16, c = (q % 16) ^ swz16(q / 16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    x_rsrc, (__attribute__((address_space(3))) void *)(sa + (wave * S::XLd + j) * S::XLanes * 16),
                    16, (int)(r * ldx * 2) + st * kXRow + 16 * c, 0, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < S::WLd; ++j) {
            const int q = (wave * S::WLd + j) * S::WLanes + lane;
            if (S::WLanes == kWave || lane < S::WLanes) {
                const int n = q / 4, c = (q % 4) ^ swz4(q / 4);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    w_rsrc,
                    (__attribute__((address_space(3))) void *)(sa + kXBytes + (wave * S::WLd + j) * S::WLanes * 16),
                    16, (int)(n * ldw) + st * kWRow + 16 * c, 0, 0, 0);
            }
        }
    };

    // Scales and zero points of this lane's weight rows for the K steps of
    // stage st (steps past the end repeat the last one; they are not used).
    uint32_t sz_raw[kKS][kWN][2];
    auto load_sz = [&](int st) {
#pragma unroll
        for (int s = 0; s < kKS; ++s) {
            const int kt = min(st * kKS + s, ksteps - 1);
#pragma unroll
            for (int j = 0; j < kWN; ++j) {
                const int n = min(n0 + wave * kTW + j * 32 + l32, N - 1);
                sz_raw[s][j][0] = scales[(int64_t)kt * N + n];
                sz_raw[s][j][1] = zeros[(int64_t)kt * N + n];
            }
        }
    };

    const int x_base = l32 * kXRow;                                    // + i * 32 rows
    const int x_swz = swz16(l32);
    const int w_row = wave * kTW + l32;                                // + j * 32 rows
    const int w_base = kXBytes + w_row * kWRow;
    const int w_swz = swz4(w_row);

    v16f acc[kWM][kWN];
#pragma unroll
    for (int i = 0; i < kWM; ++i)
#pragma unroll
        for (int j = 0; j < kWN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.f;

    // Sub-step v of a stage: K step v / 4, 16-wide slice v % 4 of it.  Lane
    // half h holds k = 8 h .. 8 h + 7 of the slice: x slot 8 (v / 4) + 2 (v % 4)
    // + h of its row, and dword 2 (v % 4) + h of the step's 32 packed bytes.
    const int nstages = (ksteps + kKS - 1) / kKS;
    // One stage of NSUB sub-steps (a full stage, or the single K step of a
    // last stage that K leaves short), as straight-line code.
    auto run_stage = [&](int st, auto nsub_c) {
        constexpr int nsub = decltype(nsub_c)::value;
        // This stage's DMA and scales have landed once each wave has waited
        // for its own; the barrier extends that to the block and retires every
        // read of the other buffer (stage st - 1), which is refilled below.
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        float sc[kKS][kWN], m8s[kKS][kWN], zp[kKS][kWN];
#pragma unroll
        for (int s = 0; s < kKS; ++s)
#pragma unroll
            for (int j = 0; j < kWN; ++j) {
                sc[s][j] = bf16_to_f32(sz_raw[s][j][0]);
                m8s[s][j] = -8.f * sc[s][j];
                zp[s][j] = bf16_to_f32(sz_raw[s][j][1]);
            }
        if (st + 1 < nstages) {
            load_sz(st + 1);
            issue_stage(st + 1);
        }
        const lds_u8 *sa = smem + (st % kNst) * kStage;
        uint32_t pk[kKS][kWN][4];
#pragma unroll
        for (int s = 0; s < nsub / 4; ++s)
#pragma unroll
            for (int j = 0; j < kWN; ++j)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    pk[s][j][u] = *(lds_u32 *)(sa + w_base + j * 32 * kWRow + 16 * ((2 * s + (u >> 1)) ^ w_swz) +
                                               4 * ((2 * u + h) & 3));
        u32x4 xf[2][kWM];
        auto read_x = [&](u32x4 (&f)[kWM], int v) {
            const int slot = (8 * (v / 4) + 2 * (v % 4) + h) ^ x_swz;
#pragma unroll
            for (int i = 0; i < kWM; ++i)
                f[i] = *(lds_u32x4 *)(sa + x_base + i * 32 * kXRow + 16 * slot);
        };
        v8bfv wf[2][kWN];
        auto dequant = [&](v8bfv (&f)[kWN], int v) {
#pragma unroll
            for (int j = 0; j < kWN; ++j)
                f[j] = dequant8(pk[v / 4][j][v % 4], sc[v / 4][j], m8s[v / 4][j], zp[v / 4][j]);
        };
        read_x(xf[0], 0);
        dequant(wf[0], 0);
#pragma unroll
        for (int v = 0; v < nsub; ++v) {
            // One scheduling region per sub-step: the reads and the
            // dequantisation of sub-step v + 1 interleave with the MFMAs of v.
            __builtin_amdgcn_sched_barrier(0);
            if (v + 1 < nsub) {
                read_x(xf[(v + 1) & 1], v + 1);
                dequant(wf[(v + 1) & 1], v + 1);
            }
#pragma unroll
            for (int i = 0; i < kWM; ++i) {
                const v8bfv xb = __builtin_bit_cast(v8bfv, xf[v & 1][i]);
#pragma unroll
                for (int j = 0; j < kWN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[v & 1][j], xb, acc[i][j], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    static_assert(kKS == 2, "a short last stage holds one K step");
    issue_stage(0);
    load_sz(0);
    const int nfull = ksteps / kKS;
    for (int st = 0; st < nfull; ++st)
        run_stage(st, std::integral_constant<int, 4 * kKS>{});
    if (nfull < nstages)
        run_stage(nfull, std::integral_constant<int, 4>{});

    // Epilogue: lane l holds rows m = m0 + 32 i + l32 and, in register group
    // q, columns n = n0w + 32 j + 8 q + 4 h + (0..3).  Each wave stages its
    // 256 x 64 bf16 tile in LDS and writes 128-byte row pieces.
    const int n0w = n0 + wave * kTW;
    __builtin_amdgcn_s_barrier();  // every wave is done with the operand stages
    lds_u8 *wt = smem + wave * (kBM * kPitch);
#pragma unroll
    for (int j = 0; j < kWN; ++j) {
        float bc[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                bc[q][e] = bias ? bf16_to_f32(bias[min(n0w + j * 32 + 8 * q + 4 * h + e, N - 1)]) : 0.f;
#pragma unroll
        for (int i = 0; i < kWM; ++i) {
            const int ml = i * 32 + l32;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x2 pkd = {pack_bf16x2(acc[i][j][4 * q] + bc[q][0], acc[i][j][4 * q + 1] + bc[q][1]),
                                   pack_bf16x2(acc[i][j][4 * q + 2] + bc[q][2], acc[i][j][4 * q + 3] + bc[q][3])};
                *(__attribute__((address_space(3))) u32x2 *)(wt + ml * kPitch + (j * 32 + 8 * q + 4 * h) * 2) = pkd;
            }
        }
    }
    constexpr int kChunks = kTW * 2 / 16;  // 16-byte chunks per staged row
    constexpr int kRows = kWave / kChunks;
#pragma unroll 4
    for (int it = 0; it < kBM / kRows; ++it) {
        const int ml = it * kRows + lane / kChunks;
        const int c = lane % kChunks;
        const u32x4 v = *(lds_u32x4 *)(wt + ml * kPitch + 16 * c);
        const int m = m0 + ml, n = n0w + 8 * c;
        if (m < M && n < N)
            *reinterpret_cast<u32x4 *>(out + (int64_t)m * ldo + n) = v;
    }
}


template <int WM, int WN, int NW>
hipError_t launch_shape(const uint16_t *x, int M, int K, int64_t ldx, const uint8_t *packed, int64_t ldw,
                        const uint16_t *scales, const uint16_t *zeros, int N, const uint16_t *bias,
                        uint16_t *out, int64_t ldo, hipStream_t s)
{
    using S = Shape<WM, WN, NW>;
    auto kern = awq_gemm_kernel<WM, WN, NW>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::Smem);
    if (attr != hipSuccess)
        return attr;
    const int tiles = ((M + S::BM - 1) / S::BM) * ((N + S::BN - 1) / S::BN);
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(NW * kWave), S::Smem, s, x, ldx, M, K, packed, ldw, scales,
                       zeros, N, bias, out, ldo);
    return hipGetLastError();
}

}  // namespace

int launch_awq_gemm(const uint16_t *x, int M, int K, int64_t ldx, const uint8_t *packed, int64_t ldw,
                    const uint16_t *scales, const uint16_t *zeros, int N, const uint16_t *bias,
                    uint16_t *out, int64_t ldo, void *stream)
{
    if (M <= 0)
        return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // 256 x 256 tiles (one wave per SIMD, each dequantised weight fragment
    // reused for 8 row tiles) or 128 x 128 tiles (two blocks per CU).  The
    // time is about the tiles per CU times the time of one tile, and a large
    // tile measured about 3.1 times a small one (four times the work), so the
    // large tiles win unless their last round leaves much of the chip idle:
    // M = 1024, N = 18432 makes 288 large tiles (two rounds, 185 us) or 1152
    // small ones (4.5 per CU, 151 us); M = 4096 makes 1152 large tiles (475 us)
    // or 4608 small ones (550 us).
    constexpr int64_t kCus = 256;
    const int64_t big = ((M + 255) / 256) * (int64_t)((N + 255) / 256);
    const int64_t small = ((M + 127) / 128) * (int64_t)((N + 127) / 128);
    if (31 * ((big + kCus - 1) / kCus) <= 10 * ((small + kCus - 1) / kCus))
        return (int)launch_shape<8, 2, 4>(x, M, K, ldx, packed, ldw, scales, zeros, N, bias, out, ldo, s);
    return (int)launch_shape<4, 1, 4>(x, M, K, ldx, packed, ldw, scales, zeros, N, bias, out, ldo, s);
}

}  // namespace ck
