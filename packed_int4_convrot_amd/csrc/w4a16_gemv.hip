// AWQ W4A16 GEMV: bf16 activations times packed uint4 weights with per-group
// scales and zero points, W[n,k] = (q - 8) * s[k/64, n] + z[k/64, n]
// ("comfy_kitchen/tensor/awq_w4a16.py", module docstring and dequantize()).
// The page's eager path materialises W in bf16 and calls a matmul; here W is
// never built.  Per 64-wide group g and output column n:
//   y += s[g,n] * sum_k x_k (q_k - 8) + z[g,n] * X_g,   X_g = sum_k x_k
//      = s[g,n] * P_g + (z[g,n] - 136 s[g,n]) * X_g,     P_g = sum_k x_k (128 + q_k)
// P_g runs on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate): the
// weight operand is bf16(128 + q), which is the exact bit pattern 0x4300 | q,
// built from the packed bytes with one byte permute per two weights.  X_g is
// computed once per group by the same instruction with an all-ones operand.
//
// Operand layouts (16 x 32 x 16): A lane l holds 8 bf16 of row m = l % 16,
// k-block l / 16; B lane l holds 8 bf16 of column n = l % 16, k-block l / 16;
// D lane l holds D[4*(l/16) + i][l % 16].  The weight decode yields k order
// [0,2,4,6,1,3,5,7] inside each 8-wide block; the activations are permuted to
// match when they are loaded (once per wave).
#include "ck_device.h"
#include "launch.h"

namespace ck {
namespace {

constexpr int kMaxWaves = 8;  // 512 threads: up to 256 VGPRs per lane
constexpr int kGpw = 8;  // K-groups per wave held in registers

__device__ __forceinline__ v8bf as_v8bf(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    v4i v{(int)a, (int)b, (int)c, (int)d};
    return __builtin_bit_cast(v8bf, v);
}

// 8 bf16 (four dwords, natural k order) -> k order [0,2,4,6,1,3,5,7].
__device__ __forceinline__ v8bf x_perm8(uint4 w)
{
    return as_v8bf(perm(w.y, w.x, 0x05040100u), perm(w.w, w.z, 0x05040100u),
                   perm(w.y, w.x, 0x07060302u), perm(w.w, w.z, 0x07060302u));
}

// One packed dword (k = 0..7) -> bf16(128 + q) in k order [0,2,4,6,1,3,5,7].
__device__ __forceinline__ v8bf w_bf16_plus128(uint32_t d)
{
    const uint32_t e = d & 0x0f0f0f0fu;
    const uint32_t o = (d >> 4) & 0x0f0f0f0fu;
    const uint32_t m = 0x43434343u;
    return as_v8bf(perm(m, e, 0x04010400u), perm(m, e, 0x04030402u), perm(m, o, 0x04010400u),
                   perm(m, o, 0x04030402u));
}

__global__ __launch_bounds__(kMaxWaves * kWave) void w4a16_gemv_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int M, int K, const uint8_t *__restrict__ packed,
    int64_t ldw, const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros, int N,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ out, int64_t ldo, int gpw)
{
    extern __shared__ float red[];  // [KS][64][4]
    const int ks = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int ng = K / 64;
    const int g0 = wave * gpw;
    const int cnt = max(0, min(gpw, ng - g0));
    const int col = lane % 16, kb = lane / 16;

    // All activation loads and the first tile's weight loads are issued
    // before any is used (clamped addresses; out-of-range values zeroed).
    const int ntiles = N / 16;
    int tile = blockIdx.x;
    u32x4 raw[kGpw][2];
#pragma unroll
    for (int j = 0; j < kGpw; ++j)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int m = min(col, M - 1);
            const int g = min(g0 + j, ng - 1);
            raw[j][s] = *reinterpret_cast<const u32x4 *>(x + (int64_t)m * ldx + 64 * g + 16 * kb + 8 * s);
        }
    u32x2 bw[kGpw];
    uint16_t sv[kGpw], zv[kGpw];
    auto load_tile = [&](int t) {
        const int n = t * 16 + col;
        const uint8_t *wrow = packed + (int64_t)n * ldw + 8 * kb + 32 * g0;
#pragma unroll
        for (int j = 0; j < kGpw; ++j)
            if (j < cnt) {
                bw[j] = load_nt8(wrow + 32 * j);
                sv[j] = scales[(int64_t)(g0 + j) * N + n];
                zv[j] = zeros[(int64_t)(g0 + j) * N + n];
            }
    };
    if (tile < ntiles)
        load_tile(tile);

    // Activation operands (two 32-wide halves per group) and the group sums X.
    v8bf a[kGpw][2];
    v4f xs[kGpw];
    const v8bf ones = as_v8bf(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
#pragma unroll
    for (int j = 0; j < kGpw; ++j) {
        const bool live = j < cnt && col < M;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint4 w = make_uint4(raw[j][s][0], raw[j][s][1], raw[j][s][2], raw[j][s][3]);
            a[j][s] = live ? x_perm8(w) : as_v8bf(0u, 0u, 0u, 0u);
        }
        v4f z{0.f, 0.f, 0.f, 0.f};
        z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j][0], ones, z, 0, 0, 0);
        xs[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j][1], ones, z, 0, 0, 0);
    }

    for (; tile < ntiles; tile += gridDim.x) {
        float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kGpw; ++j)
            if (j < cnt) {
                v4f p{0.f, 0.f, 0.f, 0.f};
                p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j][0], w_bf16_plus128(bw[j][0]), p, 0, 0, 0);
                p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j][1], w_bf16_plus128(bw[j][1]), p, 0, 0, 0);
                const float s = bf16_to_f32(sv[j]);
                const float c = __builtin_fmaf(-136.f, s, bf16_to_f32(zv[j]));
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    y[i] = __builtin_fmaf(s, p[i], __builtin_fmaf(c, xs[j][i], y[i]));
            }
        if (tile + (int)gridDim.x < ntiles)
            load_tile(tile + gridDim.x);
        *reinterpret_cast<float4 *>(red + (wave * kWave + lane) * 4) = make_float4(y[0], y[1], y[2], y[3]);
        __syncthreads();
        for (int e = threadIdx.x; e < kWave * 4; e += blockDim.x) {
            const int l = e / 4, i = e % 4;
            const int m = 4 * (l / 16) + i;
            const int nn = tile * 16 + l % 16;
            if (m < M) {
                float v = 0.f;
                for (int w = 0; w < ks; ++w)
                    v += red[w * kWave * 4 + e];
                if (bias)
                    v += bf16_to_f32(bias[nn]);
                out[(int64_t)m * ldo + nn] = f32_to_bf16(v);
            }
        }
        __syncthreads();
    }
}

}  // namespace

bool w4a16_supports(int64_t K) { return (K / 64 + kGpw - 1) / kGpw <= kMaxWaves; }

int launch_w4a16_gemv(const uint16_t *x, int M, int K, int64_t ldx, const uint8_t *packed,
                      int64_t ldw, const uint16_t *scales, const uint16_t *zeros, int N,
                      const uint16_t *bias, uint16_t *out, int64_t ldo, void *stream)
{
    if (M <= 0)
        return 0;
    const int ng = K / 64;
    int ks = (ng + kGpw - 1) / kGpw;
    if (ks < 4)
        ks = ng < 4 ? ng : 4;
    const int gpw = (ng + ks - 1) / ks;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const size_t smem = (size_t)ks * kWave * 4 * sizeof(float);
    hipLaunchKernelGGL(w4a16_gemv_kernel, dim3(N / 16), dim3(ks * kWave), smem, s, x, ldx, M, K,
                       packed, ldw, scales, zeros, N, bias, out, ldo, gpw);
    return (int)hipGetLastError();
}

}  // namespace ck
