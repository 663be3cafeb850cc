// AWQ W4A16 GEMV: bf16 activations times packed uint4 weights with per-group
// scales and zero points, W[n,k] = (q - 8) * s[k/64, n] + z[k/64, n]
// ("comfy_kitchen/tensor/awq_w4a16.py", module docstring and dequantize()).
// The page's eager path materialises W in bf16 and calls a matmul; here W is
// never built.  For a 64-wide group g and output column n,
//   sum_k x_k W[n,k] = s[g,n] * P + (z[g,n] - 136 s[g,n]) * X,
//   P = sum_k x_k (128 + q_k),   X = sum_k x_k,
// and both sums split over any partition of the group's columns.
//
// The product streams the weights once, so the kernel is laid out for HBM:
//   * lanes own KL = 32 or 16 columns: wave w of a block owns columns k in
//     [64 KL w, 64 KL (w + 1)); lane l owns the KL columns from 64 KL w + KL l
//     (half or a quarter of a group), i.e. KL / 2 packed bytes of every weight
//     row, so each load instruction reads 1 KiB or 512 bytes of one row.  The
//     launcher takes the width that leaves fewer lanes past K (K = 3072: three
//     waves of 16-column lanes, all busy, instead of two waves of 32-column
//     lanes with half of the second idle);
//   * a block owns 8 consecutive weight rows n0 .. n0 + 7; a lane loads its
//     activations, then the 8 scales and 8 zero points of its group for those
//     rows (one 16-byte load each, N contiguous), then the 8 weight rows.
//     Loads retire in issue order, so the activation work waits only for the
//     activations while the weights stream in;
//   * bf16(128 + q) is the bit pattern 0x4300 | q, so one byte permute against
//     a 0x43 constant turns two nibbles into a bf16 pair; v_dot2_f32_bf16
//     multiplies it with the matching activation pair and accumulates in fp32
//     (the products are exact: 8-bit by 8-bit significands).  Low nibbles are
//     even k and high nibbles odd k, so the activations are paired to match
//     ((x0,x2), (x4,x6), (x1,x3), (x5,x7) per 8 columns) once per lane;
//   * the per-lane partials s P + (z - 136 s) X of the 8 rows are summed by
//     the transposed lane reduction, then across waves through LDS in a fixed
//     order, and the bias is added once.
#include "ck_device.h"
#include "gemv_reduce.h"
#include "launch.h"

namespace ck {
namespace {

constexpr int kMaxWaves = 8;  // K <= 16384
constexpr int kRows = 8;      // weight rows per block

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), c, false);
}

template <int M, int KL>
__global__ __launch_bounds__(kMaxWaves * kWave) void w4a16_gemv_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int K, const uint8_t *__restrict__ packed, int64_t ldw,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros, int N,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ out, int64_t ldo)
{
    constexpr int R = kRows;
    constexpr int NQ = KL / 8;  // 8-column units (weight dwords) per lane
    static_assert(KL == 32 || KL == 16, "lane width");
    __shared__ uint32_t s_red[kMaxWaves][R][M];

    const int nw = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int n0 = xcd_block(blockIdx.x, gridDim.x) * R;
    const int kbase = kWave * KL * wave + KL * lane;
    const bool active = kbase < K;
    const int kc = active ? kbase : K - KL;  // clamped: every address stays inside the row
    const int64_t g = kc / 64;

    // Activation rows are handled in passes of up to 4 against the weight
    // registers, which bounds the registers held for activation pairs.
    constexpr int MC = M < 4 ? M : 4;
    constexpr int NPASS = (M + MC - 1) / MC;

    // 1. Loads: the first pass's activations, then the group's scales and zero
    //    points, then the weights.
    u32x4 xr[MC][NQ];
    auto load_x = [&](int mb) {
#pragma unroll
        for (int m = 0; m < MC; ++m)
#pragma unroll
            for (int c = 0; c < NQ; ++c)
                xr[m][c] = mb + m < M ? *reinterpret_cast<const u32x4 *>(x + (int64_t)(mb + m) * ldx + kc + 8 * c)
                                      : u32x4{0u, 0u, 0u, 0u};
    };
    load_x(0);
    const u32x4 sv = *reinterpret_cast<const u32x4 *>(scales + g * N + n0);
    const u32x4 zv = *reinterpret_cast<const u32x4 *>(zeros + g * N + n0);
    uint32_t wv[R][NQ];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint8_t *src = packed + (int64_t)(n0 + r) * ldw + kc / 2;
        if constexpr (KL == 32) {
            const u32x4 t = load_nt16(src);
            wv[r][0] = t[0], wv[r][1] = t[1], wv[r][2] = t[2], wv[r][3] = t[3];
        } else {
            const u32x2 t = load_nt8(src);
            wv[r][0] = t[0], wv[r][1] = t[1];
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads in this order

    const int row = lane >> 3;
    const bool owner = (lane & 7) == 0;
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        uint32_t part[MC][R];
        const int mb = pass * MC;
        if (pass > 0) {
            __builtin_amdgcn_sched_barrier(0);  // passes run one after another
            load_x(mb);
        }
        // 2. Activation pairs in the nibble order, and the lane's activation sums.
        uint32_t xp[MC][4 * NQ];
        float xs[MC];
#pragma unroll
        for (int m = 0; m < MC; ++m) {
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const u32x4 w = xr[m][i];  // bf16 of columns kc + 8 i .. + 7
                xp[m][4 * i + 0] = active ? perm(w[1], w[0], 0x05040100u) : 0u;  // (x0, x2)
                xp[m][4 * i + 1] = active ? perm(w[3], w[2], 0x05040100u) : 0u;  // (x4, x6)
                xp[m][4 * i + 2] = active ? perm(w[1], w[0], 0x07060302u) : 0u;  // (x1, x3)
                xp[m][4 * i + 3] = active ? perm(w[3], w[2], 0x07060302u) : 0u;  // (x5, x7)
            }
            float t = 0.f;
#pragma unroll
            for (int j = 0; j < 4 * NQ; ++j)
                t = dot2(xp[m][j], 0x3F803F80u, t);  // bf16 (1, 1)
            xs[m] = t;
        }

        // 3. Per weight row: P over the lane's 32 columns, then the group terms.
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float acc[MC];
#pragma unroll
            for (int m = 0; m < MC; ++m)
                acc[m] = 0.f;
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const uint32_t lo = wv[r][i] & 0x0f0f0f0fu;         // q of k = 0, 2, 4, 6
                const uint32_t hi = (wv[r][i] >> 4) & 0x0f0f0f0fu;  // q of k = 1, 3, 5, 7
                const uint32_t w0 = perm(0x43434343u, lo, 0x04010400u);  // bf16(128+q) of (k0, k2)
                const uint32_t w1 = perm(0x43434343u, lo, 0x04030402u);  // (k4, k6)
                const uint32_t w2 = perm(0x43434343u, hi, 0x04010400u);  // (k1, k3)
                const uint32_t w3 = perm(0x43434343u, hi, 0x04030402u);  // (k5, k7)
#pragma unroll
                for (int m = 0; m < MC; ++m) {
                    acc[m] = dot2(w0, xp[m][4 * i + 0], acc[m]);
                    acc[m] = dot2(w1, xp[m][4 * i + 1], acc[m]);
                    acc[m] = dot2(w2, xp[m][4 * i + 2], acc[m]);
                    acc[m] = dot2(w3, xp[m][4 * i + 3], acc[m]);
                }
            }
            const uint32_t sw = sv[r / 2], zw = zv[r / 2];
            const float s = __uint_as_float((r & 1) ? (sw & 0xffff0000u) : (sw << 16));
            const float z = __uint_as_float((r & 1) ? (zw & 0xffff0000u) : (zw << 16));
            const float zc = __builtin_fmaf(-136.f, s, z);
#pragma unroll
            for (int m = 0; m < MC; ++m)
                part[m][r] = __float_as_uint(__builtin_fmaf(s, acc[m], zc * xs[m]));
            if constexpr (M > 1)
                __builtin_amdgcn_sched_barrier(0);  // one row's decode live at a time
        }
        // 4. Sum the pass's rows over the lanes of the wave (the waves are summed
        //    below, in a fixed order); done per pass, so that only one pass's
        //    partials are live.
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            if (mb + m < M) {
                const uint32_t t = transposed_row_sum<R, true>(part[m], lane);
                if (owner)
                    s_red[wave][row][mb + m] = t;
            }
        }
    }
    __syncthreads();
    if (threadIdx.x < R * M) {
        const int r = threadIdx.x / M, m = threadIdx.x % M;
        const int n = n0 + r;
        float y = __uint_as_float(s_red[0][r][m]);
        for (int w = 1; w < nw; ++w)
            y += __uint_as_float(s_red[w][r][m]);
        if (bias)
            y += bf16_to_f32(bias[n]);
        out[(int64_t)m * ldo + n] = f32_to_bf16(y);
    }
}

template <int M>
hipError_t launch_m(const uint16_t *x, int64_t ldx, int K, const uint8_t *packed, int64_t ldw,
                    const uint16_t *scales, const uint16_t *zeros, int N, const uint16_t *bias,
                    uint16_t *out, int64_t ldo, hipStream_t s)
{
    // Lane width: 16 columns where that leaves fewer lanes past K and the block
    // stays within kMaxWaves waves, else 32.
    const int w32 = (K + 2047) / 2048, w16 = (K + 1023) / 1024;
    const bool narrow = w16 <= kMaxWaves && 1024 * w16 - K < 2048 * w32 - K;
    const dim3 grid((unsigned)(N / kRows));
    const dim3 block((unsigned)(kWave * (narrow ? w16 : w32)));
    if (narrow)
        hipLaunchKernelGGL((w4a16_gemv_kernel<M, 16>), grid, block, 0, s, x, ldx, K, packed, ldw, scales, zeros,
                           N, bias, out, ldo);
    else
        hipLaunchKernelGGL((w4a16_gemv_kernel<M, 32>), grid, block, 0, s, x, ldx, K, packed, ldw, scales, zeros,
                           N, bias, out, ldo);
    return hipGetLastError();
}

}  // namespace

int launch_w4a16_gemv(const uint16_t *x, int M, int K, int64_t ldx, const uint8_t *packed,
                      int64_t ldw, const uint16_t *scales, const uint16_t *zeros, int N,
                      const uint16_t *bias, uint16_t *out, int64_t ldo, void *stream)
{
    if (M <= 0)
        return 0;
    if (!w4a16_supports(K) || K % 64 != 0 || N % kRows != 0)
        return (int)hipErrorInvalidValue;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    switch (M) {
    case 1: e = launch_m<1>(x, ldx, K, packed, ldw, scales, zeros, N, bias, out, ldo, s); break;
    case 2: e = launch_m<2>(x, ldx, K, packed, ldw, scales, zeros, N, bias, out, ldo, s); break;
    case 3: e = launch_m<3>(x, ldx, K, packed, ldw, scales, zeros, N, bias, out, ldo, s); break;
    case 4: e = launch_m<4>(x, ldx, K, packed, ldw, scales, zeros, N, bias, out, ldo, s); break;
    case 5: e = launch_m<5>(x, ldx, K, packed, ldw, scales, zeros, N, bias, out, ldo, s); break;
    case 6: e = launch_m<6>(x, ldx, K, packed, ldw, scales, zeros, N, bias, out, ldo, s); break;
    case 7: e = launch_m<7>(x, ldx, K, packed, ldw, scales, zeros, N, bias, out, ldo, s); break;
    case 8: e = launch_m<8>(x, ldx, K, packed, ldw, scales, zeros, N, bias, out, ldo, s); break;
    default: e = hipErrorInvalidValue; break;
    }
    return (int)e;
}

}  // namespace ck
