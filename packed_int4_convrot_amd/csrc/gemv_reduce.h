// Cross-lane helpers shared by the decode GEMV kernels: lane exchanges by
// DPP / ds_swizzle and the transposed reduction of per-row partial sums.
#pragma once
#include "ck_device.h"

namespace ck {

// v from lane (lane ^ MASK), MASK in {1, 2, 4, 8, 16}.
template <int MASK>
__device__ __forceinline__ uint32_t lane_xor_u(uint32_t v)
{
    if constexpr (MASK == 1)
        return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
    else if constexpr (MASK == 2)
        return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
    else if constexpr (MASK == 8)
        return __builtin_amdgcn_update_dpp(0u, v, 0x128, 0xF, 0xF, true);  // row_ror:8 = lane ^ 8
    else
        return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (MASK << 10));
}

// v from a partner lane in another half of its 8-lane group (DPP
// row_half_mirror: lane i <-> 7 - i within each group of 8), so the pair
// differs in bit 2 like lane ^ 4, without the LDS-pipe round trip of
// ds_swizzle.  Enough wherever only the set of pairs across bit 2 matters
// (sums and maxima over the 8 lanes).
__device__ __forceinline__ uint32_t lane_mirror8_u(uint32_t v)
{
    return __builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, true);
}

// v from lane 15 - i of its 16-lane row (DPP row_mirror): pairs across bit 3.
__device__ __forceinline__ uint32_t lane_mirror16_u(uint32_t v)
{
    return __builtin_amdgcn_update_dpp(0u, v, 0x140, 0xF, 0xF, true);
}

template <bool F>
__device__ __forceinline__ uint32_t add32(uint32_t a, uint32_t b)
{
    if constexpr (F)
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    else
        return a + b;
}

// One halving step of the transposed reduction on V values per lane: lanes with
// bit MASK set keep the upper V / 2 rows, the others the lower, and each adds
// its partner's (lane ^ MASK) share of the rows it keeps.
template <int MASK, int V, bool F>
__device__ __forceinline__ void halve_rows(uint32_t *p, int lane)
{
    const bool hi = lane & MASK;
#pragma unroll
    for (int j = 0; j < V / 2; ++j) {
        const uint32_t keep = hi ? p[j + V / 2] : p[j];
        const uint32_t send = hi ? p[j] : p[j + V / 2];
        p[j] = add32<F>(keep, lane_xor_u<MASK>(send));
    }
}

// Sum of p[r] over the 64 lanes for r < R (R = 8, 16 or 32).  Afterwards lane
// l holds the total of row l >> (6 - log2 R) (every lane of that row group
// holds the same value).
template <int R, bool F>
__device__ __forceinline__ uint32_t transposed_row_sum(uint32_t (&p)[R], int lane)
{
    static_assert(R == 8 || R == 16 || R == 32, "R");
#pragma unroll
    for (int j = 0; j < R / 2; ++j) {  // lane ^ 32: upper half keeps rows + R/2
        const auto s = __builtin_amdgcn_permlane32_swap(p[j], p[j + R / 2], false, false);
        p[j] = add32<F>(s[0], s[1]);
    }
#pragma unroll
    for (int j = 0; j < R / 4; ++j) {  // lane ^ 16: odd 16-lane rows keep rows + R/4
        const auto s = __builtin_amdgcn_permlane16_swap(p[j], p[j + R / 4], false, false);
        p[j] = add32<F>(s[0], s[1]);
    }
    halve_rows<8, R / 4, F>(p, lane);                       // R / 8 rows left
    if constexpr (R >= 16) halve_rows<4, R / 8, F>(p, lane);
    if constexpr (R >= 32) halve_rows<2, R / 16, F>(p, lane);
    uint32_t v = p[0];
    if constexpr (R == 8) v = add32<F>(v, lane_mirror8_u(v));
    if constexpr (R <= 16) v = add32<F>(v, lane_xor_u<2>(v));
    v = add32<F>(v, lane_xor_u<1>(v));
    return v;
}

// Transposed lane reduction of part[M0 .. M0 + B)[R] (B = 4, 2 or 1 rows, as
// many as fit in 32 values), then the rest; the owner lanes store the wave's
// sums to red[r][m].
template <int M, int R, bool F, int M0>
__device__ __forceinline__ void reduce_rows(uint32_t (&part)[M][R], int lane, uint32_t (&red)[R][M])
{
    if constexpr (M0 < M) {
        constexpr int left = M - M0;
        constexpr int B = (R == 8 && left >= 4) ? 4 : (R <= 16 && left >= 2 && 2 * R <= 32) ? 2 : 1;
        constexpr int V = B * R;
        constexpr int kShift = V == 32 ? 1 : V == 16 ? 2 : 3;
        uint32_t flat[V];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int r = 0; r < R; ++r)
                flat[b * R + r] = part[M0 + b][r];
        const uint32_t t = transposed_row_sum<V, F>(flat, lane);
        const int v = lane >> kShift;  // b * R + r
        if ((lane & ((1 << kShift) - 1)) == 0)
            red[v % R][M0 + v / R] = t;
        reduce_rows<M, R, F, M0 + B>(part, lane, red);
    }
}

}  // namespace ck
