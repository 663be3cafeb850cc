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

template <bool F>
__device__ __forceinline__ uint32_t add32(uint32_t a, uint32_t b)
{
    if constexpr (F)
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    else
        return a + b;
}

// Sum of p[r] over the 64 lanes for r < R (R = 8 or 16).  Afterwards lane l
// holds the total of row l >> (6 - log2 R) (every lane of that row group
// holds the same value).
template <int R, bool F>
__device__ __forceinline__ uint32_t transposed_row_sum(uint32_t (&p)[R], int lane)
{
    static_assert(R == 8 || R == 16, "R");
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
    const bool b3 = lane & 8;
#pragma unroll
    for (int j = 0; j < R / 8; ++j) {  // lane ^ 8
        const uint32_t keep = b3 ? p[j + R / 8] : p[j];
        const uint32_t send = b3 ? p[j] : p[j + R / 8];
        p[j] = add32<F>(keep, lane_xor_u<8>(send));
    }
    uint32_t v = p[0];
    if constexpr (R == 16) {  // lane ^ 4 (two rows left)
        const bool b2 = lane & 4;
        const uint32_t keep = b2 ? p[1] : p[0];
        const uint32_t send = b2 ? p[0] : p[1];
        v = add32<F>(keep, lane_xor_u<4>(send));
    } else {
        v = add32<F>(v, lane_xor_u<4>(v));
    }
    v = add32<F>(v, lane_xor_u<2>(v));
    v = add32<F>(v, lane_xor_u<1>(v));
    return v;
}

}  // namespace ck
