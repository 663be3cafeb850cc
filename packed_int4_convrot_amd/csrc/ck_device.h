// Device-side helpers shared by the gfx950 kernels of libck.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ck {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Streaming (non-temporal) global loads for data read exactly once.
__device__ __forceinline__ u32x4 load_nt16(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x2 load_nt8(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}

// s_waitcnt vmcnt(0), the other counters untouched: this wave's vector memory
// loads (global_load_lds DMA included) have landed.
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroups are dealt to the 8 XCDs (each with its own L2) round-robin by
// index.  This renumbering gives every XCD a contiguous run of logical
// blocks, so neighbouring blocks that share cache lines (weight-scale rows,
// activation tiles) hit in the same L2.  A bijection on [0, nblocks).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_block(int b, int nblocks)
{
    const int xcd = b % kXcds, local = b / kXcds;
    const int per = nblocks / kXcds, rem = nblocks % kXcds;
    return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Per-channel scale epilogue of every W4 matmul kernel: acc * (s_w * r) + b,
// r = row scale * input scale, b = bias or 0, with one rounding for s_w * r and
// one for the fused multiply-add.  With one formula in every kernel an output
// row has the same bits whichever kernel, and so whichever batch size, computed
// it.  acc is the exact integer dot product; a kernel that holds 2^k times it
// passes s_w * 2^-k (the same products, as scaling by 2^k is exact).
__device__ __forceinline__ float epilogue_channel(float acc, float sw, float r, float b)
{
    return __builtin_fmaf(acc, sw * r, b);
}

// fp32 -> bf16 bit pattern, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Two fp32 -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    const v2bf p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

// Byte permute of the 8 bytes {hi:lo}: selector byte values 0..3 pick bytes of
// `lo`, 4..7 bytes of `hi`, 0x0c gives 0x00.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Packed-uint4 decode used by every int8 MFMA kernel.
// One packed dword holds 8 codes: byte j = (code of k=2j) | (code of k=2j+1) << 4.
// Flipping bit 3 of every nibble turns the code q into the 4-bit two's
// complement of q - 8; moving that nibble into the high half of a byte gives
// the int8 value 16 * (q - 8).  The result is two dwords of int8 lanes:
//   lo: k = 0, 2, 4, 6     hi: k = 1, 3, 5, 7   (each value is 16 * (q - 8))
// so an int32 MFMA accumulates exactly 16x the true sum (|sum| stays far below
// 2^31 for K <= 65536).  Operands on the other side are permuted to the same k
// order by act_perm16().
__device__ __forceinline__ void w4_decode_x16(uint32_t d, uint32_t &lo, uint32_t &hi)
{
    // Only bit 3 of each nibble is flipped where it survives the mask, so the
    // flip and the mask fold into one v_bitop3 per dword half.
    lo = ((d << 4) ^ 0x80808080u) & 0xf0f0f0f0u;
    hi = (d ^ 0x80808080u) & 0xf0f0f0f0u;
}

// Reorder 16 consecutive int8 values k = 0..15 (four dwords) into the order
// produced by w4_decode_x16 on two packed dwords:
//   [0,2,4,6] [1,3,5,7] [8,10,12,14] [9,11,13,15]
__device__ __forceinline__ v4i act_perm16(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3)
{
    v4i r;
    r[0] = (int)perm(w1, w0, 0x06040200u);
    r[1] = (int)perm(w1, w0, 0x07050301u);
    r[2] = (int)perm(w3, w2, 0x06040200u);
    r[3] = (int)perm(w3, w2, 0x07050301u);
    return r;
}

// Signed 4-bit activation codes packed like the weights (two's complement
// nibbles, low nibble = even k) become 16 * code in the same k order as
// w4_operand_x16, so no reordering is needed on either side.
__device__ __forceinline__ v4i a4_operand_x16(uint32_t d0, uint32_t d1)
{
    v4i r;
    r[0] = (int)((d0 << 4) & 0xf0f0f0f0u);
    r[1] = (int)(d0 & 0xf0f0f0f0u);
    r[2] = (int)((d1 << 4) & 0xf0f0f0f0u);
    r[3] = (int)(d1 & 0xf0f0f0f0u);
    return r;
}

__device__ __forceinline__ v4i w4_operand_x16(uint32_t d0, uint32_t d1)
{
    uint32_t l0, h0, l1, h1;
    w4_decode_x16(d0, l0, h0);
    w4_decode_x16(d1, l1, h1);
    v4i r;
    r[0] = (int)l0;
    r[1] = (int)h0;
    r[2] = (int)l1;
    r[3] = (int)h1;
    return r;
}

}  // namespace ck
