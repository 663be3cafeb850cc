// Internal launch interface between the C ABI (ck_api.cpp) and the kernels.
// Every function assumes its arguments were validated by the caller and
// returns the hipError_t of the launch as an int (0 = success).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ck {

// Layouts of the activation codes written by rotate-quant.
//   kRowMajor: int8 [M, ldq], one code per byte.
//   kPacked4:  W4A4 codes two per byte (4-bit two's complement, column 2j in
//              the low nibble), [M, ldq] bytes.
//   kTiled16:  int8 codes in the operand order of the few-row MFMA kernel:
//              rows in tiles of 16, each tile K/64 blocks of 1 KiB (one per
//              64-column group g); inside a block, the 16 bytes at
//              16 * (16 * kb + r) hold row r of the tile, columns
//              64 g + 16 kb .. + 15 in the order [0,2,4,6, 1,3,5,7, 8,10,12,14,
//              9,11,13,15] (the order of the nibble decode).  Tile t starts at
//              byte 16 * K * t; rows past M in the last tile are not written.
enum class CodesLayout { kRowMajor, kPacked4, kTiled16 };

int launch_rotate_quant(const uint16_t *x, int64_t M, int K, int64_t ldx, int G, int qmax,
                        int8_t *codes, int64_t ldq, float *row_scales, float *xr, int64_t ldr,
                        CodesLayout layout, void *stream);

// AWQ W4A16 prefill GEMM: out = x . W^T (+ bias), W rebuilt in bf16 as the
// page's dequantize() does; Gw = 64 scales and zero points [K/64, N].
int launch_awq_gemm(const uint16_t *x, int M, int K, int64_t ldx, const uint8_t *packed, int64_t ldw,
                    const uint16_t *scales, const uint16_t *zeros, int N, const uint16_t *bias,
                    uint16_t *out, int64_t ldo, void *stream);

// Offline weight producer: rotate N bf16 weight rows of K columns by H_G,
// quantise to codes in [-7, 7] with bf16 scales per row (per_group false) or
// per 64-column group ([K/64, N]), and pack q = code + 8 two per byte.
int launch_quantize_weights(const uint16_t *w, int64_t N, int K, int64_t ldw_in, int G, bool per_group,
                            uint8_t *packed, int64_t ldp, uint16_t *scales, void *stream);

// Decode GEMV for 1 <= M <= 8 (VALU dot4, 1 KiB coalesced weight rows).  With
// G != 0 (M <= 2) it rotates and quantises the bf16 rows x itself (fused linear); with
// G == 0 it reads given codes and row_scales.  acc_out != nullptr (G == 0
// only) selects the int32 test epilogue.
int launch_w4_gemv(const uint16_t *x, int64_t ldx, int G, int qmax, const int8_t *codes, int64_t ldq,
                   const float *row_scales, int M, int K, const uint8_t *packed, int64_t ldw,
                   const uint16_t *w_scales, bool per_group, int N, const uint16_t *bias, float x_scale,
                   uint16_t *out, int64_t ldo, int32_t *acc_out, int64_t lda, void *stream);
// The decode GEMV: 1 <= M <= 8 activation rows, one wave per 2048 columns of K,
// at most 8 waves; the fused rotate-quant form takes one or two rows.
constexpr int kGemvMaxWaves = 8;
constexpr int kGemvMaxM = 8;
constexpr int kGemvMaxFusedRows = 2;
inline bool w4_gemv_supports(int64_t M, int64_t K)
{
    return M >= 1 && M <= kGemvMaxM && K <= 2048 * kGemvMaxWaves;
}
inline bool w4_gemv_fused_supports(int64_t M, int64_t K) { return w4_gemv_supports(M, K) && M <= kGemvMaxFusedRows; }

// Skinny path: M <= 64, weights streamed once, activations held in registers.
// acc_out != nullptr selects the int32 test epilogue.
// codes: row-major int8 [M, ldq], or (tiled, ldq ignored) the kTiled16 layout.
int launch_w4_skinny(const int8_t *codes, int64_t ldq, bool tiled, const float *row_scales, int M,
                     int K, const uint8_t *packed, int64_t ldw, const uint16_t *w_scales,
                     bool per_group, int N, const uint16_t *bias, float x_scale,
                     uint16_t *out, int64_t ldo, int32_t *acc_out, int64_t lda, void *stream);
// Shape of the few-row kernel: MT = ceil(M / 16) m-tiles; GPW groups per wave,
// chosen so that the register copy of the activations (GPW * MT * 4 VGPRs)
// stays at most 128; KS = ceil(K / 64 / GPW) <= 8 waves.
constexpr int kSkinnyMaxWaves = 8;
struct SkinnyShape {
    int mt, ks, gpw;
};
inline bool skinny_shape(int64_t M, int64_t K, SkinnyShape &s)
{
    if (M < 1 || M > 64)
        return false;
    const int ng = (int)(K / 64);
    s.mt = M <= 16 ? 1 : M <= 32 ? 2 : 4;
    s.gpw = s.mt == 1 ? 16 : s.mt == 2 ? (ng <= 8 * kSkinnyMaxWaves ? 8 : 16) : 8;
    s.ks = (ng + s.gpw - 1) / s.gpw;
    return s.ks >= 1 && s.ks <= kSkinnyMaxWaves;
}
inline bool w4_skinny_supports(int64_t M, int64_t K)
{
    SkinnyShape s;
    return skinny_shape(M, K, s);
}

// Tiled MFMA GEMM for larger M.
int launch_w4_gemm(const int8_t *codes, int64_t ldq, const float *row_scales, int M, int K,
                   const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, bool per_group,
                   int N, const uint16_t *bias, float x_scale, uint16_t *out, int64_t ldo,
                   int32_t *acc_out, int64_t lda, bool a4, void *stream);

int launch_w4a16_gemv(const uint16_t *x, int M, int K, int64_t ldx, const uint8_t *packed,
                      int64_t ldw, const uint16_t *scales, const uint16_t *zeros, int N,
                      const uint16_t *bias, uint16_t *out, int64_t ldo, void *stream);
inline bool w4a16_supports(int64_t K) { return K >= 64 && K <= 2048 * kGemvMaxWaves; }

// Library-owned device scratch of the allocation-free linear (static_scratch.hip):
// 64 MiB of codes plus 64 KiB of row scales, so that 8192 rows of K = 16384 (or
// 16384 rows of K = 8192) packed two codes per byte fit.
constexpr size_t kStaticScratchBytes = (size_t(64) << 20) + (size_t(64) << 10);
// Its size in bytes, and its address on the current device, which must be the
// device of `stream` (NULL: the null stream); looked up once per device.  Returns
// 0 or a hipError_t.
size_t static_scratch_bytes();
int static_scratch(void *stream, void **ptr);

}  // namespace ck
