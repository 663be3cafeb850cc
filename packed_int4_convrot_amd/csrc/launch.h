// Internal launch interface between the C ABI (ck_api.cpp) and the kernels.
// Every function assumes its arguments were validated by the caller and
// returns the hipError_t of the launch as an int (0 = success).
#pragma once

#include <stdint.h>

namespace ck {

int launch_rotate_quant(const uint16_t *x, int64_t M, int K, int64_t ldx, int G, int qmax,
                        int8_t *codes, int64_t ldq, float *row_scales, float *xr, int64_t ldr,
                        bool packed4, void *stream);

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
// G != 0 (M = 1) it rotates and quantises the bf16 row x itself (fused linear); with
// G == 0 it reads given codes and row_scales.  acc_out != nullptr (G == 0
// only) selects the int32 test epilogue.
int launch_w4_gemv(const uint16_t *x, int64_t ldx, int G, int qmax, const int8_t *codes, int64_t ldq,
                   const float *row_scales, int M, int K, const uint8_t *packed, int64_t ldw,
                   const uint16_t *w_scales, bool per_group, int N, const uint16_t *bias, float x_scale,
                   uint16_t *out, int64_t ldo, int32_t *acc_out, int64_t lda, void *stream);
bool w4_gemv_supports(int64_t M, int64_t K);
bool w4_gemv_fused_supports(int64_t M, int64_t K);  // G != 0 form

// Skinny path: M <= 64, weights streamed once, activations held in registers.
// acc_out != nullptr selects the int32 test epilogue.
int launch_w4_skinny(const int8_t *codes, int64_t ldq, const float *row_scales, int M, int K,
                     const uint8_t *packed, int64_t ldw, const uint16_t *w_scales,
                     bool per_group, int N, const uint16_t *bias, float x_scale,
                     uint16_t *out, int64_t ldo, int32_t *acc_out, int64_t lda, void *stream);
bool w4_skinny_supports(int64_t M, int64_t K);

// Tiled MFMA GEMM for larger M.
int launch_w4_gemm(const int8_t *codes, int64_t ldq, const float *row_scales, int M, int K,
                   const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, bool per_group,
                   int N, const uint16_t *bias, float x_scale, uint16_t *out, int64_t ldo,
                   int32_t *acc_out, int64_t lda, bool a4, void *stream);

int launch_w4a16_gemv(const uint16_t *x, int M, int K, int64_t ldx, const uint8_t *packed,
                      int64_t ldw, const uint16_t *scales, const uint16_t *zeros, int N,
                      const uint16_t *bias, uint16_t *out, int64_t ldo, void *stream);
bool w4a16_supports(int64_t K);

}  // namespace ck
