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

// Decode GEMV for 1 <= M <= 8 (VALU dot4, 1 KiB coalesced weight rows) on
// given codes and row_scales.  acc_out != nullptr selects the int32 test
// epilogue.
int launch_w4_gemv(const int8_t *codes, int64_t ldq, const float *row_scales, int M, int K,
                   const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, bool per_group, int N,
                   const uint16_t *bias, float x_scale, uint16_t *out, int64_t ldo, int32_t *acc_out,
                   int64_t lda, void *stream);
// The decode GEMV: 1 <= M <= 8 activation rows, one wave per 2048 columns of K,
// at most 8 waves.
constexpr int kGemvMaxWaves = 8;
constexpr int kGemvMaxM = 8;
inline bool w4_gemv_supports(int64_t M, int64_t K)
{
    return M >= 1 && M <= kGemvMaxM && K <= 2048 * kGemvMaxWaves;
}

// The whole decode linear in one launch (w4_gemv_fused.hip): rotate-quant of
// 1 <= M <= 4 bf16 rows and the GEMV, one workgroup of up to 16 waves per
// compute unit.  Workgroup shape: nws streaming waves (S = ceil(K / 2048)
// column slices for each of RB blocks of 8 weight rows, at most 12 waves) and
// nwr rotation waves (a multiple of 4 that fits in 16, no more than the
// 8-column chunks of a row need), cpr chunks per rotation thread and row (M * cpr <= 8: the
// rotated values stay in registers), lds bytes of dynamic LDS (the M * K
// codes, raised above half the CU's LDS when the grid fits the chip, so that
// no CU runs two workgroups).  RB is the largest that covers N with one
// workgroup per CU and leaves the rotation enough waves.
constexpr int kGemvFusedMaxRows = 4;
constexpr int kFusedMaxWaves = 16, kFusedMaxStreamWaves = 12, kFusedMaxChunks = 8;
struct FusedGemvShape {
    int nb, nws, nwr, s, rb, cpr, lds;
};
inline bool w4_gemv_fused_shape(int64_t M, int64_t K, int64_t N, int ncu, FusedGemvShape &sh)
{
    if (M < 1 || M > kGemvFusedMaxRows || K < 64 || K > 2048 * kGemvMaxWaves || K % 64 != 0 || N < 8 ||
        N % 8 != 0 || ncu < 1)
        return false;
    const int64_t nrb = N / 8, nchunk = K / 8, s = (K + 2047) / 2048;
    int64_t rb = (nrb + ncu - 1) / ncu;
    if (rb * s > kFusedMaxStreamWaves)
        rb = kFusedMaxStreamWaves / s;
    for (; rb >= 1; --rb) {
        const int64_t nws = rb * s;
        // A multiple of 4 rotation waves: consecutive waves of a workgroup go
        // to the CU's 4 SIMDs in turn, so each SIMD gets the same share.
        int64_t nwr = (kFusedMaxWaves - nws) / 4 * 4;
        if (nwr > (nchunk + 63) / 64)
            nwr = (nchunk + 63) / 64;
        const int64_t c = (nchunk + 64 * nwr - 1) / (64 * nwr);
        const int64_t cpr = c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : 8;
        if (c > 8 || M * cpr > kFusedMaxChunks)
            continue;
        sh.s = (int)s, sh.rb = (int)rb, sh.nws = (int)nws, sh.nwr = (int)nwr, sh.cpr = (int)cpr;
        sh.nb = (int)((nrb + rb - 1) / rb);
        const int64_t lds = M * K;
        constexpr int64_t kOneWorkgroupPerCu = 80 * 1024 + 16;
        sh.lds = (int)(sh.nb <= ncu && lds < kOneWorkgroupPerCu ? kOneWorkgroupPerCu : lds);
        return true;
    }
    return false;
}
inline bool w4_gemv_fused_supports(int64_t M, int64_t K)
{
    FusedGemvShape sh;
    return w4_gemv_fused_shape(M, K, 8, 1, sh);
}
int launch_w4_gemv_fused(const uint16_t *x, int64_t ldx, int G, int qmax, int M, int K, const uint8_t *packed,
                         int64_t ldw, const uint16_t *w_scales, bool per_group, int N, const uint16_t *bias,
                         float x_scale, uint16_t *out, int64_t ldo, void *stream);

// The whole linear in one launch on int8 MFMA (w4_skinny_fused.hip): rotate-quant
// of 1 <= M <= 8 bf16 rows (K <= 4096) and the few-row matmul, one workgroup
// per compute unit.  Workgroup shape: nws = t * s streaming waves (s = ceil(K /
// 2048) slices of 32 K-groups for each of t tiles of 16 weight rows; the
// workgroup's rows, a multiple of 8, fill t tiles except perhaps 8 rows of the
// last) and kSfRotWaves rotation waves (one 8-column chunk per thread and row).
// lds: t * s slices of 16 rows (kSfSlicePitch bytes apart), their weight scales
// (kSfScaleDwords each) and partial sums (2 KiB each: two 16-group blocks), and
// the codes (kSfCodeGroup bytes per K-group, 32 s groups),
// raised above half the CU's LDS when the grid fits the chip, so that no CU
// runs two workgroups.
constexpr int kSfMaxRows = 8, kSfRotWaves = 8, kSfGroupsPerWave = 32, kSfMaxStreamWaves = 8;
constexpr int kSfSlicePitch = 1040, kSfCodeGroup = 576, kSfScaleDwords = 256;
constexpr int kSfMaxLds = 160 * 1024 - 512;  // the CU's LDS less the static counters (at most 288 bytes)
struct SkinnyFusedShape {
    int nb, rows, t, s, nws, lds;
};
inline bool w4_skinny_fused_shape(int64_t M, int64_t K, int64_t N, int ncu, SkinnyFusedShape &sh)
{
    if (M < 1 || M > kSfMaxRows || K < 64 || K % 64 != 0 || K > 8 * 64 * kSfRotWaves || N < 16 || N % 16 != 0 ||
        ncu < 1)
        return false;
    const int64_t ng = K / 64, s = (ng + kSfGroupsPerWave - 1) / kSfGroupsPerWave;
    const int64_t per_wave = 16 * kSfSlicePitch + 4 * kSfScaleDwords + 2 * 1024;
    const int64_t codes = (int64_t)kSfCodeGroup * kSfGroupsPerWave * s;
    int64_t tmax = (kSfMaxLds - codes) / (s * per_wave);
    if (tmax * s > kSfMaxStreamWaves)
        tmax = kSfMaxStreamWaves / s;
    if (tmax < 1)
        return false;
    int64_t rows = ((N + ncu - 1) / ncu + 7) / 8 * 8;
    if (rows > 16 * tmax)
        rows = 16 * tmax;
    const int64_t t = (rows + 15) / 16;
    sh.rows = (int)rows, sh.t = (int)t, sh.s = (int)s, sh.nws = (int)(t * s);
    sh.nb = (int)((N + rows - 1) / rows);
    const int64_t lds = t * s * per_wave + codes;
    constexpr int64_t kOneWorkgroupPerCu = 80 * 1024 + 16;
    sh.lds = (int)(sh.nb <= ncu && lds < kOneWorkgroupPerCu ? kOneWorkgroupPerCu : lds);
    return true;
}
inline bool w4_skinny_fused_supports(int64_t M, int64_t K)
{
    SkinnyFusedShape sh;
    return w4_skinny_fused_shape(M, K, 16, 1, sh);
}
int launch_w4_skinny_fused(const uint16_t *x, int64_t ldx, int G, int qmax, int M, int K, const uint8_t *packed,
                           int64_t ldw, const uint16_t *w_scales, bool per_group, int N, const uint16_t *bias,
                           float x_scale, uint16_t *out, int64_t ldo, void *stream);


// Compute units of the current device (looked up once per device; 256 if the
// query fails).
int device_cu_count();

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
