/*
 * ck.h - C ABI of the ConvRot packed-INT4 linear for AMD Instinct MI355X (gfx950).
 *
 * The library (libck.so) implements one hot path with hand-written HIP kernels:
 *
 *   x (bf16 [M,K])
 *     -> group-wise Walsh-Hadamard rotation (contiguous groups of G columns,
 *        H_G / sqrt(G), Sylvester natural order)
 *     -> rowwise absmax quantisation to int8 (qmax 127, "W4A8") or int4
 *        (qmax 7, "W4A4"; one value per byte)
 *     -> integer matmul with packed uint4 weights, int32 accumulation
 *     -> scale epilogue (row scale x weight scale), bf16 out.
 *
 * Sources (page titles):
 *  [RQ]   "[PR #155] [Feat][Ascend] Add fused RotateQuant backend", section
 *         "What this PR does": quantize_and_rotate_rowwise fuses the rotation
 *         matmul and the dynamic rowwise quantisation; group sizes 16, 64 and
 *         256; non-contiguous inputs; unsupported shapes are declined; the
 *         public API keeps scales positive (all-zero rows).
 *  [AWQ]  "comfy_kitchen/tensor/awq_w4a16.py", module docstring and
 *         dequantize(): qweight (N, K//2) packed uint4, bits 0..3 = column
 *         2j, bits 4..7 = column 2j+1, value = code - 8; per-group scales and
 *         zeros of shape (K // G, N); W = (q - 8) * s + z.
 *  [GEMV] "[PR #182] HIP port of #176: W4A8 decode GEMV and fused
 *         GatedDeltaNet decode", description: register-side int4 decode feeding
 *         integer dot products, rowwise x weight-scale epilogue.
 *  [SD]   "feat: support packed INT4 convrot models" (stable-diffusion.cpp),
 *         summary: W4A4 and W4A8 packed-INT4 ConvRot matmul with optional bias
 *         and input scale; 64-element ConvRot groups.
 *  [W4A4] "[PR #212] [Perf][Ascend] Reuse unpacked W4A4 weights within an
 *         explicit scope", summary: the public ConvRot W4A4 Linear dispatcher;
 *         packed weights may be int8 or uint8 tensors and may be strided.
 *
 * Conventions for every entry point:
 *  - bf16 values are passed as uint16_t bit patterns.
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees, copies to the host or synchronises; work is
 *    enqueued on `stream` (a hipStream_t; NULL = the null stream) and inputs
 *    must stay alive until that work completes.  Outputs are fully written.
 *  - Matrices are row-major with explicit row strides in ELEMENTS (bytes for
 *    the packed weights, whose element is a byte holding two codes).
 *  - Arguments are validated before anything is enqueued.  A failed check
 *    returns a status and enqueues nothing; ck_last_error_msg() then gives a
 *    thread-local description.  Faults inside a kernel surface at the
 *    caller's next synchronisation.
 *  - M == 0 is a valid no-op.
 *  - Shape rules.  CK_ERR_INVALID_ARG: K <= 0, K % 64 != 0 or K % G != 0
 *    (a row must split into whole 64-column weight-scale groups and whole
 *    rotation groups).  CK_ERR_UNSUPPORTED (valid, outside what this build
 *    serves): G not in {16, 64, 256}; bits not in {8, 4}; K > 32768;
 *    N % 16 != 0; weight-scale group Gw != 64 for per-group scales;
 *    M or N >= 2^22 (one launch's grid); for shapes that run the tiled
 *    GEMM ceil(M / 128) * ceil(N / 256) >= 2^23; row strides of codes and
 *    packed weights ldq, ldw > 2^23 bytes.
 *  - Every entry point returns a ck_status (CK_OK on success).
 *  - Alignment (CK_ERR_INVALID_ARG otherwise): x and codes 16-byte aligned,
 *    ldx % 8 == 0, ldq % 16 == 0, packed weights 16-byte aligned with
 *    ldw % 16 == 0; per-group weight scales, AWQ scales and zero points
 *    16-byte aligned (per-channel weight scales 2-byte aligned); outputs
 *    16-byte aligned with 16-byte aligned rows (bf16: ldo % 8 == 0; int32
 *    test outputs: lda % 4 == 0).
 */
#ifndef CK_H
#define CK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CK_OK = 0,
    CK_ERR_INVALID_ARG = 1, /* null pointer, bad stride/alignment, overlap, K%G, ... */
    CK_ERR_UNSUPPORTED = 2, /* valid request outside the shapes this build serves   */
    CK_ERR_WORKSPACE = 3,   /* workspace pointer missing or smaller than required   */
    CK_ERR_HIP = 4          /* the HIP runtime refused a launch                      */
} ck_status;

/* Weight-scale kinds.
 * CK_WS_PER_CHANNEL: bf16 [N], one scale per output column.
 * CK_WS_PER_GROUP:   bf16 [K/Gw, N] (N contiguous), one scale per (K-group, n),
 *                    Gw = 64; same layout as the per-group scales in [AWQ]. */
typedef enum { CK_WS_PER_CHANNEL = 0, CK_WS_PER_GROUP = 1 } ck_wscale_kind;

/* Static string for a status code. */
const char *ck_status_str(ck_status status);

/* Thread-local message of the last failed call on this thread ("" if none). */
const char *ck_last_error_msg(void);

/* Library version, e.g. "ck 0.1 gfx950". */
const char *ck_version(void);

/*
 * ck_rotate_quant  [RQ]
 * Rotate each contiguous group of G columns of every row of x by H_G/sqrt(G)
 * and quantise the row by its absolute maximum a (over the whole row):
 *   row_scales[m] = a / qmax, codes[m,k] = round_half_even(xr[m,k] * qmax / a)
 * with qmax = 127 (bits 8) or 7 (bits 4); the multiply uses the fp32
 * reciprocal qmax/a and the codes never exceed +-qmax.  An all-zero row gets
 * codes 0 and row_scales[m] = 1.0 (positive-scale contract of [RQ]).
 *   x          bf16 [M, ldx]; the first K columns of each row are read
 *   codes      int8 [M, ldq]; the first K columns are written (int4 codes are
 *              stored one value per byte, range [-7, 7])
 *   row_scales fp32 [M]
 * codes/row_scales must not overlap x.
 */
ck_status ck_rotate_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G,
                    int32_t bits, int8_t *codes, int64_t ldq, float *row_scales,
                    void *stream);

/*
 * ck_w4_gemm_q  [GEMV] [AWQ] [SD]
 * Matmul half of the linear, for activations that are already rotated and
 * quantised (for example by ck_rotate_quant, or reused across linears that
 * share an input as [SD] does with its activation cache):
 *   acc[m,n]    = sum_k codes[m,k] * (q[n,k] - 8)               (exact int32)
 *   per channel: out[m,n] = row_scales[m] * w_scales[n] * acc[m,n]
 *   per group:   out[m,n] = row_scales[m] * sum_g w_scales[g,n] * acc_g[m,n]
 *   (+ bias[n] when bias != NULL), rounded to bf16 (nearest even).
 *   codes      int8 [M, ldq] (int8 or int4 values)
 *   row_scales fp32 [M]
 *   packed     uint8 [N, ldw]: byte j of row n holds column 2j in bits 0..3
 *              and column 2j+1 in bits 4..7; code q in [0,15] means q - 8
 *   w_scales   bf16, layout given by scale_kind (ck_wscale_kind); Gw = 64
 *   bias       bf16 [N] or NULL
 *   out        bf16 [M, ldo]; must not overlap any input
 * Any M >= 0.  Small M (<= 64, with K small enough for the activations to
 * stay in registers) runs the weight-streaming kernel of ck_w4_gemv; every
 * other shape runs the tiled MFMA GEMM.
 */
ck_status ck_w4_gemm_q(const int8_t *codes, int64_t ldq, const float *row_scales, int64_t M,
                 int64_t K, const uint8_t *packed, int64_t ldw, const uint16_t *w_scales,
                 int32_t scale_kind, int32_t Gw, int64_t N, const uint16_t *bias,
                 uint16_t *out, int64_t ldo, void *stream);

/*
 * ck_w4_gemv  [GEMV]
 * Decode form of ck_w4_gemm_q for 1 <= M <= 8 and K <= 16384
 * (CK_ERR_UNSUPPORTED otherwise): the same arithmetic, run by a kernel that
 * streams the packed weights once (VALU dot products for M <= 5, MFMA for
 * 6 <= M <= 8 when K fits its range).
 */
ck_status ck_w4_gemv(const int8_t *codes, int64_t ldq, const float *row_scales, int64_t M,
               int64_t K, const uint8_t *packed, int64_t ldw, const uint16_t *w_scales,
               int32_t scale_kind, int32_t Gw, int64_t N, const uint16_t *bias,
               uint16_t *out, int64_t ldo, void *stream);

/*
 * ck_rotate_quant_packed4  [RQ] [W4A4]
 * ck_rotate_quant(bits = 4) with the codes stored two per byte:
 *   codes4  uint8 [M, ldq], ldq >= K/2 bytes and a multiple of 16, 16-byte
 *           aligned; byte j of a row holds column 2j in bits 0..3 and column
 *           2j + 1 in bits 4..7, each code in [-7, 7] as 4-bit two's
 *           complement;
 *   row_scales fp32 [M] as in ck_rotate_quant.
 * The codes are the same as ck_rotate_quant's.  Quantised once, they can be
 * reused by every ck_w4a4_gemm_packed that shares the input (the activation
 * cache of [SD], for inputs of scale 1).
 */
ck_status ck_rotate_quant_packed4(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G,
                            uint8_t *codes4, int64_t ldq, float *row_scales, void *stream);

/*
 * ck_w4a4_gemm_packed  [W4A4] [SD]
 * ck_w4_gemm_q on W4A4 codes packed two per byte (as ck_rotate_quant_packed4
 * writes them), on the tiled MFMA GEMM for every M >= 1:
 *   out[m,n] = bf16( acc[m,n] * row_scales[m] * s_w(n) (+ bias[n]) ),
 *   acc[m,n] = sum_k code[m,k] * (q[n,k] - 8).
 * Weights, scales, bias and out as in ck_w4_gemm_q; codes4 uint8 [M, ldq],
 * ldq >= K/2.  This is the matmul half of ck_w4a4_linear for M > 64.
 */
ck_status ck_w4a4_gemm_packed(const uint8_t *codes4, int64_t ldq, const float *row_scales, int64_t M,
                        int64_t K, const uint8_t *packed, int64_t ldw, const uint16_t *w_scales,
                        int32_t scale_kind, int32_t Gw, int64_t N, const uint16_t *bias,
                        uint16_t *out, int64_t ldo, void *stream);

/* Bytes of workspace ck_w4a8_linear / ck_w4a4_linear need for M rows of K
 * columns and N outputs: int8 codes for M rows rounded up to a multiple of 16
 * (K bytes per row), then the fp32 row scales, each part 256-byte aligned
 * inside the workspace.  No part depends on N, which is taken so that a later
 * matmul needing per-output scratch keeps this signature.  0 for M <= 0. */
size_t ck_linear_workspace_bytes(int64_t M, int64_t K, int64_t N);

/*
 * ck_w4a8_linear  [SD] [RQ] [GEMV]
 * Whole ConvRot linear with int8 activations:
 *   ck_rotate_quant(x, G, bits = 8) into `ws`, then ck_w4_gemm_q on `ws`,
 * both on `stream`; for 1 <= M <= 4 one launch instead (M <= 3 when
 * K > 8192), with one workgroup per compute unit, whose rotation waves
 * rotate and quantise the rows into LDS while its other waves stream the
 * weights (same codes, same results bit for bit); for 5 <= M <= 8 with
 * K <= 4096 and N >= 8192 one launch too, its products on int8 MFMA (the
 * same results as ck_rotate_quant + ck_w4_gemm_q bit for bit).  Otherwise,
 * for 6 <= M <= 64 the codes are held in the few-row kernel's operand layout
 * (16-row tiles) rather than row-major.  x_scale (> 0, finite; 1.0 for none) is the input-scale
 * factor of [SD]: the result is the linear of x_scale * x, obtained by
 * multiplying each row scale by x_scale (the codes of x_scale * x equal those
 * of x whenever x_scale is a power of two).
 *   ws        device workspace of at least ck_linear_workspace_bytes(M, K)
 *             bytes, 256-byte aligned; CK_ERR_WORKSPACE if smaller or NULL
 *             (with M > 0).  Its contents are scratch.
 */
ck_status ck_w4a8_linear(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G,
                   const uint8_t *packed, int64_t ldw, const uint16_t *w_scales,
                   int32_t scale_kind, int32_t Gw, int64_t N, const uint16_t *bias,
                   float x_scale, uint16_t *out, int64_t ldo, void *ws, size_t ws_bytes,
                   void *stream);

/*
 * ck_w4a4_linear  [W4A4] [SD]
 * As ck_w4a8_linear with int4 activations (qmax 7, symmetric).  When the
 * tiled GEMM serves M (more rows than the few-row kernels take), the codes are
 * held in the workspace two per byte (4-bit two's complement, column 2j in
 * the low nibble), as ck_rotate_quant_packed4 writes them; the result is
 * the same as with one code per byte.
 */
ck_status ck_w4a4_linear(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G,
                   const uint8_t *packed, int64_t ldw, const uint16_t *w_scales,
                   int32_t scale_kind, int32_t Gw, int64_t N, const uint16_t *bias,
                   float x_scale, uint16_t *out, int64_t ldo, void *ws, size_t ws_bytes,
                   void *stream);

/*
 * ck_w4a4_linear_noalloc
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): ck_w4a4_linear
 * with the codes and row scales held in a scratch array owned by the library
 * instead of a caller workspace.  Same arguments minus ws / ws_bytes, same
 * kernels, same results bit for bit.
 *   - The scratch is a static device array of 64 MiB + 64 KiB (67174400 bytes), one
 *     copy on each GPU that loads the library, kept until the process ends.
 *     A call needing more returns CK_ERR_UNSUPPORTED before anything is
 *     enqueued: M * K / 2 bytes of packed codes (tiled GEMM, M > 64),
 *     ceil(M / 16) * 16 * K bytes (the few-row kernel's 16-row tiles) or M * K
 *     bytes (the GEMV), each rounded up to 256, plus 4 * M bytes of row
 *     scales rounded up to 256; the one-launch decode shapes (M <= 4, or
 *     M <= 3 when K > 8192; 5 <= M <= 8 with K <= 4096 and N >= 8192) use
 *     no scratch.
 *     For example M = 8192 rows fit up to K = 16384, and M = 16384 rows up
 *     to K = 8192.
 *   - The call allocates nothing (no hipMalloc, no allocating library call).
 *     Its scratch address on a device is looked up (hipGetSymbolAddress) on the
 *     first call made with that device current; `stream` must belong to the
 *     current device (CK_ERR_HIP otherwise).
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents; each call writes all it reads.  Calls that can overlap
 *     on one GPU (different streams, or threads without ordering) race on the
 *     scratch: order them on one stream.
 */
ck_status ck_w4a4_linear_noalloc(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G,
                                 const uint8_t *packed, int64_t ldw, const uint16_t *w_scales,
                                 int32_t scale_kind, int32_t Gw, int64_t N, const uint16_t *bias,
                                 float x_scale, uint16_t *out, int64_t ldo, void *stream);

/*
 * ck_w4a16_gemv  [AWQ]
 * AWQ W4A16 product with fp activations (no activation quantisation):
 *   W[n,k]   = (q[n,k] - 8) * scales[k/Gw, n] + zeros[k/Gw, n]
 *   out[m,n] = sum_k x[m,k] * W[n,k]  (+ bias[n]), fp32 arithmetic, bf16 out.
 *   x       bf16 [M, ldx], 1 <= M <= 8 and K <= 16384 (CK_ERR_UNSUPPORTED
 *           otherwise)
 *   packed  uint8 [N, ldw] as in ck_w4_gemm_q
 *   scales, zeros  bf16 [K/Gw, N], Gw = 64, each 16-byte aligned
 *           (CK_ERR_INVALID_ARG otherwise)
 *   bias    bf16 [N] or NULL;  out bf16 [M, ldo]
 * The weight is never materialised; it is decoded in registers.
 */
ck_status ck_w4a16_gemv(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                  const uint8_t *packed, int64_t ldw, const uint16_t *scales,
                  const uint16_t *zeros, int32_t Gw, int64_t N, const uint16_t *bias,
                  uint16_t *out, int64_t ldo, void *stream);

/*
 * ck_w4a16_gemm  [AWQ]
 * AWQ W4A16 product for any number of rows (prefill), on the page's
 * dequantise path (dequantize(), used when no quantised kernel runs): the
 * weight is rebuilt in bf16 one tensor operation at a time,
 *   W[n,k]   = bf16( bf16((q[n,k] - 8) * scales[k/Gw, n]) + zeros[k/Gw, n] ),
 *   out[m,n] = sum_k x[m,k] * W[n,k]  (+ bias[n]), fp32 accumulation, bf16 out.
 * The rebuilt weight lives only in registers.  It differs from ck_w4a16_gemv
 * (which keeps W exact) by W's bf16 rounding.
 *   x       bf16 [M, ldx], ldx <= 2^22, any M >= 0
 *   packed  uint8 [N, ldw] as in ck_w4_gemm_q; N % 16 == 0
 *   scales, zeros  bf16 [K/Gw, N], Gw = 64, each 16-byte aligned
 *           (CK_ERR_INVALID_ARG otherwise)
 *   bias    bf16 [N] or NULL;  out bf16 [M, ldo] (16-byte aligned rows)
 */
ck_status ck_w4a16_gemm(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                  const uint8_t *packed, int64_t ldw, const uint16_t *scales,
                  const uint16_t *zeros, int32_t Gw, int64_t N, const uint16_t *bias,
                  uint16_t *out, int64_t ldo, void *stream);

/*
 * ck_quantize_weights  [SD] [AWQ]
 * Offline producer of the packed weights the matmuls consume, for a bf16
 * weight W [N, K] (row n = output column n):
 *   wr = each contiguous G-column group of each row times H_G / sqrt(G)
 *        (the rotation ck_rotate_quant applies to activations, so that the
 *        product of rotated activations and rotated weights is x . W^T);
 *   a  = max |wr| over the row (CK_WS_PER_CHANNEL) or over each 64-column
 *        group of the row (CK_WS_PER_GROUP, Gw = 64);
 *   s  = bf16(fp32(a / 7)); code = clamp(rne(fp32(wr * fp32(1 / s))), -7, 7)
 *        (code 0 where s == 0); stored q = code + 8, packed two per byte:
 *        byte j of row n = q[n, 2j] | q[n, 2j + 1] << 4.
 * The pages hold packed checkpoints ([SD] summary) and the packed layout
 * ([AWQ] module docstring) but no weight-quantiser formula; symmetric
 * absmax / 7 is the reading taken.
 *   w       bf16 [N, ldw_in], ldw_in >= K, ldw_in % 8 == 0, 16-byte aligned
 *   packed  uint8 [N, ldp], ldp >= K/2, ldp % 16 == 0, 16-byte aligned
 *   scales  bf16 [N] (per channel) or [K/64, N] (per group)
 * G and K as in ck_rotate_quant; N <= 2^22.  Runs on `stream`.
 */
ck_status ck_quantize_weights(const uint16_t *w, int64_t N, int64_t K, int64_t ldw_in, int32_t G,
                        int32_t scale_kind, uint8_t *packed, int64_t ldp, uint16_t *scales,
                        void *stream);

/* ---------------------------------------------------------------- test hooks
 * Same device code paths as above with a debug epilogue, so that each stage
 * can be compared exactly with the oracle. */

/* The rotation of ck_rotate_quant as held in registers, divided by sqrt(G)
 * (exact, sqrt(G) is a power of two): xr fp32 [M, ldr].  It runs the kernel
 * instantiation that ck_rotate_quant and ck_rotate_quant_packed4 run for the
 * same M, K and G (8-column chunks at G = 16 and for up to 64 rows of up to
 * 4096 columns, 16-column chunks otherwise).
 * The weight producer (ck_quantize_weights) always uses 8-column chunks; those
 * apply the same butterfly stages to the same operands in the same order, so
 * the values are identical, which its bit-exact test checks. */
ck_status ck_test_rotate_f32(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G,
                       float *xr, int64_t ldr, void *stream);

/* The whole linear (bits 8: ck_w4a8_linear, bits 4: ck_w4a4_linear; same
 * arguments without the workspace) always on its one-launch MFMA form, which
 * those entry points choose only for 5 to 8 rows and N >= 8192, so that every
 * launch shape of that kernel can be checked: 1 <= M <= 8, K <= 4096, any N
 * (CK_ERR_UNSUPPORTED otherwise).  Results equal ck_rotate_quant followed by
 * ck_w4_gemm_q on the few-row kernel bit for bit. */
ck_status ck_test_linear_mfma_one_launch(int32_t bits, const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                         int32_t G, const uint8_t *packed, int64_t ldw,
                                         const uint16_t *w_scales, int32_t scale_kind, int32_t Gw, int64_t N,
                                         const uint16_t *bias, float x_scale, uint16_t *out, int64_t ldo,
                                         void *stream);

/* The integer accumulators of ck_w4_gemm_q (kernel chosen by M exactly as
 * there): acc int32 [M, lda], acc[m,n] = sum_k codes[m,k] * (q[n,k] - 8). */
ck_status ck_test_gemm_i32(const int8_t *codes, int64_t ldq, int64_t M, int64_t K,
                     const uint8_t *packed, int64_t ldw, int64_t N, int32_t *acc,
                     int64_t lda, void *stream);

/* The integer accumulators of the tiled GEMM on packed W4A4 codes (codes4 as
 * written by ck_rotate_quant_packed4), for any M >= 1:
 * acc[m,n] = sum_k code[m,k] * (q[n,k] - 8), acc int32 [M, lda]. */
ck_status ck_test_gemm_i32_a4(const uint8_t *codes4, int64_t ldq, int64_t M, int64_t K,
                        const uint8_t *packed, int64_t ldw, int64_t N, int32_t *acc,
                        int64_t lda, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CK_H */
