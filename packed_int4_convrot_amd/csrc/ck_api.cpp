// C ABI of libck: argument validation and dispatch.  Pure host C++: nothing
// here touches the GPU until every check has passed, so the error paths can be
// exercised on a machine without a GPU.  Semantics of each entry point are
// documented in include/ck.h.
#include "../../include/ck.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok()
{
    g_last_error.clear();
    return CK_OK;
}

int hip_status(int e, const char *what)
{
    if (e != 0)
        return fail(CK_ERR_HIP, "%s: HIP launch failed (hipError_t %d)", what, e);
    return ok();
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte range [lo, hi) spanned by `rows` rows of `cols` elements of `esize`
// bytes with row stride `ld` elements.
struct Range {
    uintptr_t lo = 0, hi = 0;
};
Range span(const void *p, int64_t rows, int64_t cols, int64_t ld, int64_t esize)
{
    Range r;
    if (!p || rows <= 0 || cols <= 0)
        return r;
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + (uintptr_t)(((rows - 1) * ld + cols) * esize);
    return r;
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

constexpr int64_t kMaxK = 32768;
// Row strides of codes and packed weights, in bytes: the tiled GEMM addresses
// a block's 256 rows with 32-bit buffer offsets.
constexpr int64_t kMaxLd = int64_t(1) << 23;
// A launch covers at most 2^32 - 1 work-items per grid dimension.  Rotate-quant
// and the weight producer launch one workgroup of up to 1024 threads per row,
// so the rows stay below 2^22: (2^22 - 1) * 1024 = 2^32 - 1024 work-items.
constexpr int64_t kMaxRows = (int64_t(1) << 22) - 1;
// The tiled GEMM launches one 512-thread workgroup per 256 x 256 (or
// 128 x 256) output tile.
constexpr int64_t kMaxGemmTiles = (int64_t(1) << 32) / 512 - 1;

int check_k(const char *fn, int64_t K)
{
    if (K <= 0)
        return fail(CK_ERR_INVALID_ARG, "%s: K must be positive (got %lld)", fn, (long long)K);
    if (K % 64 != 0)
        return fail(CK_ERR_INVALID_ARG, "%s: K must be a multiple of 64 (got %lld)", fn, (long long)K);
    if (K > kMaxK)
        return fail(CK_ERR_UNSUPPORTED, "%s: K must be at most %lld (got %lld)", fn, (long long)kMaxK,
                    (long long)K);
    return CK_OK;
}

int check_g(const char *fn, int32_t G, int64_t K)
{
    if (G != 16 && G != 64 && G != 256)
        return fail(CK_ERR_UNSUPPORTED, "%s: rotation group G must be 16, 64 or 256 (got %d)", fn, G);
    if (K % G != 0)
        return fail(CK_ERR_INVALID_ARG, "%s: K (%lld) is not a multiple of G (%d)", fn, (long long)K, G);
    return CK_OK;
}

int check_m(const char *fn, int64_t M)
{
    if (M < 0)
        return fail(CK_ERR_INVALID_ARG, "%s: M must be >= 0 (got %lld)", fn, (long long)M);
    if (M > kMaxRows)
        return fail(CK_ERR_UNSUPPORTED, "%s: M above %lld", fn, (long long)kMaxRows);
    return CK_OK;
}

int check_x(const char *fn, const uint16_t *x, int64_t K, int64_t ldx)
{
    if (!x)
        return fail(CK_ERR_INVALID_ARG, "%s: x is NULL", fn);
    if (ldx < K || ldx % 8 != 0)
        return fail(CK_ERR_INVALID_ARG, "%s: ldx (%lld) must be >= K and a multiple of 8", fn,
                    (long long)ldx);
    if (!aligned(x, 16))
        return fail(CK_ERR_INVALID_ARG, "%s: x must be 16-byte aligned", fn);
    return CK_OK;
}

int check_codes(const char *fn, const void *codes, int64_t K, int64_t ldq)
{
    if (!codes)
        return fail(CK_ERR_INVALID_ARG, "%s: codes is NULL", fn);
    if (ldq < K || ldq % 16 != 0)
        return fail(CK_ERR_INVALID_ARG, "%s: ldq (%lld) must be >= K and a multiple of 16", fn,
                    (long long)ldq);
    if (ldq > kMaxLd)
        return fail(CK_ERR_UNSUPPORTED, "%s: ldq (%lld) must be at most %lld bytes", fn, (long long)ldq,
                    (long long)kMaxLd);
    if (!aligned(codes, 16))
        return fail(CK_ERR_INVALID_ARG, "%s: codes must be 16-byte aligned", fn);
    return CK_OK;
}

struct Weights {
    const uint8_t *packed;
    int64_t ldw;
    const uint16_t *scales;
    int32_t kind, Gw;
    int64_t N;
};

int check_weights(const char *fn, const Weights &w, int64_t K, bool need_scales)
{
    if (!w.packed)
        return fail(CK_ERR_INVALID_ARG, "%s: packed weights are NULL", fn);
    if (w.N <= 0)
        return fail(CK_ERR_INVALID_ARG, "%s: N must be positive (got %lld)", fn, (long long)w.N);
    if (w.N % 16 != 0 || w.N > kMaxRows)
        return fail(CK_ERR_UNSUPPORTED, "%s: N must be a multiple of 16 and at most %lld (got %lld)", fn,
                    (long long)kMaxRows, (long long)w.N);
    if (w.ldw < K / 2 || w.ldw % 16 != 0)
        return fail(CK_ERR_INVALID_ARG, "%s: ldw (%lld) must be >= K/2 and a multiple of 16", fn,
                    (long long)w.ldw);
    if (w.ldw > kMaxLd)
        return fail(CK_ERR_UNSUPPORTED, "%s: ldw (%lld) must be at most %lld bytes", fn, (long long)w.ldw,
                    (long long)kMaxLd);
    if (!aligned(w.packed, 16))
        return fail(CK_ERR_INVALID_ARG, "%s: packed weights must be 16-byte aligned", fn);
    if (need_scales) {
        if (!w.scales)
            return fail(CK_ERR_INVALID_ARG, "%s: weight scales are NULL", fn);
        if (w.kind != CK_WS_PER_CHANNEL && w.kind != CK_WS_PER_GROUP)
            return fail(CK_ERR_INVALID_ARG, "%s: unknown weight-scale kind %d", fn, w.kind);
        if (w.kind == CK_WS_PER_GROUP && w.Gw != 64)
            return fail(CK_ERR_UNSUPPORTED, "%s: per-group weight scales need Gw == 64 (got %d)", fn, w.Gw);
        if (!aligned(w.scales, w.kind == CK_WS_PER_GROUP ? 16 : 2))
            return fail(CK_ERR_INVALID_ARG, "%s: weight scales must be %d-byte aligned", fn,
                        w.kind == CK_WS_PER_GROUP ? 16 : 2);
    }
    return CK_OK;
}

Range scales_span(const Weights &w, int64_t K)
{
    if (w.kind == CK_WS_PER_GROUP)
        return span(w.scales, K / 64, w.N, w.N, 2);
    return span(w.scales, 1, w.N, w.N, 2);
}

// Outputs are written with 16-byte stores: 16-byte aligned rows.
int check_out(const char *fn, const void *out, int64_t N, int64_t ldo, size_t esize)
{
    if (!out)
        return fail(CK_ERR_INVALID_ARG, "%s: output is NULL", fn);
    const int64_t per16 = 16 / (int64_t)esize;
    if (ldo < N || ldo % per16 != 0)
        return fail(CK_ERR_INVALID_ARG, "%s: output stride (%lld) must be >= N and a multiple of %lld",
                    fn, (long long)ldo, (long long)per16);
    if (!aligned(out, 16))
        return fail(CK_ERR_INVALID_ARG, "%s: output must be 16-byte aligned", fn);
    return CK_OK;
}

#define CK_TRY(expr)            \
    do {                        \
        int _st = (expr);       \
        if (_st != CK_OK)       \
            return _st;         \
    } while (0)

constexpr size_t kWsAlign = 256;
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Whole-linear workspace: the int8 codes of M rows padded to a multiple of 16
// (the tiled layout of the few-row kernel fills whole 16-row tiles), then the
// fp32 row scales.
size_t codes_bytes_padded(int64_t M, int64_t K) { return (size_t)((M + 15) / 16 * 16) * (size_t)K; }
size_t workspace_bytes(int64_t M, int64_t K)
{
    if (M <= 0 || K <= 0)
        return 0;
    return round_up(codes_bytes_padded(M, K), kWsAlign) + round_up((size_t)M * sizeof(float), kWsAlign);
}

// Dispatch of the integer matmul + epilogue by M.
enum class GemmPath { kGemv, kSkinny, kTiled };

// Kernel choice for M rows of pre-quantised codes.  The VALU GEMV's work grows
// with M while the MFMA few-row kernel's does not; measured on MI355X the
// few-row kernel is faster from 6 rows on.
GemmPath pick_path(int64_t M, int64_t K)
{
    constexpr int64_t kGemvMaxRows = 5;
    const bool gemv = ck::w4_gemv_supports(M, K);
    const bool skinny = M <= 64 && ck::w4_skinny_supports(M, K);
    if (gemv && (M <= kGemvMaxRows || !skinny))
        return GemmPath::kGemv;
    return skinny ? GemmPath::kSkinny : GemmPath::kTiled;
}

int check_tiles(const char *fn, int64_t M, int64_t N)
{
    if (((M + 127) / 128) * ((N + 255) / 256) > kMaxGemmTiles)
        return fail(CK_ERR_UNSUPPORTED, "%s: M * N too large for one launch (M=%lld, N=%lld)", fn,
                    (long long)M, (long long)N);
    return CK_OK;
}

// a4: the codes are W4A4 codes packed two per byte (ldq in bytes); only the
// tiled GEMM takes them.  tiled: the codes are in the few-row kernel's operand
// layout (CodesLayout::kTiled16); only that kernel takes them.
int run_gemm(const char *fn, const void *codes, int64_t ldq, const float *rs, int64_t M, int64_t K,
             const Weights &w, const uint16_t *bias, float x_scale, uint16_t *out, int64_t ldo,
             int32_t *acc, int64_t lda, bool a4, void *stream, bool tiled = false)
{
    const bool pg = w.kind == CK_WS_PER_GROUP;
    const GemmPath path = a4 ? GemmPath::kTiled : pick_path(M, K);
    if (tiled && path != GemmPath::kSkinny)
        return fail(CK_ERR_UNSUPPORTED, "%s: tiled codes reach only the few-row kernel", fn);
    const int8_t *c8 = static_cast<const int8_t *>(codes);
    int e;
    if (path == GemmPath::kGemv) {
        e = ck::launch_w4_gemv(c8, ldq, rs, (int)M, (int)K, w.packed, w.ldw,
                               w.scales, pg, (int)w.N, bias, x_scale, out, ldo, acc, lda, stream);
    } else if (path == GemmPath::kSkinny) {
        e = ck::launch_w4_skinny(c8, ldq, tiled, rs, (int)M, (int)K, w.packed, w.ldw, w.scales, pg,
                                 (int)w.N, bias, x_scale, out, ldo, acc, lda, stream);
    } else {
        CK_TRY(check_tiles(fn, M, w.N));
        e = ck::launch_w4_gemm(c8, ldq, rs, (int)M, (int)K, w.packed, w.ldw, w.scales, pg,
                               (int)w.N, bias, x_scale, out, ldo, acc, lda, a4, stream);
    }
    return hip_status(e, fn);
}

int gemm_q_common(const char *fn, bool gemv, const int8_t *codes, int64_t ldq, const float *rs,
                  int64_t M, int64_t K, const Weights &w, const uint16_t *bias, uint16_t *out,
                  int64_t ldo, void *stream)
{
    CK_TRY(check_m(fn, M));
    CK_TRY(check_k(fn, K));
    CK_TRY(check_weights(fn, w, K, true));
    const int64_t m1 = M < 1 ? 1 : M;
    if (gemv && (M > 8 || !(ck::w4_gemv_supports(m1, K) || ck::w4_skinny_supports(m1, K))))
        return fail(CK_ERR_UNSUPPORTED, "%s: decode GEMV takes 1 <= M <= 8 and K <= 16384 (M=%lld, K=%lld)",
                    fn, (long long)M, (long long)K);
    if (M == 0)
        return ok();
    CK_TRY(check_codes(fn, codes, K, ldq));
    if (!rs)
        return fail(CK_ERR_INVALID_ARG, "%s: row_scales is NULL", fn);
    if (!aligned(rs, 4))
        return fail(CK_ERR_INVALID_ARG, "%s: row_scales must be 4-byte aligned", fn);
    if (bias && !aligned(bias, 2))
        return fail(CK_ERR_INVALID_ARG, "%s: bias must be 2-byte aligned", fn);
    CK_TRY(check_out(fn, out, w.N, ldo, 2));
    const Range ro = span(out, M, w.N, ldo, 2);
    if (overlap(ro, span(codes, M, K, ldq, 1)) || overlap(ro, span(rs, 1, M, M, 4)) ||
        overlap(ro, span(w.packed, w.N, K / 2, w.ldw, 1)) || overlap(ro, scales_span(w, K)) ||
        overlap(ro, span(bias, 1, w.N, w.N, 2)))
        return fail(CK_ERR_INVALID_ARG, "%s: output overlaps an input", fn);
    return run_gemm(fn, codes, ldq, rs, M, K, w, bias, 1.0f, out, ldo, nullptr, 0, false, stream);
}

// How the whole linear runs for M rows: one fused launch (decode), or rotate-quant
// into scratch followed by the matmul kernel that pick_path() chooses.  W4A4
// codes bound for the tiled GEMM are stored two per byte, which halves the
// codes traffic on both sides of the scratch; codes bound for the few-row
// kernel are stored in its operand layout (whole 16-row tiles).
// One launch in the MFMA form (w4_skinny_fused) from kMfmaFusedMinRows rows on
// when the weights span at least kMfmaFusedMinN rows (32 or more per CU on a
// 256-CU MI355X); the VALU GEMV form (w4_gemv_fused) up to 4 rows otherwise.
// Measured on MI355X (K = 3840, graph replay, cold weights): at N = 10240 the
// MFMA form takes 10.0 / 10.3 / 10.8 / 11.2 us at M = 5 / 6 / 7 / 8 against
// 10.8 / 12.2 / 12.5 / 12.5 us for two launches (rotate-quant + the VALU GEMV at
// M = 5, + the few-row kernel above), but 8.9 / 9.3 / 9.8 us at M = 2 / 3 / 4
// against 7.1 / 8.2 / 9.5 us for the VALU form, and at N = 3840, M = 8 it
// takes 9.6 us against 8.5 us: every CU rotates all the rows, which is the
// longer part once the CU's share of the weights is small.
constexpr int64_t kMfmaFusedMinRows = 5, kMfmaFusedMinN = 8192;
struct LinearPlan {
    bool fused;           // one launch (either form)
    bool mfma_fused;      // ... the MFMA form
    GemmPath path;
    bool a4;
    bool tiled;           // codes in CodesLayout::kTiled16
    int64_t ldq;          // bytes per row of row-major codes in the scratch
    size_t scales_off;    // offset of the fp32 row scales
    size_t used;          // scratch bytes the plan touches (0 when fused)
};

LinearPlan plan_linear(int bits, int64_t M, int64_t K, int64_t N)
{
    LinearPlan p{};
    p.mfma_fused = M >= kMfmaFusedMinRows && N >= kMfmaFusedMinN && ck::w4_skinny_fused_supports(M, K);
    p.fused = p.mfma_fused || ck::w4_gemv_fused_supports(M, K);
    p.path = pick_path(M, K);
    p.a4 = !p.fused && bits == 4 && p.path == GemmPath::kTiled;
    p.tiled = !p.fused && p.path == GemmPath::kSkinny;
    p.ldq = p.a4 ? K / 2 : K;
    p.scales_off = round_up(p.tiled ? codes_bytes_padded(M, K) : (size_t)(M * p.ldq), kWsAlign);
    p.used = p.fused ? 0 : p.scales_off + round_up((size_t)M * sizeof(float), kWsAlign);
    return p;
}

// library_scratch: the scratch is the library's static device array
// (ck_w4a4_linear_noalloc) instead of the caller's workspace ws.
// force_mfma_one_launch: run the one-launch MFMA form whatever the plan (a test
// hook for its launch shapes; it needs no scratch).
int linear_common(const char *fn, int bits, const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                  int32_t G, const Weights &w, const uint16_t *bias, float x_scale, uint16_t *out,
                  int64_t ldo, void *ws, size_t ws_bytes, void *stream, bool library_scratch = false,
                  bool force_mfma_one_launch = false)
{
    CK_TRY(check_m(fn, M));
    CK_TRY(check_k(fn, K));
    CK_TRY(check_g(fn, G, K));
    CK_TRY(check_weights(fn, w, K, true));
    if (!(x_scale > 0.f) || !std::isfinite(x_scale))
        return fail(CK_ERR_INVALID_ARG, "%s: x_scale must be positive and finite", fn);
    if (M == 0)
        return ok();
    CK_TRY(check_x(fn, x, K, ldx));
    if (bias && !aligned(bias, 2))
        return fail(CK_ERR_INVALID_ARG, "%s: bias must be 2-byte aligned", fn);
    CK_TRY(check_out(fn, out, w.N, ldo, 2));
    const Range ro = span(out, M, w.N, ldo, 2);
    const Range rx = span(x, M, K, ldx, 2);
    if (overlap(ro, rx) || overlap(ro, span(w.packed, w.N, K / 2, w.ldw, 1)) ||
        overlap(ro, scales_span(w, K)) || overlap(ro, span(bias, 1, w.N, w.N, 2)))
        return fail(CK_ERR_INVALID_ARG, "%s: output overlaps an input", fn);
    LinearPlan plan = plan_linear(bits, M, K, w.N);
    if (force_mfma_one_launch) {
        if (!ck::w4_skinny_fused_supports(M, K))
            return fail(CK_ERR_UNSUPPORTED, "%s: the one-launch MFMA form takes 1 <= M <= 8 and K <= 4096 "
                        "(M=%lld, K=%lld)", fn, (long long)M, (long long)K);
        plan.fused = plan.mfma_fused = true;
        plan.used = 0;
    }
    if (!plan.fused && plan.path == GemmPath::kTiled)
        CK_TRY(check_tiles(fn, M, w.N));
    if (library_scratch) {
        if (plan.used > ck::static_scratch_bytes())
            return fail(CK_ERR_UNSUPPORTED, "%s: M = %lld, K = %lld needs %zu bytes of scratch; the "
                        "library's static scratch holds %zu", fn, (long long)M, (long long)K, plan.used,
                        ck::static_scratch_bytes());
        ws = nullptr;
        if (plan.used > 0) {
            const int e = ck::static_scratch(stream, &ws);
            if (e != 0)
                return fail(CK_ERR_HIP, "%s: static scratch unavailable on this device or stream "
                            "(hipError_t %d)", fn, e);
        }
    } else if (!force_mfma_one_launch) {
        // The size asked of the caller does not depend on the path taken.
        const size_t need = workspace_bytes(M, K);
        if (!ws || ws_bytes < need)
            return fail(CK_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu%s)", fn, need, ws_bytes,
                        ws ? "" : ", NULL");
        if (!aligned(ws, kWsAlign))
            return fail(CK_ERR_WORKSPACE, "%s: workspace must be %zu-byte aligned", fn, kWsAlign);
        const Range rw = span(ws, 1, (int64_t)need, (int64_t)need, 1);
        if (overlap(ro, rw))
            return fail(CK_ERR_INVALID_ARG, "%s: output overlaps the workspace", fn);
        if (overlap(rw, rx) || overlap(rw, span(w.packed, w.N, K / 2, w.ldw, 1)) ||
            overlap(rw, scales_span(w, K)) || overlap(rw, span(bias, 1, w.N, w.N, 2)))
            return fail(CK_ERR_WORKSPACE, "%s: workspace overlaps an input", fn);
    }

    const int qmax = bits == 8 ? 127 : 7;
    if (plan.fused) {
        // Decode shapes: one launch that rotates, quantises and multiplies.
        const auto launch = plan.mfma_fused ? ck::launch_w4_skinny_fused : ck::launch_w4_gemv_fused;
        const int e = launch(x, ldx, G, qmax, (int)M, (int)K, w.packed, w.ldw, w.scales, w.kind == CK_WS_PER_GROUP,
                             (int)w.N, bias, x_scale, out, ldo, stream);
        return hip_status(e, fn);
    }
    int8_t *codes = static_cast<int8_t *>(ws);
    float *rs = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + plan.scales_off);
    const ck::CodesLayout layout = plan.a4      ? ck::CodesLayout::kPacked4
                                   : plan.tiled ? ck::CodesLayout::kTiled16
                                                : ck::CodesLayout::kRowMajor;
    const int e = ck::launch_rotate_quant(x, M, (int)K, ldx, G, qmax, codes, plan.ldq, rs, nullptr, 0,
                                          layout, stream);
    if (e != 0)
        return hip_status(e, fn);
    return run_gemm(fn, codes, plan.ldq, rs, M, K, w, bias, x_scale, out, ldo, nullptr, 0, plan.a4, stream,
                    plan.tiled);
}

}  // namespace

namespace {

const char *status_str_impl(int status)
{
    switch (status) {
    case CK_OK: return "CK_OK";
    case CK_ERR_INVALID_ARG: return "CK_ERR_INVALID_ARG";
    case CK_ERR_UNSUPPORTED: return "CK_ERR_UNSUPPORTED";
    case CK_ERR_WORKSPACE: return "CK_ERR_WORKSPACE";
    case CK_ERR_HIP: return "CK_ERR_HIP";
    default: return "CK_ERR_UNKNOWN";
    }
}

int ck_rotate_quant_impl(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G, int32_t bits,
                    int8_t *codes, int64_t ldq, float *row_scales, void *stream)
{
    const char *fn = "ck_rotate_quant";
    CK_TRY(check_m(fn, M));
    CK_TRY(check_k(fn, K));
    CK_TRY(check_g(fn, G, K));
    if (bits != 8 && bits != 4)
        return fail(CK_ERR_UNSUPPORTED, "%s: bits must be 8 or 4 (got %d)", fn, bits);
    if (M == 0)
        return ok();
    CK_TRY(check_x(fn, x, K, ldx));
    CK_TRY(check_codes(fn, codes, K, ldq));
    if (!row_scales || !aligned(row_scales, 4))
        return fail(CK_ERR_INVALID_ARG, "%s: row_scales must be a non-NULL 4-byte aligned pointer", fn);
    const Range rx = span(x, M, K, ldx, 2);
    if (overlap(rx, span(codes, M, K, ldq, 1)) || overlap(rx, span(row_scales, 1, M, M, 4)) ||
        overlap(span(codes, M, K, ldq, 1), span(row_scales, 1, M, M, 4)))
        return fail(CK_ERR_INVALID_ARG, "%s: codes, row_scales and x must not overlap", fn);
    const int e = ck::launch_rotate_quant(x, M, (int)K, ldx, G, bits == 8 ? 127 : 7, codes, ldq,
                                          row_scales, nullptr, 0, ck::CodesLayout::kRowMajor, stream);
    return hip_status(e, fn);
}

int ck_quantize_weights_impl(const uint16_t *w, int64_t N, int64_t K, int64_t ldw_in, int32_t G,
                        int32_t scale_kind, uint8_t *packed, int64_t ldp, uint16_t *scales, void *stream)
{
    const char *fn = "ck_quantize_weights";
    if (N < 0)
        return fail(CK_ERR_INVALID_ARG, "%s: N must be >= 0 (got %lld)", fn, (long long)N);
    if (N > kMaxRows)
        return fail(CK_ERR_UNSUPPORTED, "%s: N above %lld", fn, (long long)kMaxRows);
    CK_TRY(check_k(fn, K));
    CK_TRY(check_g(fn, G, K));
    if (scale_kind != CK_WS_PER_CHANNEL && scale_kind != CK_WS_PER_GROUP)
        return fail(CK_ERR_INVALID_ARG, "%s: unknown weight-scale kind %d", fn, scale_kind);
    if (N == 0)
        return ok();
    if (!w || ldw_in < K || ldw_in % 8 != 0 || !aligned(w, 16))
        return fail(CK_ERR_INVALID_ARG, "%s: w must be non-NULL and 16-byte aligned with ldw_in >= K, "
                    "ldw_in %% 8 == 0", fn);
    if (!packed || ldp < K / 2 || ldp % 16 != 0 || !aligned(packed, 16))
        return fail(CK_ERR_INVALID_ARG, "%s: packed must be non-NULL and 16-byte aligned with ldp >= K/2, "
                    "ldp %% 16 == 0", fn);
    if (!scales || !aligned(scales, 2))
        return fail(CK_ERR_INVALID_ARG, "%s: scales must be a non-NULL 2-byte aligned pointer", fn);
    const bool pg = scale_kind == CK_WS_PER_GROUP;
    const Range rw = span(w, N, K, ldw_in, 2), rp = span(packed, N, K / 2, ldp, 1);
    const Range rs = pg ? span(scales, K / 64, N, N, 2) : span(scales, 1, N, N, 2);
    if (overlap(rw, rp) || overlap(rw, rs) || overlap(rp, rs))
        return fail(CK_ERR_INVALID_ARG, "%s: w, packed and scales must not overlap", fn);
    const int e = ck::launch_quantize_weights(w, N, (int)K, ldw_in, G, pg, packed, ldp, scales, stream);
    return hip_status(e, fn);
}

int ck_test_rotate_f32_impl(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G, float *xr,
                       int64_t ldr, void *stream)
{
    const char *fn = "ck_test_rotate_f32";
    CK_TRY(check_m(fn, M));
    CK_TRY(check_k(fn, K));
    CK_TRY(check_g(fn, G, K));
    if (M == 0)
        return ok();
    CK_TRY(check_x(fn, x, K, ldx));
    if (!xr || ldr < K || ldr % 4 != 0 || !aligned(xr, 16))
        return fail(CK_ERR_INVALID_ARG, "%s: xr must be 16-byte aligned with ldr >= K, ldr %% 4 == 0", fn);
    if (overlap(span(x, M, K, ldx, 2), span(xr, M, K, ldr, 4)))
        return fail(CK_ERR_INVALID_ARG, "%s: xr overlaps x", fn);
    const int e = ck::launch_rotate_quant(x, M, (int)K, ldx, G, 127, nullptr, 0, nullptr, xr, ldr,
                                          ck::CodesLayout::kRowMajor, stream);
    return hip_status(e, fn);
}

int ck_rotate_quant_packed4_impl(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G,
                                 uint8_t *codes4, int64_t ldq, float *row_scales, void *stream)
{
    const char *fn = "ck_rotate_quant_packed4";
    CK_TRY(check_m(fn, M));
    CK_TRY(check_k(fn, K));
    CK_TRY(check_g(fn, G, K));
    if (M == 0)
        return ok();
    CK_TRY(check_x(fn, x, K, ldx));
    CK_TRY(check_codes(fn, codes4, K / 2, ldq));
    if (!row_scales || !aligned(row_scales, 4))
        return fail(CK_ERR_INVALID_ARG, "%s: row_scales must be a non-NULL 4-byte aligned pointer", fn);
    const Range rx = span(x, M, K, ldx, 2), rc = span(codes4, M, K / 2, ldq, 1);
    const Range rr = span(row_scales, 1, M, M, 4);
    if (overlap(rx, rc) || overlap(rx, rr) || overlap(rc, rr))
        return fail(CK_ERR_INVALID_ARG, "%s: codes4, row_scales and x must not overlap", fn);
    const int e = ck::launch_rotate_quant(x, M, (int)K, ldx, G, 7, reinterpret_cast<int8_t *>(codes4),
                                          ldq, row_scales, nullptr, 0, ck::CodesLayout::kPacked4, stream);
    return hip_status(e, fn);
}

int ck_w4_gemm_q_impl(const int8_t *codes, int64_t ldq, const float *row_scales, int64_t M, int64_t K,
                 const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, int32_t scale_kind,
                 int32_t Gw, int64_t N, const uint16_t *bias, uint16_t *out, int64_t ldo, void *stream)
{
    const Weights w{packed, ldw, w_scales, scale_kind, Gw, N};
    return gemm_q_common("ck_w4_gemm_q", false, codes, ldq, row_scales, M, K, w, bias, out, ldo, stream);
}

int ck_w4a4_gemm_packed_impl(const uint8_t *codes4, int64_t ldq, const float *row_scales, int64_t M,
                        int64_t K, const uint8_t *packed, int64_t ldw, const uint16_t *w_scales,
                        int32_t scale_kind, int32_t Gw, int64_t N, const uint16_t *bias,
                        uint16_t *out, int64_t ldo, void *stream)
{
    const char *fn = "ck_w4a4_gemm_packed";
    const Weights w{packed, ldw, w_scales, scale_kind, Gw, N};
    CK_TRY(check_m(fn, M));
    CK_TRY(check_k(fn, K));
    CK_TRY(check_weights(fn, w, K, true));
    if (M == 0)
        return ok();
    CK_TRY(check_codes(fn, codes4, K / 2, ldq));
    if (!row_scales || !aligned(row_scales, 4))
        return fail(CK_ERR_INVALID_ARG, "%s: row_scales must be a non-NULL 4-byte aligned pointer", fn);
    if (bias && !aligned(bias, 2))
        return fail(CK_ERR_INVALID_ARG, "%s: bias must be 2-byte aligned", fn);
    CK_TRY(check_out(fn, out, N, ldo, 2));
    const Range ro = span(out, M, N, ldo, 2);
    if (overlap(ro, span(codes4, M, K / 2, ldq, 1)) || overlap(ro, span(row_scales, 1, M, M, 4)) ||
        overlap(ro, span(packed, N, K / 2, ldw, 1)) || overlap(ro, scales_span(w, K)) ||
        overlap(ro, span(bias, 1, N, N, 2)))
        return fail(CK_ERR_INVALID_ARG, "%s: output overlaps an input", fn);
    return run_gemm(fn, codes4, ldq, row_scales, M, K, w, bias, 1.0f, out, ldo, nullptr, 0, true, stream);
}

int ck_w4_gemv_impl(const int8_t *codes, int64_t ldq, const float *row_scales, int64_t M, int64_t K,
               const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, int32_t scale_kind,
               int32_t Gw, int64_t N, const uint16_t *bias, uint16_t *out, int64_t ldo, void *stream)
{
    const Weights w{packed, ldw, w_scales, scale_kind, Gw, N};
    return gemm_q_common("ck_w4_gemv", true, codes, ldq, row_scales, M, K, w, bias, out, ldo, stream);
}

int ck_w4a8_linear_impl(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G,
                   const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, int32_t scale_kind,
                   int32_t Gw, int64_t N, const uint16_t *bias, float x_scale, uint16_t *out,
                   int64_t ldo, void *ws, size_t ws_bytes, void *stream)
{
    const Weights w{packed, ldw, w_scales, scale_kind, Gw, N};
    return linear_common("ck_w4a8_linear", 8, x, M, K, ldx, G, w, bias, x_scale, out, ldo, ws,
                         ws_bytes, stream);
}

int ck_w4a4_linear_impl(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G,
                   const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, int32_t scale_kind,
                   int32_t Gw, int64_t N, const uint16_t *bias, float x_scale, uint16_t *out,
                   int64_t ldo, void *ws, size_t ws_bytes, void *stream)
{
    const Weights w{packed, ldw, w_scales, scale_kind, Gw, N};
    return linear_common("ck_w4a4_linear", 4, x, M, K, ldx, G, w, bias, x_scale, out, ldo, ws,
                         ws_bytes, stream);
}

int ck_test_linear_mfma_one_launch_impl(int32_t bits, const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                        int32_t G, const uint8_t *packed, int64_t ldw, const uint16_t *w_scales,
                                        int32_t scale_kind, int32_t Gw, int64_t N, const uint16_t *bias,
                                        float x_scale, uint16_t *out, int64_t ldo, void *stream)
{
    const char *fn = "ck_test_linear_mfma_one_launch";
    if (bits != 8 && bits != 4)
        return fail(CK_ERR_INVALID_ARG, "%s: bits must be 8 or 4 (got %d)", fn, bits);
    const Weights w{packed, ldw, w_scales, scale_kind, Gw, N};
    return linear_common(fn, bits, x, M, K, ldx, G, w, bias, x_scale, out, ldo, nullptr, 0, stream, false, true);
}

int ck_w4a4_linear_noalloc_impl(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G,
                                const uint8_t *packed, int64_t ldw, const uint16_t *w_scales,
                                int32_t scale_kind, int32_t Gw, int64_t N, const uint16_t *bias,
                                float x_scale, uint16_t *out, int64_t ldo, void *stream)
{
    const Weights w{packed, ldw, w_scales, scale_kind, Gw, N};
    return linear_common("ck_w4a4_linear_noalloc", 4, x, M, K, ldx, G, w, bias, x_scale, out, ldo,
                         nullptr, 0, stream, true);
}

int ck_w4a16_gemv_impl(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const uint8_t *packed,
                  int64_t ldw, const uint16_t *scales, const uint16_t *zeros, int32_t Gw, int64_t N,
                  const uint16_t *bias, uint16_t *out, int64_t ldo, void *stream)
{
    const char *fn = "ck_w4a16_gemv";
    CK_TRY(check_m(fn, M));
    CK_TRY(check_k(fn, K));
    const Weights w{packed, ldw, scales, CK_WS_PER_GROUP, Gw, N};
    CK_TRY(check_weights(fn, w, K, true));
    if (!aligned(scales, 16) || !zeros || !aligned(zeros, 16))
        return fail(CK_ERR_INVALID_ARG, "%s: scales and zeros must be non-NULL 16-byte aligned pointers", fn);
    if (M > 8 || !ck::w4a16_supports(K))
        return fail(CK_ERR_UNSUPPORTED, "%s: takes 1 <= M <= 8 and K <= 16384 (M=%lld, K=%lld)", fn,
                    (long long)M, (long long)K);
    if (M == 0)
        return ok();
    CK_TRY(check_x(fn, x, K, ldx));
    if (bias && !aligned(bias, 2))
        return fail(CK_ERR_INVALID_ARG, "%s: bias must be 2-byte aligned", fn);
    CK_TRY(check_out(fn, out, N, ldo, 2));
    const Range ro = span(out, M, N, ldo, 2);
    if (overlap(ro, span(x, M, K, ldx, 2)) || overlap(ro, span(packed, N, K / 2, ldw, 1)) ||
        overlap(ro, span(scales, K / 64, N, N, 2)) || overlap(ro, span(zeros, K / 64, N, N, 2)) ||
        overlap(ro, span(bias, 1, N, N, 2)))
        return fail(CK_ERR_INVALID_ARG, "%s: output overlaps an input", fn);
    const int e = ck::launch_w4a16_gemv(x, (int)M, (int)K, ldx, packed, ldw, scales, zeros, (int)N,
                                        bias, out, ldo, stream);
    return hip_status(e, fn);
}

int ck_w4a16_gemm_impl(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const uint8_t *packed,
                  int64_t ldw, const uint16_t *scales, const uint16_t *zeros, int32_t Gw, int64_t N,
                  const uint16_t *bias, uint16_t *out, int64_t ldo, void *stream)
{
    const char *fn = "ck_w4a16_gemm";
    CK_TRY(check_m(fn, M));
    CK_TRY(check_k(fn, K));
    const Weights w{packed, ldw, scales, CK_WS_PER_GROUP, Gw, N};
    CK_TRY(check_weights(fn, w, K, true));
    if (!zeros || !aligned(zeros, 16))
        return fail(CK_ERR_INVALID_ARG, "%s: zeros must be a non-NULL 16-byte aligned pointer", fn);
    if (M == 0)
        return ok();
    CK_TRY(check_x(fn, x, K, ldx));
    if (ldx > kMaxLd / 2)
        return fail(CK_ERR_UNSUPPORTED, "%s: ldx (%lld) must be at most %lld elements", fn, (long long)ldx,
                    (long long)(kMaxLd / 2));
    if (bias && !aligned(bias, 2))
        return fail(CK_ERR_INVALID_ARG, "%s: bias must be 2-byte aligned", fn);
    CK_TRY(check_out(fn, out, N, ldo, 2));
    CK_TRY(check_tiles(fn, M, N));
    const Range ro = span(out, M, N, ldo, 2);
    if (overlap(ro, span(x, M, K, ldx, 2)) || overlap(ro, span(packed, N, K / 2, ldw, 1)) ||
        overlap(ro, span(scales, K / 64, N, N, 2)) || overlap(ro, span(zeros, K / 64, N, N, 2)) ||
        overlap(ro, span(bias, 1, N, N, 2)))
        return fail(CK_ERR_INVALID_ARG, "%s: output overlaps an input", fn);
    const int e = ck::launch_awq_gemm(x, (int)M, (int)K, ldx, packed, ldw, scales, zeros, (int)N, bias, out,
                                      ldo, stream);
    return hip_status(e, fn);
}

int ck_test_gemm_i32_impl(const int8_t *codes, int64_t ldq, int64_t M, int64_t K, const uint8_t *packed,
                     int64_t ldw, int64_t N, int32_t *acc, int64_t lda, void *stream)
{
    const char *fn = "ck_test_gemm_i32";
    CK_TRY(check_m(fn, M));
    CK_TRY(check_k(fn, K));
    const Weights w{packed, ldw, nullptr, CK_WS_PER_CHANNEL, 64, N};
    CK_TRY(check_weights(fn, w, K, false));
    if (M == 0)
        return ok();
    CK_TRY(check_codes(fn, codes, K, ldq));
    CK_TRY(check_out(fn, acc, N, lda, 4));
    const Range ra = span(acc, M, N, lda, 4);
    if (overlap(ra, span(codes, M, K, ldq, 1)) || overlap(ra, span(packed, N, K / 2, ldw, 1)))
        return fail(CK_ERR_INVALID_ARG, "%s: acc overlaps an input", fn);
    return run_gemm(fn, codes, ldq, nullptr, M, K, w, nullptr, 1.0f, nullptr, 0, acc, lda, false, stream);
}

int ck_test_gemm_i32_a4_impl(const uint8_t *codes4, int64_t ldq, int64_t M, int64_t K,
                        const uint8_t *packed, int64_t ldw, int64_t N, int32_t *acc, int64_t lda,
                        void *stream)
{
    const char *fn = "ck_test_gemm_i32_a4";
    CK_TRY(check_m(fn, M));
    CK_TRY(check_k(fn, K));
    const Weights w{packed, ldw, nullptr, CK_WS_PER_CHANNEL, 64, N};
    CK_TRY(check_weights(fn, w, K, false));
    if (M == 0)
        return ok();
    CK_TRY(check_codes(fn, codes4, K / 2, ldq));
    CK_TRY(check_out(fn, acc, N, lda, 4));
    const Range ra = span(acc, M, N, lda, 4);
    if (overlap(ra, span(codes4, M, K / 2, ldq, 1)) || overlap(ra, span(packed, N, K / 2, ldw, 1)))
        return fail(CK_ERR_INVALID_ARG, "%s: acc overlaps an input", fn);
    return run_gemm(fn, codes4, ldq, nullptr, M, K, w, nullptr, 1.0f, nullptr, 0, acc, lda, true, stream);
}

}  // namespace

extern "C" {

const char *ck_status_str(ck_status status) { return status_str_impl(status); }

const char *ck_last_error_msg(void) { return g_last_error.c_str(); }

const char *ck_version(void) { return "ck 0.2 gfx950"; }

size_t ck_linear_workspace_bytes(int64_t M, int64_t K, int64_t N)
{
    (void)N;  // the codes and row scales do not depend on N
    return workspace_bytes(M, K);
}

ck_status ck_rotate_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G, int32_t
                          bits, int8_t *codes, int64_t ldq, float *row_scales, void *stream)
{
    return static_cast<ck_status>(ck_rotate_quant_impl(x, M, K, ldx, G, bits, codes, ldq,
            row_scales, stream));
}

ck_status ck_quantize_weights(const uint16_t *w, int64_t N, int64_t K, int64_t ldw_in, int32_t G,
                              int32_t scale_kind, uint8_t *packed, int64_t ldp, uint16_t *scales,
                              void *stream)
{
    return static_cast<ck_status>(ck_quantize_weights_impl(w, N, K, ldw_in, G, scale_kind, packed,
            ldp, scales, stream));
}

ck_status ck_test_linear_mfma_one_launch(int32_t bits, const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                         int32_t G, const uint8_t *packed, int64_t ldw, const uint16_t *w_scales,
                                         int32_t scale_kind, int32_t Gw, int64_t N, const uint16_t *bias,
                                         float x_scale, uint16_t *out, int64_t ldo, void *stream)
{
    return static_cast<ck_status>(ck_test_linear_mfma_one_launch_impl(bits, x, M, K, ldx, G, packed, ldw, w_scales,
                                                                      scale_kind, Gw, N, bias, x_scale, out, ldo,
                                                                      stream));
}

ck_status ck_test_rotate_f32(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G, float
                             *xr, int64_t ldr, void *stream)
{
    return static_cast<ck_status>(ck_test_rotate_f32_impl(x, M, K, ldx, G, xr, ldr, stream));
}

ck_status ck_rotate_quant_packed4(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G,
                                  uint8_t *codes4, int64_t ldq, float *row_scales, void *stream)
{
    return static_cast<ck_status>(ck_rotate_quant_packed4_impl(x, M, K, ldx, G, codes4, ldq,
            row_scales, stream));
}

ck_status ck_w4_gemm_q(const int8_t *codes, int64_t ldq, const float *row_scales, int64_t M, int64_t
                       K, const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, int32_t
                       scale_kind, int32_t Gw, int64_t N, const uint16_t *bias, uint16_t *out,
                       int64_t ldo, void *stream)
{
    return static_cast<ck_status>(ck_w4_gemm_q_impl(codes, ldq, row_scales, M, K, packed, ldw,
            w_scales, scale_kind, Gw, N, bias, out, ldo, stream));
}

ck_status ck_w4a4_gemm_packed(const uint8_t *codes4, int64_t ldq, const float *row_scales, int64_t
                              M, int64_t K, const uint8_t *packed, int64_t ldw, const uint16_t
                              *w_scales, int32_t scale_kind, int32_t Gw, int64_t N, const uint16_t
                              *bias, uint16_t *out, int64_t ldo, void *stream)
{
    return static_cast<ck_status>(ck_w4a4_gemm_packed_impl(codes4, ldq, row_scales, M, K, packed,
            ldw, w_scales, scale_kind, Gw, N, bias, out, ldo, stream));
}

ck_status ck_w4_gemv(const int8_t *codes, int64_t ldq, const float *row_scales, int64_t M, int64_t
                     K, const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, int32_t
                     scale_kind, int32_t Gw, int64_t N, const uint16_t *bias, uint16_t *out, int64_t
                     ldo, void *stream)
{
    return static_cast<ck_status>(ck_w4_gemv_impl(codes, ldq, row_scales, M, K, packed, ldw,
            w_scales, scale_kind, Gw, N, bias, out, ldo, stream));
}

ck_status ck_w4a8_linear(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G, const
                         uint8_t *packed, int64_t ldw, const uint16_t *w_scales, int32_t scale_kind,
                         int32_t Gw, int64_t N, const uint16_t *bias, float x_scale, uint16_t *out,
                         int64_t ldo, void *ws, size_t ws_bytes, void *stream)
{
    return static_cast<ck_status>(ck_w4a8_linear_impl(x, M, K, ldx, G, packed, ldw, w_scales,
            scale_kind, Gw, N, bias, x_scale, out, ldo, ws, ws_bytes, stream));
}

ck_status ck_w4a4_linear(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G, const
                         uint8_t *packed, int64_t ldw, const uint16_t *w_scales, int32_t scale_kind,
                         int32_t Gw, int64_t N, const uint16_t *bias, float x_scale, uint16_t *out,
                         int64_t ldo, void *ws, size_t ws_bytes, void *stream)
{
    return static_cast<ck_status>(ck_w4a4_linear_impl(x, M, K, ldx, G, packed, ldw, w_scales,
            scale_kind, Gw, N, bias, x_scale, out, ldo, ws, ws_bytes, stream));
}

ck_status ck_w4a16_gemv(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const uint8_t *packed,
                        int64_t ldw, const uint16_t *scales, const uint16_t *zeros, int32_t Gw,
                        int64_t N, const uint16_t *bias, uint16_t *out, int64_t ldo, void *stream)
{
    return static_cast<ck_status>(ck_w4a16_gemv_impl(x, M, K, ldx, packed, ldw, scales, zeros, Gw,
            N, bias, out, ldo, stream));
}

ck_status ck_w4a16_gemm(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const uint8_t *packed,
                        int64_t ldw, const uint16_t *scales, const uint16_t *zeros, int32_t Gw,
                        int64_t N, const uint16_t *bias, uint16_t *out, int64_t ldo, void *stream)
{
    return static_cast<ck_status>(ck_w4a16_gemm_impl(x, M, K, ldx, packed, ldw, scales, zeros, Gw,
            N, bias, out, ldo, stream));
}

ck_status ck_test_gemm_i32(const int8_t *codes, int64_t ldq, int64_t M, int64_t K, const uint8_t
                           *packed, int64_t ldw, int64_t N, int32_t *acc, int64_t lda, void *stream)
{
    return static_cast<ck_status>(ck_test_gemm_i32_impl(codes, ldq, M, K, packed, ldw, N, acc, lda,
            stream));
}

ck_status ck_test_gemm_i32_a4(const uint8_t *codes4, int64_t ldq, int64_t M, int64_t K, const
                              uint8_t *packed, int64_t ldw, int64_t N, int32_t *acc, int64_t lda,
                              void *stream)
{
    return static_cast<ck_status>(ck_test_gemm_i32_a4_impl(codes4, ldq, M, K, packed, ldw, N, acc,
            lda, stream));
}

ck_status ck_w4a4_linear_noalloc(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t G,
                                 const uint8_t *packed, int64_t ldw, const uint16_t *w_scales,
                                 int32_t scale_kind, int32_t Gw, int64_t N, const uint16_t *bias,
                                 float x_scale, uint16_t *out, int64_t ldo, void *stream)
{
    return static_cast<ck_status>(ck_w4a4_linear_noalloc_impl(x, M, K, ldx, G, packed, ldw, w_scales,
                                                               scale_kind, Gw, N, bias, x_scale, out,
                                                               ldo, stream));
}

}  // extern "C"
