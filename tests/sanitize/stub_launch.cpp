// Host stand-ins for the kernel launchers of libck, so that the C ABI
// (ck_api.cpp) can be built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and driven without a GPU.
//
// Each stand-in records its arguments and then touches the first and the last
// element of every row that the real kernel reads or writes, with the layout
// the kernel assumes.  The driver allocates every host buffer at exactly the
// size its entry point documents, so a validation gap, a wrong stride or a
// workspace carved past its end shows up as a heap-buffer-overflow.
#include "stub_launch.h"

#include <cstdlib>
#include <cstring>

namespace stub {

Call last;
int next_status = 0;
int calls = 0;
std::vector<Call> log;

void reset()
{
    last = Call{};
    next_status = 0;
    calls = 0;
    log.clear();
}

namespace {

volatile uint8_t g_sink;

void read_rows(const void *p, int64_t rows, int64_t row_bytes, int64_t ld_bytes)
{
    if (!p || rows <= 0 || row_bytes <= 0)
        return;
    const uint8_t *b = static_cast<const uint8_t *>(p);
    for (int64_t r = 0; r < rows; ++r) {
        g_sink = b[r * ld_bytes];
        g_sink = b[r * ld_bytes + row_bytes - 1];
    }
}

void write_rows(void *p, int64_t rows, int64_t row_bytes, int64_t ld_bytes)
{
    if (!p || rows <= 0 || row_bytes <= 0)
        return;
    uint8_t *b = static_cast<uint8_t *>(p);
    for (int64_t r = 0; r < rows; ++r) {
        b[r * ld_bytes] = 0x5a;
        b[r * ld_bytes + row_bytes - 1] = 0xa5;
    }
}

// Per-channel scales are [N]; per-group ones [K/64, N].
void read_wscales(const uint16_t *s, bool per_group, int K, int N)
{
    read_rows(s, per_group ? K / 64 : 1, 2 * (int64_t)N, 2 * (int64_t)N);
}

int finish(Call c)
{
    last = c;
    log.push_back(c);
    ++calls;
    const int st = next_status;
    next_status = 0;
    return st;
}

// Shared by the three integer matmul kernels: codes (one byte each, or two
// per byte when a4), row scales, packed weights, weight scales, bias, and the
// bf16 output or the int32 accumulators.
void touch_matmul(const int8_t *codes, int64_t ldq, const float *rs, int M, int K, const uint8_t *packed,
                  int64_t ldw, const uint16_t *ws, bool pg, int N, const uint16_t *bias, uint16_t *out,
                  int64_t ldo, int32_t *acc, int64_t lda, bool a4)
{
    read_rows(codes, M, a4 ? K / 2 : K, ldq);
    read_rows(packed, N, K / 2, ldw);
    if (acc) {
        write_rows(acc, M, 4 * (int64_t)N, 4 * lda);
        return;
    }
    read_rows(rs, 1, 4 * (int64_t)M, 4 * (int64_t)M);
    read_wscales(ws, pg, K, N);
    read_rows(bias, 1, 2 * (int64_t)N, 2 * (int64_t)N);
    write_rows(out, M, 2 * (int64_t)N, 2 * ldo);
}

std::vector<uint8_t> g_scratch;

}  // namespace
}  // namespace stub

namespace ck {

int launch_rotate_quant(const uint16_t *x, int64_t M, int K, int64_t ldx, int G, int qmax, int8_t *codes,
                        int64_t ldq, float *row_scales, float *xr, int64_t ldr, CodesLayout layout, void *stream)
{
    using namespace stub;
    const bool packed4 = layout == CodesLayout::kPacked4, tiled = layout == CodesLayout::kTiled16;
    read_rows(x, M, 2 * (int64_t)K, 2 * ldx);
    if (tiled && codes) {
        // Row m: 16 bytes at 16 * (m % 16) of every 256-byte kb slot of its
        // tile's K / 64 blocks; first and last of them.
        for (int64_t m = 0; m < M; ++m) {
            int8_t *t = codes + (m / 16) * (int64_t)K * 16 + (m % 16) * 16;
            t[0] = 1;
            t[(K / 64 - 1) * 1024 + 3 * 256 + 15] = 1;
        }
    } else {
        write_rows(codes, M, packed4 ? K / 2 : K, ldq);
    }
    write_rows(row_scales, 1, 4 * M, 4 * M);
    write_rows(xr, M, 4 * (int64_t)K, 4 * ldr);
    Call c{};
    c.kernel = Kernel::kRotateQuant;
    c.M = M, c.K = K, c.G = G, c.qmax = qmax, c.ldq = ldq, c.packed4 = packed4, c.tiled = tiled;
    c.x = x, c.codes = codes, c.row_scales = row_scales, c.xr = xr, c.stream = stream;
    return finish(c);
}

int launch_awq_gemm(const uint16_t *x, int M, int K, int64_t ldx, const uint8_t *packed, int64_t ldw,
                    const uint16_t *scales, const uint16_t *zeros, int N, const uint16_t *bias, uint16_t *out,
                    int64_t ldo, void *stream)
{
    using namespace stub;
    read_rows(x, M, 2 * (int64_t)K, 2 * ldx);
    read_rows(packed, N, K / 2, ldw);
    read_wscales(scales, true, K, N);
    read_wscales(zeros, true, K, N);
    read_rows(bias, 1, 2 * (int64_t)N, 2 * (int64_t)N);
    write_rows(out, M, 2 * (int64_t)N, 2 * ldo);
    Call c{};
    c.kernel = Kernel::kAwqGemm;
    c.M = M, c.K = K, c.N = N, c.x = x, c.out = out, c.stream = stream;
    return finish(c);
}

int launch_quantize_weights(const uint16_t *w, int64_t N, int K, int64_t ldw_in, int G, bool per_group,
                            uint8_t *packed, int64_t ldp, uint16_t *scales, void *stream)
{
    using namespace stub;
    read_rows(w, N, 2 * (int64_t)K, 2 * ldw_in);
    write_rows(packed, N, K / 2, ldp);
    write_rows(scales, per_group ? K / 64 : 1, 2 * N, 2 * N);
    Call c{};
    c.kernel = Kernel::kQuantizeWeights;
    c.N = N, c.K = K, c.G = G, c.per_group = per_group, c.stream = stream;
    return finish(c);
}

int launch_w4_gemv(const int8_t *codes, int64_t ldq, const float *row_scales, int M, int K,
                   const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, bool per_group, int N,
                   const uint16_t *bias, float x_scale, uint16_t *out, int64_t ldo, int32_t *acc_out,
                   int64_t lda, void *stream)
{
    using namespace stub;
    touch_matmul(codes, ldq, row_scales, M, K, packed, ldw, w_scales, per_group, N, bias, out, ldo, acc_out,
                 lda, false);
    Call c{};
    c.kernel = Kernel::kGemv;
    c.M = M, c.K = K, c.N = N, c.ldq = ldq, c.per_group = per_group;
    c.x_scale = x_scale, c.codes = codes, c.row_scales = row_scales, c.out = out, c.acc = acc_out;
    c.stream = stream;
    return finish(c);
}

int launch_w4_gemv_fused(const uint16_t *x, int64_t ldx, int G, int qmax, int M, int K, const uint8_t *packed,
                         int64_t ldw, const uint16_t *w_scales, bool per_group, int N, const uint16_t *bias,
                         float x_scale, uint16_t *out, int64_t ldo, void *stream)
{
    using namespace stub;
    FusedGemvShape sh;
    if (!w4_gemv_fused_shape(M, K, N, 256, sh))
        return 1;  // hipErrorInvalidValue
    read_rows(x, M, 2 * (int64_t)K, 2 * ldx);
    touch_matmul(nullptr, 0, nullptr, M, K, packed, ldw, w_scales, per_group, N, bias, out, ldo, nullptr, 0,
                 false);
    Call c{};
    c.kernel = Kernel::kGemvFused;
    c.M = M, c.K = K, c.N = N, c.G = G, c.qmax = qmax, c.per_group = per_group;
    c.x_scale = x_scale, c.x = x, c.out = out, c.stream = stream;
    return finish(c);
}

int launch_w4_skinny_fused(const uint16_t *x, int64_t ldx, int G, int qmax, int M, int K, const uint8_t *packed,
                           int64_t ldw, const uint16_t *w_scales, bool per_group, int N, const uint16_t *bias,
                           float x_scale, uint16_t *out, int64_t ldo, void *stream)
{
    using namespace stub;
    SkinnyFusedShape sh;
    if (!w4_skinny_fused_shape(M, K, N, 256, sh))
        return 1;  // hipErrorInvalidValue
    read_rows(x, M, 2 * (int64_t)K, 2 * ldx);
    touch_matmul(nullptr, 0, nullptr, M, K, packed, ldw, w_scales, per_group, N, bias, out, ldo, nullptr, 0,
                 false);
    Call c{};
    c.kernel = Kernel::kSkinnyFused;
    c.M = M, c.K = K, c.N = N, c.G = G, c.qmax = qmax, c.per_group = per_group;
    c.x_scale = x_scale, c.x = x, c.out = out, c.stream = stream;
    return finish(c);
}

int launch_w4_skinny(const int8_t *codes, int64_t ldq, bool tiled, const float *row_scales, int M, int K,
                     const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, bool per_group, int N,
                     const uint16_t *bias, float x_scale, uint16_t *out, int64_t ldo, int32_t *acc_out,
                     int64_t lda, void *stream)
{
    using namespace stub;
    if (tiled) {
        // Whole 16-row tiles are read; in a partial last tile only the rows below M.
        for (int t = 0; t * 16 < M; ++t) {
            const int8_t *base = codes + (int64_t)t * K * 16;
            const int live = M - 16 * t < 16 ? M - 16 * t : 16;
            g_sink = base[0];
            g_sink = live == 16 ? base[(int64_t)K * 16 - 1] : base[(K / 64 - 1) * 1024 + 3 * 256 + (live - 1) * 16 + 15];
        }
        touch_matmul(nullptr, 0, row_scales, M, K, packed, ldw, w_scales, per_group, N, bias, out, ldo, acc_out,
                     lda, false);
    } else {
        touch_matmul(codes, ldq, row_scales, M, K, packed, ldw, w_scales, per_group, N, bias, out, ldo,
                     acc_out, lda, false);
    }
    Call c{};
    c.kernel = Kernel::kSkinny;
    c.M = M, c.K = K, c.N = N, c.ldq = ldq, c.tiled = tiled, c.per_group = per_group, c.x_scale = x_scale;
    c.codes = codes, c.row_scales = row_scales, c.out = out, c.acc = acc_out, c.stream = stream;
    return finish(c);
}

int launch_w4_gemm(const int8_t *codes, int64_t ldq, const float *row_scales, int M, int K,
                   const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, bool per_group, int N,
                   const uint16_t *bias, float x_scale, uint16_t *out, int64_t ldo, int32_t *acc_out,
                   int64_t lda, bool a4, void *stream)
{
    using namespace stub;
    touch_matmul(codes, ldq, row_scales, M, K, packed, ldw, w_scales, per_group, N, bias, out, ldo, acc_out,
                 lda, a4);
    Call c{};
    c.kernel = Kernel::kGemm;
    c.M = M, c.K = K, c.N = N, c.ldq = ldq, c.per_group = per_group, c.a4 = a4, c.x_scale = x_scale;
    c.codes = codes, c.row_scales = row_scales, c.out = out, c.acc = acc_out, c.stream = stream;
    return finish(c);
}

int launch_w4a16_gemv(const uint16_t *x, int M, int K, int64_t ldx, const uint8_t *packed, int64_t ldw,
                      const uint16_t *scales, const uint16_t *zeros, int N, const uint16_t *bias, uint16_t *out,
                      int64_t ldo, void *stream)
{
    using namespace stub;
    read_rows(x, M, 2 * (int64_t)K, 2 * ldx);
    read_rows(packed, N, K / 2, ldw);
    read_wscales(scales, true, K, N);
    read_wscales(zeros, true, K, N);
    read_rows(bias, 1, 2 * (int64_t)N, 2 * (int64_t)N);
    write_rows(out, M, 2 * (int64_t)N, 2 * ldo);
    Call c{};
    c.kernel = Kernel::kW4a16Gemv;
    c.M = M, c.K = K, c.N = N, c.x = x, c.out = out, c.stream = stream;
    return finish(c);
}

// The library's static scratch, as a host array of the same size.
size_t static_scratch_bytes() { return kStaticScratchBytes; }

int static_scratch(void *stream, void **ptr)
{
    (void)stream;
    if (stub::g_scratch.empty())
        stub::g_scratch.resize(kStaticScratchBytes);
    *ptr = stub::g_scratch.data();
    return 0;
}

}  // namespace ck

namespace stub {
const void *scratch_base() { return g_scratch.empty() ? nullptr : g_scratch.data(); }
}  // namespace stub
