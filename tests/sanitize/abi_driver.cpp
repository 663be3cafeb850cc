// Drives every entry point of the C ABI (ck_api.cpp) against the host
// stand-ins of stub_launch.cpp, under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Checks, for each entry point:
//  - the status of valid calls and of each class of invalid argument;
//  - which kernel a valid call reaches, with which codes layout, and that the
//    workspace (caller's or the library's static scratch) is carved inside
//    its documented size;
//  - that every buffer the launch touches stays inside an allocation of
//    exactly the size the entry point documents (ASan reports otherwise).
// Prints "abi driver: N checks, 0 failures" and exits 0 when all pass.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <limits>
#include <vector>

#include "../../include/ck.h"
#include "stub_launch.h"

namespace {

int g_checks = 0, g_failures = 0;

#define EXPECT(cond)                                                               \
    do {                                                                           \
        ++g_checks;                                                                \
        if (!(cond)) {                                                             \
            ++g_failures;                                                          \
            fprintf(stderr, "%s:%d: EXPECT(%s) failed; last error: %s\n", __FILE__, \
                    __LINE__, #cond, ck_last_error_msg());                         \
        }                                                                          \
    } while (0)

// Host buffers of an exact byte size (ASan red zones start at the last byte).
struct Pool {
    std::vector<void *> ptrs;
    template <class T>
    T *get(size_t bytes, size_t align = 256)
    {
        void *p = nullptr;
        if (align < sizeof(void *))
            align = sizeof(void *);
        if (posix_memalign(&p, align, bytes ? bytes : 1) != 0) {
            fprintf(stderr, "allocation of %zu bytes failed\n", bytes);
            exit(2);
        }
        ptrs.push_back(p);
        return static_cast<T *>(p);
    }
    ~Pool()
    {
        for (void *p : ptrs)
            free(p);
    }
};

// Bytes spanned by `rows` rows of `cols` elements of `esize` bytes, stride ld.
size_t rows_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t esize)
{
    return rows <= 0 ? 0 : (size_t)(((rows - 1) * ld + cols) * esize);
}

bool contains(const void *base, size_t bytes, const void *p)
{
    const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
    return q >= b && q < b + bytes;
}

// Packed weights [N, ldw] bytes, scales per channel [N] or per group [K/64, N].
struct W {
    uint8_t *packed;
    int64_t ldw;
    uint16_t *scales;
    int kind;
    int64_t N;
};

W make_weights(Pool &pool, int64_t N, int64_t K, int kind, int64_t pad = 16)
{
    W w;
    w.N = N;
    w.ldw = K / 2 + pad;
    w.kind = kind;
    w.packed = pool.get<uint8_t>(rows_bytes(N, K / 2, w.ldw, 1));
    w.scales = pool.get<uint16_t>((size_t)(kind == CK_WS_PER_GROUP ? K / 64 : 1) * N * 2);
    return w;
}

void test_status_strings()
{
    EXPECT(strcmp(ck_status_str(CK_OK), "CK_OK") == 0);
    EXPECT(strcmp(ck_status_str(CK_ERR_INVALID_ARG), "CK_ERR_INVALID_ARG") == 0);
    EXPECT(strcmp(ck_status_str(CK_ERR_UNSUPPORTED), "CK_ERR_UNSUPPORTED") == 0);
    EXPECT(strcmp(ck_status_str(CK_ERR_WORKSPACE), "CK_ERR_WORKSPACE") == 0);
    EXPECT(strcmp(ck_status_str(CK_ERR_HIP), "CK_ERR_HIP") == 0);
    EXPECT(strcmp(ck_status_str((ck_status)99), "CK_ERR_UNKNOWN") == 0);
    EXPECT(ck_version() && strstr(ck_version(), "gfx950"));
}

void test_workspace_bytes()
{
    EXPECT(ck_linear_workspace_bytes(0, 3840, 16) == 0);
    EXPECT(ck_linear_workspace_bytes(-3, 3840, 16) == 0);
    EXPECT(ck_linear_workspace_bytes(1, 64, 16) == 1024 + 256);         // codes padded to 16 rows
    EXPECT(ck_linear_workspace_bytes(300, 3840, 16) == 304 * 3840 + 1280);
    EXPECT(ck_linear_workspace_bytes(8192, 3840, 3840) == (size_t)8192 * 3840 + 32768);
}

void test_rotate_quant()
{
    Pool pool;
    const int64_t M = 3, K = 192, ldx = 200, ldq = 208;
    uint16_t *x = pool.get<uint16_t>(rows_bytes(M, K, ldx, 2));
    int8_t *codes = pool.get<int8_t>(rows_bytes(M, K, ldq, 1));
    float *rs = pool.get<float>(M * 4, 4);
    for (int bits : {8, 4}) {
        stub::reset();
        EXPECT(ck_rotate_quant(x, M, K, ldx, 64, bits, codes, ldq, rs, nullptr) == CK_OK);
        EXPECT(stub::calls == 1 && stub::last.kernel == stub::Kernel::kRotateQuant);
        EXPECT(stub::last.qmax == (bits == 8 ? 127 : 7) && !stub::last.packed4 && stub::last.G == 64);
        EXPECT(stub::last.codes == codes && stub::last.row_scales == rs && !stub::last.xr);
        EXPECT(ck_last_error_msg()[0] == '\0');
    }
    stub::reset();
    EXPECT(ck_rotate_quant(nullptr, 0, K, ldx, 64, 8, nullptr, ldq, nullptr, nullptr) == CK_OK);
    EXPECT(stub::calls == 0);
    EXPECT(ck_rotate_quant(x, -1, K, ldx, 64, 8, codes, ldq, rs, nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_rotate_quant(x, int64_t(1) << 22, K, ldx, 64, 8, codes, ldq, rs, nullptr) == CK_ERR_UNSUPPORTED);
    EXPECT(ck_rotate_quant(x, M, 100, ldx, 4, 8, codes, ldq, rs, nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_rotate_quant(x, M, 0, ldx, 64, 8, codes, ldq, rs, nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_rotate_quant(x, M, 32768 + 64, 32832, 64, 8, codes, 32832, rs, nullptr) == CK_ERR_UNSUPPORTED);
    EXPECT(ck_rotate_quant(x, M, K, ldx, 32, 8, codes, ldq, rs, nullptr) == CK_ERR_UNSUPPORTED);
    EXPECT(ck_rotate_quant(x, M, K, ldx, 256, 8, codes, ldq, rs, nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_rotate_quant(x, M, K, ldx, 64, 5, codes, ldq, rs, nullptr) == CK_ERR_UNSUPPORTED);
    EXPECT(ck_rotate_quant(x + 1, M, K, ldx, 64, 8, codes, ldq, rs, nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_rotate_quant(x, M, K, 196, 64, 8, codes, ldq, rs, nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_rotate_quant(x, M, K, ldx, 64, 8, codes, 200, rs, nullptr) == CK_ERR_INVALID_ARG);
    int8_t *codes_off = pool.get<int8_t>(rows_bytes(M, K, ldq, 1) + 16);
    EXPECT(ck_rotate_quant(x, M, K, ldx, 64, 8, codes_off + 16, ldq, rs, nullptr) == CK_OK);  // 16-B aligned
    EXPECT(ck_rotate_quant(x, M, K, ldx, 64, 8, codes_off + 8, ldq, rs, nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_rotate_quant(x, M, K, ldx, 64, 8, codes, ldq, nullptr, nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_rotate_quant(x, M, K, ldx, 64, 8, reinterpret_cast<int8_t *>(x), ldq, rs, nullptr) ==
           CK_ERR_INVALID_ARG);
    EXPECT(ck_rotate_quant(x, M, K, ldx, 64, 8, codes, ldq, reinterpret_cast<float *>(codes), nullptr) ==
           CK_ERR_INVALID_ARG);
    EXPECT(strstr(ck_last_error_msg(), "must not overlap"));
}

void test_rotate_quant_packed4_and_f32()
{
    Pool pool;
    const int64_t M = 5, K = 256, ldx = 256, ldq4 = 144, ldr = 260;
    uint16_t *x = pool.get<uint16_t>(rows_bytes(M, K, ldx, 2));
    uint8_t *c4 = pool.get<uint8_t>(rows_bytes(M, K / 2, ldq4, 1));
    float *rs = pool.get<float>(M * 4, 4);
    float *xr = pool.get<float>(rows_bytes(M, K, ldr, 4));
    for (int G : {16, 64, 256}) {
        stub::reset();
        EXPECT(ck_rotate_quant_packed4(x, M, K, ldx, G, c4, ldq4, rs, nullptr) == CK_OK);
        EXPECT(stub::last.kernel == stub::Kernel::kRotateQuant && stub::last.packed4 && stub::last.qmax == 7);
        EXPECT(stub::last.G == G && stub::last.ldq == ldq4);
        stub::reset();
        EXPECT(ck_test_rotate_f32(x, M, K, ldx, G, xr, ldr, nullptr) == CK_OK);
        EXPECT(stub::last.kernel == stub::Kernel::kRotateQuant && stub::last.xr == xr && !stub::last.codes);
    }
    EXPECT(ck_rotate_quant_packed4(x, M, K, ldx, 64, c4, 112, rs, nullptr) == CK_ERR_INVALID_ARG);  // ldq % 16
    EXPECT(ck_rotate_quant_packed4(x, M, K, ldx, 64, c4, 96, rs, nullptr) == CK_ERR_INVALID_ARG);   // < K/2
    EXPECT(ck_rotate_quant_packed4(x, M, K, ldx, 64, c4, ldq4, reinterpret_cast<float *>(c4), nullptr) ==
           CK_ERR_INVALID_ARG);
    EXPECT(ck_test_rotate_f32(x, M, K, ldx, 64, xr, 258, nullptr) == CK_ERR_INVALID_ARG);  // ldr % 4
    EXPECT(ck_test_rotate_f32(x, M, K, ldx, 64, xr + 1, ldr, nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_test_rotate_f32(x, M, K, ldx, 64, reinterpret_cast<float *>(x), ldr, nullptr) ==
           CK_ERR_INVALID_ARG);
}

void test_quantize_weights()
{
    Pool pool;
    const int64_t N = 48, K = 320, ldw_in = 328, ldp = 176;
    uint16_t *w = pool.get<uint16_t>(rows_bytes(N, K, ldw_in, 2));
    uint8_t *packed = pool.get<uint8_t>(rows_bytes(N, K / 2, ldp, 1));
    uint16_t *sc_pg = pool.get<uint16_t>((size_t)(K / 64) * N * 2, 2);
    uint16_t *sc_pc = pool.get<uint16_t>((size_t)N * 2, 2);
    stub::reset();
    EXPECT(ck_quantize_weights(w, N, K, ldw_in, 64, CK_WS_PER_GROUP, packed, ldp, sc_pg, nullptr) == CK_OK);
    EXPECT(stub::last.kernel == stub::Kernel::kQuantizeWeights && stub::last.per_group);
    EXPECT(ck_quantize_weights(w, N, K, ldw_in, 16, CK_WS_PER_CHANNEL, packed, ldp, sc_pc, nullptr) == CK_OK);
    EXPECT(!stub::last.per_group && stub::last.G == 16 && stub::calls == 2);
    EXPECT(ck_quantize_weights(nullptr, 0, K, ldw_in, 64, CK_WS_PER_GROUP, nullptr, ldp, nullptr, nullptr) ==
           CK_OK);
    EXPECT(stub::calls == 2);
    EXPECT(ck_quantize_weights(w, -1, K, ldw_in, 64, 0, packed, ldp, sc_pc, nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_quantize_weights(w, N, K, ldw_in, 64, 2, packed, ldp, sc_pc, nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_quantize_weights(w, N, K, ldw_in, 256, 0, packed, ldp, sc_pc, nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_quantize_weights(w, N, K, 324, 64, 0, packed, ldp, sc_pc, nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_quantize_weights(w, N, K, ldw_in, 64, 0, packed, 168, sc_pc, nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_quantize_weights(w, N, K, ldw_in, 64, 0, packed, ldp, reinterpret_cast<uint16_t *>(packed),
                               nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_quantize_weights(w, N, K, ldw_in, 64, 0, reinterpret_cast<uint8_t *>(w), ldp, sc_pc, nullptr) ==
           CK_ERR_INVALID_ARG);
}

stub::Kernel expected_kernel(int64_t M, int64_t K)
{
    // 1..5 rows: VALU GEMV; up to 64 rows: the few-row MFMA kernel while the
    // activations fit its registers; otherwise the tiled GEMM.  A GEMV-capable
    // shape the few-row kernel cannot take stays on the GEMV.
    const bool gemv = M >= 1 && M <= 8 && K <= 16384;
    const bool skinny = ck::w4_skinny_supports(M, K);
    if (gemv && (M <= 5 || !skinny))
        return stub::Kernel::kGemv;
    return skinny ? stub::Kernel::kSkinny : stub::Kernel::kGemm;
}

// The whole linear in one launch: the MFMA form for 5 to 8 rows, K <= 4096 and
// at least 8192 weight rows, else the VALU GEMV form (up to 4 rows).
stub::Kernel expected_fused(int64_t M, int64_t K, int64_t N)
{
    if (M >= 5 && M <= 8 && K >= 64 && K <= 4096 && K % 64 == 0 && N >= 8192)
        return stub::Kernel::kSkinnyFused;
    if (ck::w4_gemv_fused_supports(M, K))
        return stub::Kernel::kGemvFused;
    return stub::Kernel::kNone;
}

void test_gemm_dispatch()
{
    struct Case {
        int64_t M, K;
        stub::Kernel k;
    };
    const Case cases[] = {
        {1, 3840, stub::Kernel::kGemv},     {5, 3840, stub::Kernel::kGemv},
        {6, 3840, stub::Kernel::kSkinny},   {8, 10240, stub::Kernel::kGemv},
        {32, 3840, stub::Kernel::kSkinny},  {64, 3840, stub::Kernel::kSkinny},
        {65, 3840, stub::Kernel::kGemm},    {300, 3840, stub::Kernel::kGemm},
        {3, 32768, stub::Kernel::kGemm},    {6, 16384, stub::Kernel::kGemv},
        {8, 16384, stub::Kernel::kGemv},    {40, 16384, stub::Kernel::kGemm},
    };
    for (const Case &c : cases) {
        EXPECT(expected_kernel(c.M, c.K) == c.k);
        for (int kind : {CK_WS_PER_CHANNEL, CK_WS_PER_GROUP}) {
            Pool pool;
            const int64_t N = 48, ldq = c.K + 16, ldo = N + 8;
            const W w = make_weights(pool, N, c.K, kind);
            int8_t *codes = pool.get<int8_t>(rows_bytes(c.M, c.K, ldq, 1));
            float *rs = pool.get<float>(c.M * 4, 4);
            uint16_t *bias = pool.get<uint16_t>(N * 2, 2);
            uint16_t *out = pool.get<uint16_t>(rows_bytes(c.M, N, ldo, 2));
            stub::reset();
            EXPECT(ck_w4_gemm_q(codes, ldq, rs, c.M, c.K, w.packed, w.ldw, w.scales, kind, 64, N, bias, out,
                                ldo, nullptr) == CK_OK);
            EXPECT(stub::calls == 1 && stub::last.kernel == c.k && !stub::last.a4);
            EXPECT(stub::last.per_group == (kind == CK_WS_PER_GROUP) && stub::last.x_scale == 1.0f);
            EXPECT(stub::last.codes == codes && stub::last.out == out && !stub::last.acc);
            // The decode entry takes 1..8 rows and K <= 16384, on the same kernels.
            stub::reset();
            const ck_status st = ck_w4_gemv(codes, ldq, rs, c.M, c.K, w.packed, w.ldw, w.scales, kind, 64, N,
                                            bias, out, ldo, nullptr);
            if (c.M <= 8 && c.K <= 16384) {
                EXPECT(st == CK_OK && stub::last.kernel == c.k);
            } else {
                EXPECT(st == CK_ERR_UNSUPPORTED && stub::calls == 0);
            }
        }
        // The int32 test hook picks the kernel by M the same way.
        Pool pool;
        const int64_t N = 32, ldq = c.K, lda = N + 4;
        const W w = make_weights(pool, N, c.K, CK_WS_PER_CHANNEL, 0);
        int8_t *codes = pool.get<int8_t>(rows_bytes(c.M, c.K, ldq, 1));
        int32_t *acc = pool.get<int32_t>(rows_bytes(c.M, N, lda, 4));
        stub::reset();
        EXPECT(ck_test_gemm_i32(codes, ldq, c.M, c.K, w.packed, w.ldw, N, acc, lda, nullptr) == CK_OK);
        EXPECT(stub::last.kernel == c.k && stub::last.acc == acc && !stub::last.out);
    }
}

void test_gemm_invalid()
{
    Pool pool;
    const int64_t M = 4, K = 256, N = 32, ldq = 256, ldo = 32;
    const W w = make_weights(pool, N, K, CK_WS_PER_GROUP);
    int8_t *codes = pool.get<int8_t>(rows_bytes(M, K, ldq, 1));
    float *rs = pool.get<float>(M * 4, 4);
    uint16_t *out = pool.get<uint16_t>(rows_bytes(M, N, ldo, 2));
    auto gq = [&](const int8_t *c, int64_t m, int64_t k, const uint8_t *p, int64_t ldw, const uint16_t *s,
                  int kind, int gw, int64_t n, const uint16_t *b, uint16_t *o, int64_t lo) {
        return ck_w4_gemm_q(c, ldq, rs, m, k, p, ldw, s, kind, gw, n, b, o, lo, nullptr);
    };
    stub::reset();
    EXPECT(gq(codes, 0, K, w.packed, w.ldw, w.scales, 1, 64, N, nullptr, nullptr, ldo) == CK_OK);
    EXPECT(gq(codes, M, K, nullptr, w.ldw, w.scales, 1, 64, N, nullptr, out, ldo) == CK_ERR_INVALID_ARG);
    EXPECT(gq(codes, M, K, w.packed, w.ldw, w.scales, 1, 64, 40, nullptr, out, 40) == CK_ERR_UNSUPPORTED);
    EXPECT(gq(codes, M, K, w.packed, w.ldw, w.scales, 1, 64, 0, nullptr, out, ldo) == CK_ERR_INVALID_ARG);
    EXPECT(gq(codes, M, K, w.packed, 120, w.scales, 1, 64, N, nullptr, out, ldo) == CK_ERR_INVALID_ARG);
    EXPECT(gq(codes, M, K, w.packed, w.ldw, w.scales, 1, 32, N, nullptr, out, ldo) == CK_ERR_UNSUPPORTED);
    EXPECT(gq(codes, M, K, w.packed, w.ldw, w.scales, 3, 64, N, nullptr, out, ldo) == CK_ERR_INVALID_ARG);
    EXPECT(gq(codes, M, K, w.packed, w.ldw, w.scales + 1, 1, 64, N, nullptr, out, ldo) == CK_ERR_INVALID_ARG);
    EXPECT(gq(codes, M, K, w.packed, w.ldw, w.scales + 1, 0, 64, N, nullptr, out, ldo) == CK_OK);  // 2-B ok
    EXPECT(gq(codes, M, K, w.packed, w.ldw, nullptr, 1, 64, N, nullptr, out, ldo) == CK_ERR_INVALID_ARG);
    EXPECT(gq(codes, M, K, w.packed, w.ldw, w.scales, 1, 64, N, nullptr, out, 36) == CK_ERR_INVALID_ARG);
    EXPECT(gq(codes, M, K, w.packed, w.ldw, w.scales, 1, 64, N, nullptr, out + 4, ldo) == CK_ERR_INVALID_ARG);
    EXPECT(gq(codes, M, K, w.packed, w.ldw, w.scales, 1, 64, N, w.scales, out, ldo) == CK_OK);
    EXPECT(gq(codes, M, K, w.packed, w.ldw, w.scales, 1, 64, N, reinterpret_cast<uint16_t *>(w.packed) + 1,
              reinterpret_cast<uint16_t *>(w.packed), ldo) == CK_ERR_INVALID_ARG);
    EXPECT(gq(codes, M, K, w.packed, w.ldw, w.scales, 1, 64, N, nullptr, reinterpret_cast<uint16_t *>(codes),
              ldo) == CK_ERR_INVALID_ARG);
    EXPECT(strstr(ck_last_error_msg(), "overlaps"));
    EXPECT(ck_w4_gemm_q(codes, ldq, nullptr, M, K, w.packed, w.ldw, w.scales, 1, 64, N, nullptr, out, ldo,
                        nullptr) == CK_ERR_INVALID_ARG);
    EXPECT(ck_w4_gemv(codes, ldq, rs, 9, K, w.packed, w.ldw, w.scales, 1, 64, N, nullptr, out, ldo, nullptr) ==
           CK_ERR_UNSUPPORTED);
    // A row stride past what the tiled GEMM's 32-bit offsets address.
    EXPECT(ck_w4_gemm_q(codes, (int64_t(1) << 23) + 16, rs, M, K, w.packed, w.ldw, w.scales, 1, 64, N,
                        nullptr, out, ldo, nullptr) == CK_ERR_UNSUPPORTED);
    // ceil(M / 128) * ceil(N / 256) tiles beyond one launch: 2^14 x 2^14.  The call
    // returns before any launch, so the output is a bare address that nothing
    // dereferences, placed (2^45) away from the heap so that the overlap checks
    // over its 2^44-byte span pass and the tile check is the one that fails.
    const int64_t bigM = int64_t(1) << 21, bigN = (int64_t(1) << 22) - 16;
    uint16_t *far_out = reinterpret_cast<uint16_t *>(uintptr_t(1) << 45);
    EXPECT(ck_w4_gemm_q(codes, ldq, rs, bigM, K, w.packed, w.ldw, w.scales, 1, 64, bigN, nullptr, far_out, bigN,
                        nullptr) == CK_ERR_UNSUPPORTED);
    EXPECT(strstr(ck_last_error_msg(), "too large"));
    EXPECT(stub::calls == 2);
}

void test_gemm_packed()
{
    for (int64_t M : {1, 7, 64, 65, 200}) {
        Pool pool;
        const int64_t K = 512, N = 64, ldq = 272, ldo = 64, lda = 68;
        const W w = make_weights(pool, N, K, CK_WS_PER_CHANNEL);
        uint8_t *c4 = pool.get<uint8_t>(rows_bytes(M, K / 2, ldq, 1));
        float *rs = pool.get<float>(M * 4, 4);
        uint16_t *out = pool.get<uint16_t>(rows_bytes(M, N, ldo, 2));
        int32_t *acc = pool.get<int32_t>(rows_bytes(M, N, lda, 4));
        stub::reset();
        EXPECT(ck_w4a4_gemm_packed(c4, ldq, rs, M, K, w.packed, w.ldw, w.scales, 0, 64, N, nullptr, out, ldo,
                                   nullptr) == CK_OK);
        EXPECT(stub::last.kernel == stub::Kernel::kGemm && stub::last.a4 && stub::last.ldq == ldq);
        EXPECT(ck_test_gemm_i32_a4(c4, ldq, M, K, w.packed, w.ldw, N, acc, lda, nullptr) == CK_OK);
        EXPECT(stub::last.kernel == stub::Kernel::kGemm && stub::last.a4 && stub::last.acc == acc);
        EXPECT(ck_w4a4_gemm_packed(c4, 240, rs, M, K, w.packed, w.ldw, w.scales, 0, 64, N, nullptr, out, ldo,
                                   nullptr) == CK_ERR_INVALID_ARG);
        EXPECT(ck_test_gemm_i32_a4(c4, ldq, M, K, w.packed, w.ldw, N, reinterpret_cast<int32_t *>(c4), lda,
                                   nullptr) == CK_ERR_INVALID_ARG);
        EXPECT(stub::calls == 2);
    }
}

// The whole linear with a caller workspace of exactly ck_linear_workspace_bytes.
void test_linear()
{
    struct Case {
        int64_t M, K;
        int G;
    };
    const Case cases[] = {{1, 3840, 64}, {2, 3840, 16}, {3, 16384, 64}, {4, 8192, 256}, {4, 10240, 256}, {8, 3840, 64},
                          {32, 3840, 64}, {64, 1024, 16}, {65, 3840, 256}, {300, 640, 64}};
    for (const Case &c : cases) {
        for (int bits : {8, 4}) {
            Pool pool;
            const int64_t N = 64, ldx = c.K + 8, ldo = N;
            const W w = make_weights(pool, N, c.K, CK_WS_PER_GROUP);
            uint16_t *x = pool.get<uint16_t>(rows_bytes(c.M, c.K, ldx, 2));
            uint16_t *out = pool.get<uint16_t>(rows_bytes(c.M, N, ldo, 2));
            const size_t need = ck_linear_workspace_bytes(c.M, c.K, N);
            uint8_t *ws = pool.get<uint8_t>(need);
            auto lin = bits == 8 ? ck_w4a8_linear : ck_w4a4_linear;
            stub::reset();
            EXPECT(lin(x, c.M, c.K, ldx, c.G, w.packed, w.ldw, w.scales, 1, 64, N, nullptr, 0.5f, out, ldo, ws,
                       need, nullptr) == CK_OK);
            const stub::Kernel mm = expected_kernel(c.M, c.K);
            if (expected_fused(c.M, c.K, N) != stub::Kernel::kNone) {
                // Decode: one fused launch rotates, quantises and multiplies.
                EXPECT(stub::calls == 1 && stub::last.kernel == expected_fused(c.M, c.K, N));
                EXPECT(stub::last.G == c.G && stub::last.x == x && stub::last.qmax == (bits == 8 ? 127 : 7));
                EXPECT(stub::last.x_scale == 0.5f);
                continue;
            }
            EXPECT(stub::calls == 2);
            if (stub::calls != 2)
                continue;
            const stub::Call &rq = stub::log[0], &g = stub::log[1];
            const bool a4 = bits == 4 && mm == stub::Kernel::kGemm;
            const bool tiled = mm == stub::Kernel::kSkinny;
            EXPECT(rq.kernel == stub::Kernel::kRotateQuant && rq.G == c.G && rq.packed4 == a4);
            EXPECT(rq.tiled == tiled && g.tiled == tiled);
            EXPECT(rq.qmax == (bits == 8 ? 127 : 7) && rq.ldq == (a4 ? c.K / 2 : c.K));
            EXPECT(rq.codes == ws && contains(ws, need, rq.row_scales));
            EXPECT(reinterpret_cast<uintptr_t>(rq.row_scales) % 256 == 0);
            EXPECT(g.kernel == mm && g.a4 == a4 && g.codes == rq.codes && g.row_scales == rq.row_scales);
            EXPECT(g.ldq == rq.ldq && g.x_scale == 0.5f && g.out == out);
        }
    }
}

// Workgroup shapes of the one-launch decode linear: for every M, K, N and CU
// count, the row blocks are covered exactly once by the streaming waves, the
// rotation threads cover every 8-column chunk with a chunk count the kernel is
// instantiated for, the LDS holds the codes, and whether a shape exists
// depends on M and K alone (the linear decides before it knows the device).
void test_fused_gemv_shapes()
{
    for (int64_t M = 1; M <= 5; ++M)
        for (int64_t K = 64; K <= 16384 + 64; K += 64)
            for (int64_t N : {8, 16, 264, 3840, 10240, 18432, 65536})
                for (int ncu : {1, 80, 256, 304}) {
                    ck::FusedGemvShape sh;
                    const bool ok = ck::w4_gemv_fused_shape(M, K, N, ncu, sh);
                    EXPECT(ok == ck::w4_gemv_fused_supports(M, K));
                    // with one row block per workgroup: M * cpr <= 8 chunks of 8 per rotation thread
                    const int64_t s = (K + 2047) / 2048, nch = K / 8;
                    const int64_t nwr1 = std::min<int64_t>((16 - s) / 4 * 4, (nch + 63) / 64);
                    const int64_t c1 = (nch + 64 * nwr1 - 1) / (64 * nwr1);
                    const int64_t cpr1 = c1 <= 1 ? 1 : c1 <= 2 ? 2 : c1 <= 4 ? 4 : 8;
                    EXPECT(ok == (M <= 4 && K <= 16384 && M * cpr1 <= 8));
                    if (!ok)
                        continue;
                    const int64_t nrb = N / 8;
                    EXPECT(sh.s == s && sh.rb >= 1 && sh.nws == sh.rb * sh.s && sh.nws <= 12);
                    EXPECT((int64_t)sh.nb * sh.rb >= nrb && (int64_t)(sh.nb - 1) * sh.rb < nrb);
                    EXPECT(sh.nwr >= 1 && sh.nws + sh.nwr <= 16 && (sh.nwr % 4 == 0 || sh.nwr * 64 >= nch));
                    EXPECT(sh.cpr == 1 || sh.cpr == 2 || sh.cpr == 4 || sh.cpr == 8);
                    EXPECT((int64_t)sh.cpr * 64 * sh.nwr >= nch && M * sh.cpr <= ck::kFusedMaxChunks);
                    EXPECT(sh.lds >= M * K && sh.lds <= 160 * 1024);
                    EXPECT(sh.nb > ncu || sh.lds > 80 * 1024);
                }
    // The decode workloads: M = 1 .. 4 at K = 3840 fuse, with five 8-row blocks
    // per workgroup on 256 CUs at N = 10240.
    ck::FusedGemvShape sh;
    EXPECT(ck::w4_gemv_fused_shape(1, 3840, 10240, 256, sh) && sh.nb == 256 && sh.rb == 5 && sh.nwr == 4);
    EXPECT(ck::w4_gemv_fused_supports(4, 3840) && ck::w4_gemv_fused_supports(2, 16384));
    EXPECT(!ck::w4_gemv_fused_supports(3, 16384) && !ck::w4_gemv_fused_supports(5, 64));
}

// The one-launch MFMA linear: its workgroup shapes (one workgroup per CU,
// every LDS byte inside the CU, the rows of N covered once), the linear's own
// choice of it (5 to 8 rows, N >= 8192), and its test entry point for any N.
void test_mfma_one_launch()
{
    for (int64_t M = 1; M <= 9; ++M)
        for (int64_t K = 64; K <= 4096 + 64; K += 64)
            for (int64_t N : {16, 48, 3840, 4112, 10240, 16384, 65536})
                for (int ncu : {1, 80, 256}) {
                    ck::SkinnyFusedShape sh;
                    const bool ok = ck::w4_skinny_fused_shape(M, K, N, ncu, sh);
                    EXPECT(ok == (M <= 8 && K <= 4096));
                    EXPECT(ok == ck::w4_skinny_fused_supports(M, K));
                    if (!ok)
                        continue;
                    const int64_t s = (K / 64 + 31) / 32;
                    EXPECT(sh.s == s && sh.rows % 8 == 0 && sh.rows >= 8 && sh.t == (sh.rows + 15) / 16);
                    EXPECT(sh.nws == sh.t * sh.s && sh.nws + ck::kSfRotWaves <= 16);
                    EXPECT((int64_t)sh.nb * sh.rows >= N && (int64_t)(sh.nb - 1) * sh.rows < N);
                    const int64_t need = (int64_t)sh.nws * (16 * ck::kSfSlicePitch + 4 * ck::kSfScaleDwords + 2048) +
                                        ck::kSfCodeGroup * 32 * s;
                    EXPECT(sh.lds >= need && sh.lds <= ck::kSfMaxLds);
                    EXPECT(sh.nb > ncu || sh.lds > 80 * 1024);
                }
    // N = 10240 on 256 CUs: 40 rows (two tiles and a half tile) per workgroup.
    ck::SkinnyFusedShape sh;
    EXPECT(ck::w4_skinny_fused_shape(8, 3840, 10240, 256, sh) && sh.nb == 256 && sh.rows == 40 && sh.nws == 6);
    for (int64_t M : {4, 5, 6, 8})
        for (int64_t N : {8176, 8192}) {
            Pool pool;
            const int64_t K = 3840, ldx = K, ldo = N;
            const W w = make_weights(pool, N, K, CK_WS_PER_GROUP);
            uint16_t *x = pool.get<uint16_t>(rows_bytes(M, K, ldx, 2));
            uint16_t *out = pool.get<uint16_t>(rows_bytes(M, N, ldo, 2));
            const size_t need = ck_linear_workspace_bytes(M, K, N);
            uint8_t *ws = pool.get<uint8_t>(need);
            stub::reset();
            EXPECT(ck_w4a8_linear(x, M, K, ldx, 64, w.packed, w.ldw, w.scales, 1, 64, N, nullptr, 1.f, out, ldo,
                                  ws, need, nullptr) == CK_OK);
            // 4 rows: the VALU one-launch form; 5 to 8 rows and N >= 8192: the MFMA one;
            // otherwise two launches.
            const stub::Kernel one = M >= 5 && N >= 8192 ? stub::Kernel::kSkinnyFused
                                     : M <= 4            ? stub::Kernel::kGemvFused
                                                         : stub::Kernel::kNone;
            EXPECT(one == expected_fused(M, K, N));
            EXPECT(one != stub::Kernel::kNone ? stub::calls == 1 && stub::last.kernel == one
                                              : stub::calls == 2 && stub::last.kernel != stub::Kernel::kSkinnyFused);
        }
    {
        Pool pool;
        const int64_t M = 3, K = 256, N = 48;
        const W w = make_weights(pool, N, K, CK_WS_PER_CHANNEL);
        uint16_t *x = pool.get<uint16_t>(rows_bytes(8, 4160, 4160, 2));
        uint16_t *out = pool.get<uint16_t>(rows_bytes(9, N, N, 2));
        stub::reset();
        EXPECT(ck_test_linear_mfma_one_launch(4, x, M, K, K, 16, w.packed, w.ldw, w.scales, 0, 64, N, nullptr, 2.f,
                                              out, N, nullptr) == CK_OK);
        EXPECT(stub::calls == 1 && stub::last.kernel == stub::Kernel::kSkinnyFused && stub::last.qmax == 7 &&
               stub::last.G == 16 && stub::last.x_scale == 2.f);
        stub::reset();
        EXPECT(ck_test_linear_mfma_one_launch(5, x, M, K, K, 16, w.packed, w.ldw, w.scales, 0, 64, N, nullptr, 1.f,
                                              out, N, nullptr) == CK_ERR_INVALID_ARG);
        EXPECT(ck_test_linear_mfma_one_launch(8, x, 9, K, K, 16, w.packed, w.ldw, w.scales, 0, 64, N, nullptr, 1.f,
                                              out, N, nullptr) == CK_ERR_UNSUPPORTED);
        EXPECT(stub::calls == 0);
    }
}

void test_linear_invalid()
{
    Pool pool;
    const int64_t M = 40, K = 512, N = 32, ldx = 512, ldo = 32;
    const W w = make_weights(pool, N, K, CK_WS_PER_CHANNEL);
    uint16_t *x = pool.get<uint16_t>(rows_bytes(M, K, ldx, 2));
    uint16_t *out = pool.get<uint16_t>(rows_bytes(M, N, ldo, 2));
    const size_t need = ck_linear_workspace_bytes(M, K, N);
    uint8_t *ws = pool.get<uint8_t>(need + 256);
    auto lin = [&](const uint16_t *xx, int G, float xs, uint16_t *o, void *wsp, size_t wsb) {
        return ck_w4a4_linear(xx, M, K, ldx, G, w.packed, w.ldw, w.scales, 0, 64, N, nullptr, xs, o, ldo, wsp,
                              wsb, nullptr);
    };
    stub::reset();
    EXPECT(lin(x, 64, 1.f, out, ws, need - 1) == CK_ERR_WORKSPACE);
    EXPECT(lin(x, 64, 1.f, out, nullptr, need) == CK_ERR_WORKSPACE);
    EXPECT(lin(x, 64, 1.f, out, ws + 16, need) == CK_ERR_WORKSPACE);
    EXPECT(strstr(ck_last_error_msg(), "aligned"));
    EXPECT(lin(x, 64, 0.f, out, ws, need) == CK_ERR_INVALID_ARG);
    EXPECT(lin(x, 64, -2.f, out, ws, need) == CK_ERR_INVALID_ARG);
    EXPECT(lin(x, 64, std::numeric_limits<float>::infinity(), out, ws, need) == CK_ERR_INVALID_ARG);
    EXPECT(lin(x, 64, std::numeric_limits<float>::quiet_NaN(), out, ws, need) == CK_ERR_INVALID_ARG);
    EXPECT(lin(x, 256, 1.f, out, ws, need) == CK_OK);
    EXPECT(lin(x, 128, 1.f, out, ws, need) == CK_ERR_UNSUPPORTED);
    EXPECT(lin(x, 48, 1.f, out, ws, need) == CK_ERR_UNSUPPORTED);
    EXPECT(lin(x, 64, 1.f, reinterpret_cast<uint16_t *>(ws), ws, need) == CK_ERR_INVALID_ARG);
    EXPECT(lin(x, 64, 1.f, x, ws, need) == CK_ERR_INVALID_ARG);
    EXPECT(lin(x, 64, 1.f, out, reinterpret_cast<uint8_t *>(x), need) == CK_ERR_WORKSPACE);
    EXPECT(lin(x + 4, 64, 1.f, out, ws, need) == CK_ERR_INVALID_ARG);
    EXPECT(stub::calls == 2);
    // A launch failure is reported with the HIP error and stops the sequence.
    stub::reset();
    stub::next_status = 98;
    EXPECT(lin(x, 64, 1.f, out, ws, need) == CK_ERR_HIP);
    EXPECT(stub::calls == 1 && strstr(ck_last_error_msg(), "hipError_t 98"));
    // An error message is cleared by the next successful call.
    EXPECT(lin(x, 64, 1.f, out, ws, need) == CK_OK);
    EXPECT(ck_last_error_msg()[0] == '\0');
}

// The allocation-free linear: the same plan, carved from the library scratch.
void test_noalloc()
{
    struct Case {
        int64_t M, K;
        bool fits;
    };
    const Case cases[] = {{1, 3840, true},      {4, 3840, true},      {17, 3840, true},
                          {32, 3840, true},     {64, 32768, true},    {300, 3840, true},
                          {8192, 3840, true},   {8192, 16384, true},  {16384, 8192, true},
                          {8192, 16448, false}, {16448, 8192, false}};
    for (const Case &c : cases) {
        Pool pool;
        const int64_t N = 16, ldx = c.K, ldo = N;
        const W w = make_weights(pool, N, c.K, CK_WS_PER_CHANNEL, 0);
        uint16_t *x = pool.get<uint16_t>(rows_bytes(c.M, c.K, ldx, 2));
        uint16_t *out = pool.get<uint16_t>(rows_bytes(c.M, N, ldo, 2));
        stub::reset();
        const ck_status st = ck_w4a4_linear_noalloc(x, c.M, c.K, ldx, 64, w.packed, w.ldw, w.scales, 0, 64, N,
                                                    nullptr, 1.f, out, ldo, nullptr);
        if (!c.fits) {
            EXPECT(st == CK_ERR_UNSUPPORTED && stub::calls == 0);
            EXPECT(strstr(ck_last_error_msg(), "static scratch"));
            continue;
        }
        EXPECT(st == CK_OK);
        if (expected_fused(c.M, c.K, N) != stub::Kernel::kNone) {
            EXPECT(stub::calls == 1 && stub::last.kernel == expected_fused(c.M, c.K, N) && stub::last.G == 64);
            continue;
        }
        EXPECT(stub::calls == 2);
        if (stub::calls != 2)
            continue;
        const stub::Call &rq = stub::log[0], &g = stub::log[1];
        const void *base = stub::scratch_base();
        EXPECT(rq.codes == base && contains(base, ck::kStaticScratchBytes, rq.row_scales));
        const bool tiled = expected_kernel(c.M, c.K) == stub::Kernel::kGemm;
        EXPECT(rq.packed4 == tiled && g.a4 == tiled && g.codes == rq.codes && g.kernel == expected_kernel(c.M, c.K));
        EXPECT(rq.tiled == (g.kernel == stub::Kernel::kSkinny) && g.tiled == rq.tiled);
    }
}

void test_w4a16()
{
    Pool pool;
    const int64_t K = 384, N = 48, ldx = 392, ldo = 56;
    const W w = make_weights(pool, N, K, CK_WS_PER_GROUP);
    uint16_t *zeros = pool.get<uint16_t>((size_t)(K / 64) * N * 2);
    uint16_t *bias = pool.get<uint16_t>(N * 2, 2);
    for (int64_t M : {1, 3, 8}) {
        Pool p2;
        uint16_t *x = p2.get<uint16_t>(rows_bytes(M, K, ldx, 2));
        uint16_t *out = p2.get<uint16_t>(rows_bytes(M, N, ldo, 2));
        stub::reset();
        EXPECT(ck_w4a16_gemv(x, M, K, ldx, w.packed, w.ldw, w.scales, zeros, 64, N, bias, out, ldo, nullptr) ==
               CK_OK);
        EXPECT(stub::last.kernel == stub::Kernel::kW4a16Gemv && stub::last.M == M);
        EXPECT(ck_w4a16_gemv(x, M, K, ldx, w.packed, w.ldw, w.scales + 1, zeros, 64, N, bias, out, ldo,
                             nullptr) == CK_ERR_INVALID_ARG);
        EXPECT(ck_w4a16_gemv(x, M, K, ldx, w.packed, w.ldw, w.scales, nullptr, 64, N, bias, out, ldo,
                             nullptr) == CK_ERR_INVALID_ARG);
        EXPECT(ck_w4a16_gemv(x, M, K, ldx, w.packed, w.ldw, w.scales, zeros, 64, N, bias,
                             reinterpret_cast<uint16_t *>(zeros), N, nullptr) == CK_ERR_INVALID_ARG);
        EXPECT(stub::calls == 1);
    }
    for (int64_t M : {1, 9, 130}) {
        Pool p2;
        uint16_t *x = p2.get<uint16_t>(rows_bytes(M, K, ldx, 2));
        uint16_t *out = p2.get<uint16_t>(rows_bytes(M, N, ldo, 2));
        stub::reset();
        EXPECT(ck_w4a16_gemm(x, M, K, ldx, w.packed, w.ldw, w.scales, zeros, 64, N, bias, out, ldo, nullptr) ==
               CK_OK);
        EXPECT(stub::last.kernel == stub::Kernel::kAwqGemm && stub::last.M == M);
        EXPECT(ck_w4a16_gemm(x, M, K, ldx, w.packed, w.ldw, w.scales + 1, zeros, 64, N, bias, out, ldo,
                             nullptr) == CK_ERR_INVALID_ARG);
        EXPECT(ck_w4a16_gemm(x, M, K, ldx, w.packed, w.ldw, w.scales, zeros + 1, 64, N, bias, out, ldo,
                             nullptr) == CK_ERR_INVALID_ARG);
        EXPECT(ck_w4a16_gemm(x, M, K, ldx, w.packed, w.ldw, w.scales, nullptr, 64, N, bias, out, ldo,
                             nullptr) == CK_ERR_INVALID_ARG);
        EXPECT(ck_w4a16_gemm(x, M, K, ldx, w.packed, w.ldw, w.scales, zeros, 32, N, bias, out, ldo,
                             nullptr) == CK_ERR_UNSUPPORTED);
        EXPECT(stub::calls == 1);
    }
    uint16_t *x = pool.get<uint16_t>(rows_bytes(9, K, ldx, 2));
    uint16_t *out = pool.get<uint16_t>(rows_bytes(9, N, ldo, 2));
    EXPECT(ck_w4a16_gemv(x, 9, K, ldx, w.packed, w.ldw, w.scales, zeros, 64, N, bias, out, ldo, nullptr) ==
           CK_ERR_UNSUPPORTED);
    EXPECT(ck_w4a16_gemv(x, 0, K, ldx, w.packed, w.ldw, w.scales, zeros, 64, N, bias, out, ldo, nullptr) ==
           CK_OK);
}

}  // namespace

int main()
{
    test_status_strings();
    test_workspace_bytes();
    test_rotate_quant();
    test_rotate_quant_packed4_and_f32();
    test_quantize_weights();
    test_gemm_dispatch();
    test_gemm_invalid();
    test_gemm_packed();
    test_linear();
    test_fused_gemv_shapes();
    test_mfma_one_launch();
    test_linear_invalid();
    test_noalloc();
    test_w4a16();
    printf("abi driver: %d checks, %d failures\n", g_checks, g_failures);
    return g_failures == 0 ? 0 : 1;
}
