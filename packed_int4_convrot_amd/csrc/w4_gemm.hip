// Tiled int8-MFMA GEMM for the ConvRot packed-INT4 linear at large M.
//
// acc[m,n] = sum_k codes[m,k] * (q[n,k] - 8) in int32, then the scale
// epilogue (row scale x per-channel or per-group weight scale, optional bias)
// and a bf16 store.  The integer matmul with a rowwise x weight-scale epilogue
// follows the W4A8 path of "[PR #182] HIP port of #176 ..." (description) and
// the W4A4/W4A8 ConvRot matmul of "feat: support packed INT4 convrot models"
// (summary); the difference is that the int4 weights are decoded in VGPRs
// right before CDNA4 int8 MFMA instead of being unpacked to memory.
//
// Tiling (block = WGM x WGN waves):
//   * block tile BM x BN = (WGM*WM*32) x (WGN*WN*32); MFMA K step 64 (one
//     weight-scale group); a stage holds KSUB K steps;
//   * v_mfma_i32_32x32x32_i8, each wave owns WM x WN 32x32 accumulator tiles;
//     the per-channel kernel runs 8 waves (two per SIMD) on a 256 x 256 tile;
//   * operands move global -> LDS directly (global_load_lds_dwordx4, no VGPR
//     staging) into two stage buffers.  A stage covers 128 bytes of every
//     operand row where it can (4 K steps of packed nibbles): the DMA's cost
//     on gfx950 grows with the number of distinct rows (cache lines) an
//     instruction touches far more than with its bytes, so 32-byte row
//     pieces per instruction ran the fill at a quarter of the rate;
//   * one barrier per stage.  Fragment reads run one K step ahead of the
//     MFMAs (two register sets), and the first step of the next stage is read
//     right after that barrier, so LDS latency is never waited on between
//     MFMAs; the DMA of stage t + 2 goes into the buffer that stage t has
//     just finished reading: all of it at that barrier, or for four-step
//     stages a quarter there and a quarter after each of the next stage's
//     first three K steps;
//   * the per-channel and int32 tiles run each K step in a fixed order: the
//     nibble decodes sit between the MFMA pairs, and the operands of the next
//     step's first MFMAs are decoded under this step's last ones, so the
//     matrix core never waits for a run of decode instructions (4-5% faster
//     at M = 8192 than the compiler's own order);
//   * LDS rows are unpadded; the 16-byte slots inside a row are XOR-swizzled
//     by row (swizzles measured conflict-free with SQ_LDS_BANK_CONFLICT for
//     these read patterns); the DMA writes lanes contiguously, so each lane
//     loads the global chunk that belongs in its slot;
//   * each lane reads one 16-byte weight fragment per K step (both 32-wide k
//     halves) and decodes it in VGPRs; int8 activation fragments are permuted
//     to the decode's even/odd k order as they are read;
//   * blocks are renumbered so that each XCD (blocks are dealt to the 8 XCDs
//     round-robin) gets a contiguous run of tiles that share activation rows.
// Operand layouts of v_mfma_i32_32x32x32_i8: lane l holds 16 int8 of row
// (A) / column (B) l % 32, k-half l / 32; D lane l register r holds
// D[8*(r/4) + 4*(l/32) + r%4][l % 32].  Lane half h and K-half s select
// activation chunk 2h + s (codes k in [32h + 16s, +16)) and weight bytes
// [16h + 8s, +8) of the row's 32 bytes, i.e. the same 16 k values.
//
// A4 variant (W4A4): the activation codes arrive packed two per byte like the
// weights ([M][K/2] bytes, two's complement nibbles in [-7, 7]), so the
// activation stage, its DMA and its LDS reads are half as large, and both
// operands are decoded to 16 * value: the accumulator carries a factor 256.
#include <type_traits>

#include "ck_device.h"
#include "launch.h"

namespace ck {
namespace {

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

// Slot swizzle of an LDS row of S 16-byte slots, for fragment reads in which
// 32 consecutive rows read one logical slot (lane half h in bit 0 of the
// slot).  Chosen by measuring SQ_LDS_BANK_CONFLICT on gfx950: 2 slots
// ((r >> 2) ^ (r >> 3)) & 1, 8 slots (r >> 1) & 7 read without conflicts
// (e.g. r & 7 gave 2-way conflicts).
template <int S>
__device__ __forceinline__ int swz(int r)
{
    static_assert(S == 2 || S == 4 || S == 8, "slot count");
    if constexpr (S == 2)
        return ((r >> 2) ^ (r >> 3)) & 1;
    else if constexpr (S == 4)
        return (r >> 2) & 3;
    else
        return (r >> 1) & 7;
}

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) leaving vmcnt alone.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

template <int WGM, int WGN, int WM, int WN, int KSUB, bool PER_GROUP, bool OUT_I32, bool A4>
__global__ __launch_bounds__(WGM * WGN * kWave) void w4_gemm_kernel(
    const int8_t *__restrict__ codes, int64_t ldq, const float *__restrict__ row_scales, int M,
    int K, const uint8_t *__restrict__ packed, int64_t ldw, const uint16_t *__restrict__ w_scales,
    int N, const uint16_t *__restrict__ bias, float x_scale, uint16_t *__restrict__ out,
    int64_t ldo, int32_t *__restrict__ acc_out, int64_t lda)
{
    // Per-channel and int32 results are computed transposed (weights as the
    // MFMA A operand), so that a lane holds one output row and four
    // consecutive columns per register group; the per-group form keeps one
    // column per lane, which is what its per-K-step scale needs.
    constexpr bool TRANS = !PER_GROUP;
    constexpr int NWAVES = WGM * WGN;
    constexpr int BM = WGM * WM * 32;
    constexpr int BN = WGN * WN * 32;
    constexpr int A_STEP = A4 ? 32 : 64;          // activation bytes per row and K step
    constexpr int A_ROW = A_STEP * KSUB;          // ... per row and stage
    constexpr int B_ROW = 32 * KSUB;
    constexpr int A_SLOTS = A_ROW / 16, B_SLOTS = B_ROW / 16;
    constexpr int A_BYTES = BM * A_ROW;
    constexpr int STAGE = A_BYTES + BN * B_ROW;
    // DMA per wave and stage: X_LD instructions of X_LANES lanes (a tile
    // smaller than 1 KiB per wave leaves lanes idle).
    constexpr int A_PER = A_BYTES / NWAVES, B_PER = BN * B_ROW / NWAVES;
    constexpr int A_LANES = A_PER >= 1024 ? kWave : A_PER / 16;
    constexpr int B_LANES = B_PER >= 1024 ? kWave : B_PER / 16;
    constexpr int A_LD = A_PER >= 1024 ? A_PER / 1024 : 1;
    constexpr int B_LD = B_PER >= 1024 ? B_PER / 1024 : 1;
    static_assert(A_LD * NWAVES * A_LANES * 16 == A_BYTES, "A DMA split");
    static_assert(B_LD * NWAVES * B_LANES * 16 == BN * B_ROW, "B DMA split");
    static_assert(KSUB % 2 == 0, "two fragment sets alternate across stages");
    // Accumulator factor of the decoded operands: 16 (weights) or 256 (both).
    constexpr int ACC_SHIFT = A4 ? 8 : 4;
    constexpr float ACC_SCALE = A4 ? 1.f / 256.f : 1.f / 16.f;
    constexpr int AQ = A4 ? 1 : 2;                // 16-byte activation fragments per tile and K step
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_generic[];
    lds_u8 *smem = (lds_u8 *)smem_generic;

    // XCD-aware renumbering of the block index, then a grouped raster: runs
    // of kGroupM tile rows are walked column by column, so the tiles an XCD
    // runs at the same time share a few activation and weight blocks (at
    // M = 8192, N = 3840, the 32 tiles of an XCD's first round read 4
    // activation and 8 weight blocks instead of 3 and 15).
    constexpr int kGroupM = 4;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    const int tile = xcd_block(blockIdx.x, tiles);
    const int group = tile / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int group_m = min(kGroupM, tiles_m - first_m);
    const int in_group = tile - group * kGroupM * tiles_n;
    const int m0 = (first_m + in_group % group_m) * BM;
    const int n0 = (in_group / group_m) * BN;

    const int t = threadIdx.x;
    const int wave = t / kWave, lane = t % kWave;
    const int wm = wave / WGN, wn = wave % WGN;
    const int l32 = lane % 32, h = lane / 32;
    const int ksteps = K / 64;
    const int nstages = (ksteps + KSUB - 1) / KSUB;
    const int arow_bytes = A4 ? K / 2 : K;         // valid bytes of a codes row

    // Logical slot of a row's 16-byte chunk g (K step g / (A_STEP / 16)):
    // int8 activation chunks 2h + s of a K step are stored as slot 2s + h so
    // that, like the packed rows, the lane half is bit 0 of the slot.
    auto a_slot = [](int g) {
        if constexpr (A4)
            return g;
        else
            return (g & ~3) | ((g & 1) << 1) | ((g >> 1) & 1);
    };

    // Global -> LDS for stage st into buffer b, through buffer resources that
    // span exactly the block's operand rows: a row past M / N or a chunk past
    // the end of the last row reads as zero, and such results are never used.
    // (MUBUF rather than global loads: a FLAT load into LDS still in flight
    // makes the compiler wait for every LDS read, not just the ones needed.)
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(codes + (int64_t)m0 * ldq), (short)0,
        (int)((int64_t)(min(M - m0, BM) - 1) * ldq + arow_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(packed + (int64_t)n0 * ldw), (short)0,
        (int)((int64_t)(min(N - n0, BN) - 1) * ldw + K / 2), 0x00020000);
    // Part p of NP equal parts of stage st's DMA into buffer b (NP = 1: all of it).
    auto issue_part = [&](int st, int b, int p, auto np_c) {
        constexpr int NP = decltype(np_c)::value;
        lds_u8 *sa = smem + b * STAGE;
#pragma unroll
        for (int jj = 0; jj < A_LD / NP; ++jj) {
            const int j = p * (A_LD / NP) + jj;
            const int q = (wave * A_LD + j) * A_LANES + lane;
            if (A_LANES == kWave || lane < A_LANES) {
                const int r = q / A_SLOTS;
                const int g = a_slot((q % A_SLOTS) ^ swz<A_SLOTS>(r));  // a_slot is an involution
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    a_rsrc, (__attribute__((address_space(3))) void *)(sa + (wave * A_LD + j) * A_LANES * 16), 16,
                    (int)(r * ldq) + st * A_ROW + 16 * g, 0, 0, 0);
            }
        }
#pragma unroll
        for (int jj = 0; jj < B_LD / NP; ++jj) {
            const int j = p * (B_LD / NP) + jj;
            const int q = (wave * B_LD + j) * B_LANES + lane;
            if (B_LANES == kWave || lane < B_LANES) {
                const int n = q / B_SLOTS;
                const int c = (q % B_SLOTS) ^ swz<B_SLOTS>(n);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    b_rsrc, (__attribute__((address_space(3))) void *)(sa + A_BYTES + (wave * B_LD + j) * B_LANES * 16), 16,
                    (int)(n * ldw) + st * B_ROW + 16 * c, 0, 0, 0);
            }
        }
    };
    auto issue_stage = [&](int st, int b) { issue_part(st, b, 0, std::integral_constant<int, 1>{}); };
    // The DMA of a four-step stage (packed codes, per-channel and int32
    // tiles) is issued in four parts, one per K step: a burst of LDS writes
    // then no longer meets every wave's first fragment reads of the stage at
    // once (about 1% faster at M = 8192).
    constexpr bool SPLIT = KSUB == 4 && TRANS && A_LD % KSUB == 0 && B_LD % KSUB == 0;
    constexpr int NPART = SPLIT ? KSUB : 1;

    // Fragments of one K step: weight row pieces and activation row pieces.
    struct Frag {
        u32x4 b[WN];
        u32x4 a[AQ][WM];
    };
    // Fragment addresses: the row swizzles depend only on the low five bits
    // of the row (32-row tiles), so every tile of a wave shares one slot
    // offset per K step and the tiles differ by immediate offsets.
    const int swa = swz<A_SLOTS>(l32), swb = swz<B_SLOTS>(l32);
    const int a_base = (wm * WM * 32 + l32) * A_ROW;
    const int b_base = A_BYTES + (wn * WN * 32 + l32) * B_ROW;
    auto read_frag = [&](Frag &f, int b, int u) {
        const lds_u8 *sb = smem + b * STAGE + b_base + 16 * ((2 * u + h) ^ swb);
#pragma unroll
        for (int j = 0; j < WN; ++j)
            f.b[j] = *(lds_u32x4 *)(sb + j * 32 * B_ROW);
#pragma unroll
        for (int s = 0; s < AQ; ++s) {
            const int slot = A4 ? 2 * u + h : 4 * u + 2 * s + h;
            const lds_u8 *sa = smem + b * STAGE + a_base + 16 * (slot ^ swa);
#pragma unroll
            for (int i = 0; i < WM; ++i)
                f.a[s][i] = *(lds_u32x4 *)(sa + i * 32 * A_ROW);
        }
    };

    v16i acc[WM][WN];
    float y[PER_GROUP ? WM : 1][PER_GROUP ? WN : 1][PER_GROUP ? 16 : 1];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[i][j][r] = 0;
                if constexpr (PER_GROUP)
                    y[i][j][r] = 0.f;
            }

    // MFMA operands of K half s: weight tile j and activation tile i.
    auto w_operand = [](const Frag &f, int s, int j) { return w4_operand_x16(f.b[j][2 * s], f.b[j][2 * s + 1]); };
    auto a_operand = [](const Frag &f, int s, int i) {
        if constexpr (A4)
            return a4_operand_x16(f.a[0][i][2 * s], f.a[0][i][2 * s + 1]);
        else
            return act_perm16(f.a[s][i][0], f.a[s][i][1], f.a[s][i][2], f.a[s][i][3]);
    };

    // One K step on fragments f; kt is the global K step (per-group scale row).
    auto compute = [&](const Frag &f, int kt) {
        uint16_t sc[PER_GROUP ? WN : 1];
        if constexpr (PER_GROUP) {
#pragma unroll
            for (int j = 0; j < WN; ++j)
                sc[j] = w_scales[(int64_t)kt * N + min(n0 + wn * WN * 32 + j * 32 + l32, N - 1)];
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            v4i bf[WN];
#pragma unroll
            for (int j = 0; j < WN; ++j)
                bf[j] = w_operand(f, s, j);
#pragma unroll
            for (int i = 0; i < WM; ++i) {
                const v4i af = a_operand(f, s, i);
#pragma unroll
                for (int j = 0; j < WN; ++j) {
                    if constexpr (TRANS)  // D^T[n][m]: lane = row m, registers = columns n
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[j], af, acc[i][j], 0, 0, 0);
                    else  // per group: the step's first product starts from zero
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                            af, bf[j], s == 0 ? v16i{} : acc[i][j], 0, 0, 0);
                }
            }
        }
        if constexpr (PER_GROUP) {
#pragma unroll
            for (int j = 0; j < WN; ++j) {
                const float scf = bf16_to_f32(sc[j]);
#pragma unroll
                for (int i = 0; i < WM; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        y[i][j][r] = __builtin_fmaf(scf, (float)acc[i][j][r], y[i][j][r]);
            }
        }
    };

    // The same K step for the transposed 4 x 2 wave tile, in a fixed order.
    // The step's 16 MFMAs run as 8 pairs (one activation tile, both weight
    // tiles); the decodes each pair needs are placed between earlier pairs,
    // and the operands of the next K step's first pair (its head: both weight
    // tiles and activation tile 0 of K half 0) are decoded under this step's
    // last pairs.  Left to itself the compiler decoded a whole K half in one
    // run ahead of its MFMAs, and a step's head could not start before the
    // step: with two waves per SIMD the matrix core then sat idle.  The fences
    // keep every pair's decodes (6 VALU ops per tile) inside the previous
    // pair's 64 MFMA cycles.  fn holds the next step's fragments; the last
    // stage runs the plain form (its K steps may end early).
    // The bf16 tile on byte codes keeps the compiler's order: with the fixed
    // order its fragments, the next step's head and the accumulators need one
    // register more than the 256 it has (a spill in every K step).
    constexpr bool ILV = TRANS && WM == 4 && WN == 2 && (A4 || OUT_I32);
    struct Head {
        v4i b[WN];
        v4i a;
    };
    auto decode_head = [&](Head &hd, const Frag &f) {
#pragma unroll
        for (int j = 0; j < WN; ++j)
            hd.b[j] = w_operand(f, 0, j);
        hd.a = a_operand(f, 0, 0);
    };
    auto compute_ilv = [&](const Frag &f, const Head &hd, const Frag &fn, Head &hn) {
        if constexpr (ILV) {
            v4i b1[WN], a0[WM], a1[WM];
            auto pair = [&](int i, const v4i(&bf)[WN], const v4i &af) {
#pragma unroll
                for (int j = 0; j < WN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[j], af, acc[i][j], 0, 0, 0);
            };
            __builtin_amdgcn_sched_barrier(0);
            pair(0, hd.b, hd.a);
            a0[1] = a_operand(f, 0, 1);
            b1[0] = w_operand(f, 1, 0);
            __builtin_amdgcn_sched_barrier(0);
            pair(1, hd.b, a0[1]);
            a0[2] = a_operand(f, 0, 2);
            b1[1] = w_operand(f, 1, 1);
            __builtin_amdgcn_sched_barrier(0);
            pair(2, hd.b, a0[2]);
            a0[3] = a_operand(f, 0, 3);
            a1[0] = a_operand(f, 1, 0);
            __builtin_amdgcn_sched_barrier(0);
            pair(3, hd.b, a0[3]);
            a1[1] = a_operand(f, 1, 1);
            __builtin_amdgcn_sched_barrier(0);
            pair(0, b1, a1[0]);
            a1[2] = a_operand(f, 1, 2);
            hn.b[0] = w_operand(fn, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            pair(1, b1, a1[1]);
            a1[3] = a_operand(f, 1, 3);
            hn.b[1] = w_operand(fn, 0, 1);
            __builtin_amdgcn_sched_barrier(0);
            pair(2, b1, a1[2]);
            hn.a = a_operand(fn, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            pair(3, b1, a1[3]);
        }
    };
    // K step u (not a stage's last) of stage buffer b, with step u + 1 read
    // ahead and, where dma, part u + 1 of the DMA of stage dst into buffer b ^ 1.
    Frag fr[2];
    Head hd[2];
    auto step = [&](int b, int u, int kt, bool dma, int dst) {
        read_frag(fr[(u + 1) & 1], b, u + 1);
        if constexpr (SPLIT)
            if (dma)
                issue_part(dst, b ^ 1, u + 1, std::integral_constant<int, NPART>{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ILV)
            compute_ilv(fr[u & 1], hd[u & 1], fr[(u + 1) & 1], hd[(u + 1) & 1]);
        else
            compute(fr[u & 1], kt);
        __builtin_amdgcn_sched_barrier(0);
    };

    constexpr int L = A_LD + B_LD;  // DMA instructions per wave and stage
    issue_stage(0, 0);
    if (nstages > 1) {
        issue_stage(1, 1);
        wait_vmcnt<L>();
    } else {
        wait_vmcnt<0>();
    }
    // The epilogue's kernel arguments are read here, so that no scalar load
    // (which returns out of order) is pending in the loop: the LDS waits
    // there can then count just the fragment reads in flight.
    asm volatile("" ::"s"(out), "s"(bias), "s"(row_scales), "s"(w_scales), "s"(acc_out), "s"(ldo),
                 "s"(lda), "s"(x_scale));
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    read_frag(fr[0], 0, 0);
    if constexpr (ILV)
        decode_head(hd[0], fr[0]);

    // Stages that have a successor: straight-line K steps.
    int st = 0;
    for (; st + 1 < nstages; ++st) {
        const int b = st & 1;
        // Stage st + 1 was issued whole before the loop (st = 0); otherwise
        // its first part (or all of it, without SPLIT) went out at the last
        // barrier and the remaining parts go out here.
        const bool dma = st >= 1;
#pragma unroll
        for (int u = 0; u + 1 < KSUB; ++u)
            step(b, u, st * KSUB + u, dma, st + 1);
        // Every read of this buffer has returned once each wave has waited
        // for its own, and the next stage has landed once each wave has
        // waited for its own DMA; the barrier extends both to the block, so
        // the buffer can be refilled with stage st + 2 and the next stage's
        // first fragments read.
        wait_lgkm0();
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        read_frag(fr[0], b ^ 1, 0);
        if (st + 2 < nstages)
            issue_part(st + 2, b, 0, std::integral_constant<int, NPART>{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ILV)
            compute_ilv(fr[(KSUB - 1) & 1], hd[(KSUB - 1) & 1], fr[0], hd[0]);
        else
            compute(fr[(KSUB - 1) & 1], st * KSUB + KSUB - 1);
        __builtin_amdgcn_sched_barrier(0);
    }
    // The last stage, possibly partial.
    {
        const int b = st & 1;
        const int nsub = ksteps - st * KSUB;
#pragma unroll
        for (int u = 0; u < KSUB; ++u) {
            if (u < nsub) {
                if (u + 1 < nsub)
                    read_frag(fr[(u + 1) & 1], b, u + 1);
                __builtin_amdgcn_sched_barrier(0);
                compute(fr[u & 1], st * KSUB + u);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // Epilogue.
    if constexpr (TRANS) {
        // Lane l holds rows m = m0w + 32 i + l32 and, in register group q,
        // columns n = n0w + 32 j + 8 q + 4 h + (0..3).
        const int m0w = m0 + wm * WM * 32;
        const int n0w = n0 + wn * WN * 32;
        if constexpr (OUT_I32) {
#pragma unroll
            for (int i = 0; i < WM; ++i) {
                const int m = m0w + i * 32 + l32;
                if (m < M)
#pragma unroll
                    for (int j = 0; j < WN; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int n = n0w + j * 32 + 8 * q + 4 * h;
                            if (n < N) {
                                const v4i v = {acc[i][j][4 * q] >> ACC_SHIFT, acc[i][j][4 * q + 1] >> ACC_SHIFT,
                                               acc[i][j][4 * q + 2] >> ACC_SHIFT, acc[i][j][4 * q + 3] >> ACC_SHIFT};
                                *reinterpret_cast<v4i *>(acc_out + (int64_t)m * lda + n) = v;
                            }
                        }
            }
        } else {
            // Stage the wave's 32 WM x 32 WN bf16 tile in LDS (rows padded to
            // 16 bytes past the tile width) and write it back with 16-byte
            // row-contiguous stores.  Column factors (weight scale over the
            // accumulator factor) and
            // bias are loaded one 32-column tile at a time to bound registers.
            constexpr int TW = WN * 32;          // tile width (columns)
            constexpr int PITCH = TW * 2 + 16;   // bytes per staged row
            float rsc[WM];
#pragma unroll
            for (int i = 0; i < WM; ++i)
                rsc[i] = row_scales[min(m0w + i * 32 + l32, M - 1)] * x_scale;
            __builtin_amdgcn_s_barrier();        // every wave is done with the operand stages
            lds_u8 *wt = smem + wave * (WM * 32 * PITCH);
#pragma unroll
            for (int j = 0; j < WN; ++j) {
                float cs[4][4], bc[4][4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int n = min(n0w + j * 32 + 8 * q + 4 * h + t, N - 1);
                        cs[q][t] = ACC_SCALE * bf16_to_f32(w_scales[n]);
                        bc[q][t] = bias ? bf16_to_f32(bias[n]) : 0.f;
                    }
#pragma unroll
                for (int i = 0; i < WM; ++i) {
                    const int ml = i * 32 + l32;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            v[t] = epilogue_channel((float)acc[i][j][4 * q + t], cs[q][t], rsc[i], bc[q][t]);
                        const u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                        *(__attribute__((address_space(3))) u32x2 *)(wt + ml * PITCH + (j * 32 + 8 * q + 4 * h) * 2) = pk;
                    }
                }
            }
            constexpr int CHUNKS = TW * 2 / 16;      // 16-byte chunks per row
            constexpr int ROWS = kWave / CHUNKS;     // rows per store instruction
#pragma unroll
            for (int it = 0; it < WM * 32 / ROWS; ++it) {
                const int ml = it * ROWS + lane / CHUNKS;
                const int c = lane % CHUNKS;
                const u32x4 v = *(const __attribute__((address_space(3))) u32x4 *)(wt + ml * PITCH + 16 * c);
                const int m = m0w + ml, n = n0w + 8 * c;
                if (m < M && n < N)
                    *reinterpret_cast<u32x4 *>(out + (int64_t)m * ldo + n) = v;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            const int n = n0 + wn * WN * 32 + j * 32 + l32;
            if (n >= N)
                continue;
            const float bn = bias ? bf16_to_f32(bias[n]) : 0.f;
#pragma unroll
            for (int i = 0; i < WM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * WM * 32 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                    if (m < M) {
                        const float v = y[i][j][r] * ACC_SCALE * (row_scales[m] * x_scale) + bn;
                        out[(int64_t)m * ldo + n] = f32_to_bf16(v);
                    }
                }
        }
    }
}

template <int WGM, int WGN, int WM, int WN, int KSUB, bool PG, bool I32, bool A4>
hipError_t launch_t(const int8_t *codes, int64_t ldq, const float *rs, int M, int K,
                    const uint8_t *packed, int64_t ldw, const uint16_t *ws, int N,
                    const uint16_t *bias, float xs, uint16_t *out, int64_t ldo, int32_t *acc,
                    int64_t lda, hipStream_t s)
{
    constexpr int BM = WGM * WM * 32, BN = WGN * WN * 32;
    constexpr size_t stages = (size_t)2 * KSUB * (BM * (A4 ? 32 : 64) + BN * 32);
    constexpr size_t staging = PG ? 0 : (size_t)WGM * WGN * (WM * 32) * (WN * 32 * 2 + 16);
    constexpr size_t smem = stages > staging ? stages : staging;
    static_assert(smem <= 160 * 1024, "LDS");
    auto kern = w4_gemm_kernel<WGM, WGN, WM, WN, KSUB, PG, I32, A4>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (attr != hipSuccess)
        return attr;
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(WGM * WGN * kWave), smem, s, codes, ldq, rs, M, K, packed,
                       ldw, ws, N, bias, xs, out, ldo, acc, lda);
    return hipGetLastError();
}

}  // namespace

// Per-channel results: 256 x 256 tiles, or 128 x 128 tiles (two blocks per
// CU) where the large ones would leave much of the chip idle.  The time is
// about the tiles per CU times the time of one tile; kSmallTileCost is a small
// tile's time in tenths of a large tile's (W4A4, K = 3840, N = 3840: about 16.5
// against 48 us, a quarter of the work).  Measured there: M = 1024 18.5
// against 39.2 us, M = 2048 33.5 against 41.0; M = 3072 / 4096 / 8192 keep the
// large tiles (43.0 / 49.0 / 96 against 49.2 / 64 / 123 us).
constexpr int64_t kSmallTileCost = 4;
bool small_tiles(int M, int N)
{
    constexpr int64_t kCus = 256;
    const int64_t big = ((M + 255) / 256) * (int64_t)((N + 255) / 256);
    const int64_t small = ((M + 127) / 128) * (int64_t)((N + 127) / 128);
    return kSmallTileCost * ((small + kCus - 1) / kCus) < 10 * ((big + kCus - 1) / kCus);
}

int launch_w4_gemm(const int8_t *codes, int64_t ldq, const float *row_scales, int M, int K,
                   const uint8_t *packed, int64_t ldw, const uint16_t *w_scales, bool per_group,
                   int N, const uint16_t *bias, float x_scale, uint16_t *out, int64_t ldo,
                   int32_t *acc_out, int64_t lda, bool a4, void *stream)
{
    if (M <= 0)
        return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
#define CK_GEMM_LAUNCH(A4)                                                                              \
    if (acc_out)                                                                                        \
        return (int)launch_t<2, 4, 4, 2, (A4 ? 4 : 2), false, true, A4>(codes, ldq, row_scales, M, K, packed, ldw, \
                                                             w_scales, N, bias, x_scale, out, ldo,      \
                                                             acc_out, lda, s);                          \
    if (per_group)                                                                                      \
        return (int)launch_t<2, 4, 2, 2, 2, true, false, A4>(codes, ldq, row_scales, M, K, packed, ldw, \
                                                             w_scales, N, bias, x_scale, out, ldo,      \
                                                             acc_out, lda, s);                          \
    if (small_tiles(M, N))                                                                              \
        return (int)launch_t<2, 4, 2, 1, (A4 ? 4 : 2), false, false, A4>(codes, ldq, row_scales, M, K, packed, \
                                                              ldw, w_scales, N, bias, x_scale, out, ldo, \
                                                              acc_out, lda, s);                         \
    return (int)launch_t<2, 4, 4, 2, (A4 ? 4 : 2), false, false, A4>(codes, ldq, row_scales, M, K, packed, ldw,    \
                                                          w_scales, N, bias, x_scale, out, ldo,         \
                                                          acc_out, lda, s);
    if (a4) {
        CK_GEMM_LAUNCH(true)
    }
    CK_GEMM_LAUNCH(false)
#undef CK_GEMM_LAUNCH
}

}  // namespace ck
