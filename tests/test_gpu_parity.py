"""GPU parity: every HIP entry point against the CPU oracle, called through the C ABI.

Acceptance (stated with the method): integer codes and int32 accumulators are
bit-exact given identical inputs; rotation codes from the same bf16 x agree on
>= 99.99% of the elements and differ by at most 1 elsewhere (the kernel's fp32
butterflies round differently from the oracle's exact sum); bf16 outputs
satisfy max |err| <= 1e-2 (|ref| + 1) against the oracle's fp64 result from the
GPU's own codes and row scales.  Sizes cover several tiles and a ragged tail.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import DEV, assert_codes_close, assert_output_close, bf16_dev, host, i8_dev, u8_dev

pytestmark = pytest.mark.gpu

ck = pytest.importorskip("packed_int4_convrot_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# --------------------------------------------------------------- rotate-quant


@pytest.mark.parametrize("G", [16, 64, 256])
@pytest.mark.parametrize("M,K", [(37, 768), (5, 3840), (3, 10240)])
def test_rotation_matches_oracle(G, M, K):
    x = workloads.activations(M, K, seed=G + K, outliers=max(1, K // 100), zero_rows=(1,))
    xr = host(ck.rotated_f32(bf16_dev(x), G))
    ref = oracle.rotate(x, G)
    xf = np.abs(workloads.bf16_bits_to_f32(x).astype(np.float64)).reshape(M, K // G, G)
    tol = 1e-6 * np.repeat(xf.sum(-1), G, axis=1).reshape(M, K) / np.sqrt(G) + 1e-30
    assert (np.abs(xr.astype(np.float64) - ref) <= tol).all()


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("G", [16, 64, 256])
def test_codes_bit_exact_given_rotation(G, bits):
    M, K = 67, 3840
    x = workloads.activations(M, K, seed=3 * G + bits, outliers=38, zero_rows=(0, 66))
    xd = bf16_dev(x)
    codes, scales = ck.rotate_quant(xd, G, bits)
    xr = host(ck.rotated_f32(xd, G))
    ref_codes, ref_scales = oracle.quantize(xr, bits)
    assert np.array_equal(host(codes), ref_codes)
    assert np.array_equal(host(scales), ref_scales)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("G", [16, 64, 256])
def test_rotate_quant_matches_oracle(G, bits):
    M, K = 96, 3840
    x = workloads.activations(M, K, seed=G * bits, outliers=38, zero_rows=(7, 95))
    codes, scales = ck.rotate_quant(bf16_dev(x), G, bits)
    ref_codes, ref_scales = oracle.rotate_quant(x, G, bits)
    assert_codes_close(host(codes), ref_codes)
    s = host(scales)
    assert np.all(np.abs(s - ref_scales) <= 2.0 ** -20 * ref_scales)
    assert s[7] == 1.0 and s[95] == 1.0 and not host(codes)[[7, 95]].any()


# K is a multiple of 64 (the entry point's rule) and of G.
_RQ_SHAPES = [(G, K) for G in (16, 64, 256)
              for K in (max(G, 64), 3 * max(G, 64), 2304, 10240, 10496, 16384, 20480, 20736, 32768)]


@pytest.mark.parametrize("G,K", _RQ_SHAPES)
def test_rotate_quant_every_launch_shape(G, K):
    """K across every workgroup size and chunk width the launcher picks (8- and
    16-column chunks; 128, 256 and 1024 threads; rows that fill every thread's
    chunks and rows that do not), in both code layouts, against the oracle."""
    x = workloads.activations(3, K, seed=K + G, outliers=max(1, K // 400), zero_rows=(1,))
    xd = bf16_dev(x)
    ref_codes, ref_scales = oracle.rotate_quant(x, G, 4)
    codes, scales = ck.rotate_quant(xd, G, 4)
    assert_codes_close(host(codes), ref_codes, min_equal=1.0 - max(1.0, 1e-4 * codes.numel()) / codes.numel())
    assert np.all(np.abs(host(scales) - ref_scales) <= 2.0 ** -20 * ref_scales)
    c4, s4 = ck.rotate_quant_packed4(xd, G)
    lo = (host(c4) & 0x0F).astype(np.int16)
    hi = (host(c4) >> 4).astype(np.int16)
    unpacked = np.empty((3, K), dtype=np.int16)
    unpacked[:, 0::2] = lo - 16 * (lo >= 8)
    unpacked[:, 1::2] = hi - 16 * (hi >= 8)
    assert np.array_equal(unpacked.astype(np.int8), host(codes))
    assert np.array_equal(host(s4), host(scales))
    c8, _ = ck.rotate_quant(xd, G, 8)
    assert_codes_close(host(c8), oracle.rotate_quant(x, G, 8)[0],
                       min_equal=1.0 - max(1.0, 1e-4 * c8.numel()) / c8.numel())


def test_rotate_quant_small_arrays_pooled_rate():
    """The >= 99.99% code-agreement bar is a rate.  An array of n < 10^4 codes cannot
    show it (one flip is already 1/n > 10^-4), so the per-array checks above allow one
    flip there; this test holds the rate itself on the pooled codes of all those
    small arrays (every launch shape, both code widths, each G)."""
    equal = total = 0
    for G, K in _RQ_SHAPES:
        x = workloads.activations(3, K, seed=K + G, outliers=max(1, K // 400), zero_rows=(1,))
        xd = bf16_dev(x)
        for bits in (4, 8):
            d = np.abs(host(ck.rotate_quant(xd, G, bits)[0]).astype(np.int32)
                       - oracle.rotate_quant(x, G, bits)[0].astype(np.int32))
            assert d.max() <= 1
            equal += int((d == 0).sum())
            total += d.size
    assert total > 10 ** 5
    assert equal >= 0.9999 * total, "pooled agreement %.6f" % (equal / total)


def test_rotate_quant_strided_input_ignores_padding():
    M, K, ld = 9, 1024, 1152  # padding columns hold NaN
    x = workloads.activations(M, K, seed=5, outliers=10, ld=ld)
    xd = bf16_dev(x)[:, :K]
    assert xd.stride(0) == ld
    c1, s1 = ck.rotate_quant(xd, 64, 8)
    c2, s2 = ck.rotate_quant(bf16_dev(np.ascontiguousarray(x[:, :K])), 64, 8)
    assert np.isfinite(host(s1)).all()
    assert np.array_equal(host(c1), host(c2)) and np.array_equal(host(s1), host(s2))


def test_rotate_quant_deterministic():
    x = bf16_dev(workloads.activations(300, 2048, seed=1, outliers=20))
    a = [ck.rotate_quant(x, 256, 8) for _ in range(2)]
    assert torch.equal(a[0][0], a[1][0]) and torch.equal(a[0][1], a[1][1])


# ------------------------------------------------------- integer accumulators


def _rand_codes(M, K, qmax, seed):
    return np.random.default_rng(seed).integers(-qmax, qmax + 1, size=(M, K), dtype=np.int8)


@pytest.mark.parametrize("M,K,N", [
    (1, 3840, 96), (5, 384, 272), (8, 3840, 160), (16, 1024, 64), (33, 3840, 48),
    (64, 4096, 32), (65, 384, 528), (300, 1152, 272), (513, 128, 16),
    # few-row kernel: every m-tile count, a partial last wave, a single wave
    # with masked weight-slice lanes, and the widest (8-wave) slice set
    (40, 2048, 48), (20, 3840, 64), (12, 8192, 32), (9, 192, 16), (17, 4096, 16),
    (20, 6144, 32), (50, 1024, 64), (64, 3840, 16),
    # more 16-row tiles than CUs (the grid runs in several rounds)
    (8, 1024, 4112), (6, 3840, 10240), (16, 512, 10240), (33, 1024, 8192), (64, 512, 16384),
])
@pytest.mark.parametrize("qmax", [127, 7])
def test_accumulators_bit_exact(M, K, N, qmax):
    codes = _rand_codes(M, K, qmax, seed=M + K + N)
    packed = workloads.packed_weights(N, K, seed=N)
    acc = host(ck.accumulators_i32(i8_dev(codes), u8_dev(packed)))
    ref = oracle.int_gemm(codes, oracle.unpack(packed))
    assert np.array_equal(acc.astype(np.int64), ref)


@pytest.mark.parametrize("M", [3, 70])
def test_accumulators_extremes(M):
    """Largest magnitudes: every code +-127 against every weight -8 or +7, long K."""
    K, N = 32768, 32
    codes = np.full((M, K), 127, dtype=np.int8)
    codes[1::2] = -127
    packed = np.zeros((N, K // 2), dtype=np.uint8)   # all weights -8
    packed[N // 2:] = 0xFF                            # all weights +7
    acc = host(ck.accumulators_i32(i8_dev(codes), u8_dev(packed)))
    ref = oracle.int_gemm(codes, oracle.unpack(packed))
    assert np.array_equal(acc.astype(np.int64), ref)
    assert np.abs(ref).max() == 127 * 8 * K


# ------------------------------------------- W4A4 codes packed two per byte


def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """int8 codes in [-8, 7], [M, K] -> bytes [M, K/2]: column 2j in bits 0..3,
    column 2j + 1 in bits 4..7, each as 4-bit two's complement."""
    c = codes.astype(np.uint8) & 0x0F
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def _unpack_nibbles(b: np.ndarray) -> np.ndarray:
    lo = (b & 0x0F).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    out = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int16)
    out[:, 0::2] = lo - 16 * (lo >= 8)
    out[:, 1::2] = hi - 16 * (hi >= 8)
    return out.astype(np.int8)


def test_nibble_helpers_round_trip():
    c = _rand_codes(3, 64, 8, seed=1).clip(-8, 7)
    assert np.array_equal(_unpack_nibbles(_pack_nibbles(c)), c)
    assert _pack_nibbles(np.array([[1, -1]], dtype=np.int8))[0, 0] == 0xF1


@pytest.mark.parametrize("G", [16, 64, 256])
@pytest.mark.parametrize("M,K", [(67, 3840), (1, 256), (300, 1024)])
def test_packed_w4a4_codes_equal_byte_codes(G, M, K):
    """The packed store of rotate-quant holds exactly the bits=4 codes and scales."""
    x = workloads.activations(M, K, seed=G + M, outliers=max(1, K // 100), zero_rows=(0,))
    xd = bf16_dev(x)
    codes4, s4 = ck.rotate_quant_packed4(xd, G)
    codes, s = ck.rotate_quant(xd, G, 4)
    assert np.array_equal(_unpack_nibbles(host(codes4)), host(codes))
    assert np.array_equal(host(s4), host(s))
    ref_codes, _ = oracle.rotate_quant(x, G, 4)
    assert_codes_close(_unpack_nibbles(host(codes4)), ref_codes)


def test_packed_w4a4_codes_strided_input():
    M, K, ld = 9, 1024, 1152  # padding columns hold NaN
    x = workloads.activations(M, K, seed=6, outliers=10, ld=ld)
    xd = bf16_dev(x)[:, :K]
    c1, s1 = ck.rotate_quant_packed4(xd, 64)
    c2, s2 = ck.rotate_quant(bf16_dev(np.ascontiguousarray(x[:, :K])), 64, 4)
    assert np.array_equal(_unpack_nibbles(host(c1)), host(c2)) and np.array_equal(host(s1), host(s2))


@pytest.mark.parametrize("M,K,N", [
    (1, 64, 16), (5, 384, 272), (64, 4096, 32), (65, 384, 528), (300, 1152, 272),
    (513, 128, 16), (257, 3840, 544), (1000, 640, 48),
])
def test_accumulators_a4_bit_exact(M, K, N):
    codes = _rand_codes(M, K, 7, seed=M + K + N + 1)
    packed = workloads.packed_weights(N, K, seed=N + 1)
    acc = host(ck.accumulators_i32_a4(u8_dev(_pack_nibbles(codes)), K, u8_dev(packed)))
    ref = oracle.int_gemm(codes, oracle.unpack(packed))
    assert np.array_equal(acc.astype(np.int64), ref)


@pytest.mark.parametrize("per_group", [False, True])
@pytest.mark.parametrize("M", [1, 2, 4, 5, 6, 8])
def test_decode_kernels_against_tiled_gemm_same_inputs(M, per_group):
    """The decode kernels (VALU GEMV up to 5 rows, few-row MFMA kernel from 6) and the
    tiled GEMM on the same W4A4 codes: the int32 accumulators are identical.  The bf16
    outputs can differ only through the fp32 order of the scale epilogue (the GEMV folds
    per-group scales per half group and lane, the tiled GEMM per 64-wide K step): at
    most one bf16 step, in at most 0.1% of the outputs."""
    K, N = 3840, 1024
    inp = workloads.linear_inputs(M, K, N, seed=M + 50, outliers=8, scale="group" if per_group else "channel",
                                  with_bias=True)
    xd, wd = bf16_dev(inp["x"]), u8_dev(inp["packed"])
    sd, bd = bf16_dev(inp["w_scales"]), bf16_dev(inp["bias"])
    codes, scales = ck.rotate_quant(xd, 64, 4)
    codes4, scales4 = ck.rotate_quant_packed4(xd, 64)
    assert torch.equal(scales, scales4)
    acc_decode = ck.accumulators_i32(codes, wd)
    acc_tiled = ck.accumulators_i32_a4(codes4, K, wd)
    assert torch.equal(acc_decode, acc_tiled)
    out_decode = host(ck.gemm_q(codes, scales, wd, sd, per_group, bias=bd))
    out_tiled = host(ck.gemm_packed4(codes4, scales4, wd, sd, per_group, bias=bd))
    # Measured on MI355X: all outputs identical at these shapes, for both scale kinds.
    ulp = np.maximum(np.abs(out_tiled), np.float32(2.0 ** -126)) * np.float32(2.0 ** -7)
    r = np.abs(out_decode - out_tiled) / ulp
    assert r.max() <= 1.0 and (r > 0).mean() <= 1e-3


def test_accumulators_a4_extremes():
    """Every code +-7 against every weight -8 or +7, longest K."""
    M, K, N = 70, 32768, 32
    codes = np.full((M, K), 7, dtype=np.int8)
    codes[1::2] = -7
    packed = np.zeros((N, K // 2), dtype=np.uint8)   # all weights -8
    packed[N // 2:] = 0xFF                            # all weights +7
    acc = host(ck.accumulators_i32_a4(u8_dev(_pack_nibbles(codes)), K, u8_dev(packed)))
    ref = oracle.int_gemm(codes, oracle.unpack(packed))
    assert np.array_equal(acc.astype(np.int64), ref)
    assert np.abs(ref).max() == 7 * 8 * K


@pytest.mark.parametrize("per_group", [True, False])
@pytest.mark.parametrize("M", [1, 7, 64, 257])
def test_gemm_packed4_matches_oracle(M, per_group):
    """ck_w4a4_gemm_packed at every M (the tiled GEMM on packed codes) against the
    oracle epilogue on the same codes and scales."""
    K, N = 1280, 272
    inp = workloads.linear_inputs(M, K, N, seed=M + 17, outliers=13, scale="group" if per_group else "channel",
                                  zero_rows=(M - 1,) if M > 2 else (), with_bias=(M % 2 == 1))
    codes4, rs = ck.rotate_quant_packed4(bf16_dev(inp["x"]), 64)
    bias = None if inp["bias"] is None else bf16_dev(inp["bias"])
    out = host(ck.gemm_packed4(codes4, rs, u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), per_group, bias=bias))
    ref = oracle.gemm_q(_unpack_nibbles(host(codes4)), host(rs), inp["packed"], inp["w_scales"], per_group,
                        bias=inp["bias"])
    assert_output_close(out, ref)


def test_activation_cache_reuses_packed_codes():
    """One packed rotate-quant serves several linears on the same input (Q, K, V-like
    weights of different widths): each result is bit-identical to its own whole linear."""
    M, K, G = 300, 2304, 256
    x = bf16_dev(workloads.activations(M, K, seed=4, outliers=23))
    codes4, rs = ck.rotate_quant_packed4(x, G)
    for i, N in enumerate((384, 128, 128)):
        w = workloads.linear_inputs(1, K, N, seed=40 + i, outliers=1, scale="channel")
        wd, sd = u8_dev(w["packed"]), bf16_dev(w["w_scales"])
        cached = ck.gemm_packed4(codes4, rs, wd, sd, False)
        whole = ck.linear(x, G, 4, wd, sd, False)
        assert torch.equal(cached.view(torch.int16), whole.view(torch.int16))


@pytest.mark.parametrize("per_group", [True, False])
@pytest.mark.parametrize("M", [65, 129, 300])
def test_w4a4_linear_tiled_path(M, per_group):
    """The tiled path of the W4A4 linear (packed codes in the workspace) against
    the oracle epilogue on the GPU's own byte codes, at ragged M and N."""
    K, N = 2304, 400
    inp = workloads.linear_inputs(M, K, N, seed=M + 3, outliers=20, scale="group" if per_group else "channel",
                                  zero_rows=(M - 1,), with_bias=True)
    xd = bf16_dev(inp["x"])
    out = host(ck.linear(xd, 256, 4, u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), per_group,
                         bias=bf16_dev(inp["bias"])))
    codes, scales = ck.rotate_quant(xd, 256, 4)
    ref = oracle.gemm_q(host(codes), host(scales), inp["packed"], inp["w_scales"], per_group, bias=inp["bias"])
    assert_output_close(out, ref)


# ------------------------------------------------------------ matmul outputs


@pytest.mark.parametrize("per_group", [True, False])
@pytest.mark.parametrize("M", [1, 4, 8, 13, 32, 64, 100, 257])
def test_gemm_q_outputs(M, per_group):
    K, N = 1280, 272
    inp = workloads.linear_inputs(M, K, N, seed=M, outliers=13, scale="group" if per_group else "channel",
                                  zero_rows=(M - 1,) if M > 2 else (), with_bias=(M % 2 == 0))
    codes, scales = oracle.rotate_quant(inp["x"], 64, 8)
    out = ck.gemm_q(i8_dev(codes), torch.from_numpy(scales).to(DEV), u8_dev(inp["packed"]),
                    bf16_dev(inp["w_scales"]), per_group,
                    bias=None if inp["bias"] is None else bf16_dev(inp["bias"]))
    ref = oracle.gemm_q(codes, scales, inp["packed"], inp["w_scales"], per_group, bias=inp["bias"])
    assert_output_close(host(out), ref)


@pytest.mark.parametrize("per_group", [True, False])
@pytest.mark.parametrize("M,N", [(8, 4112), (33, 10240)])
def test_gemm_q_outputs_more_tiles_than_cus(M, N, per_group):
    """Few-row kernel with more 16-row tiles than CUs (257 and 640 workgroups), with
    per-group and per-channel scales and a bias, against the oracle; the whole linear
    (codes in the kernel's tiled layout) equals rotate-quant + gemm_q bit for bit."""
    K = 1024
    inp = workloads.linear_inputs(M, K, N, seed=M + N, outliers=9, scale="group" if per_group else "channel",
                                  zero_rows=(1,), with_bias=True)
    codes, scales = oracle.rotate_quant(inp["x"], 64, 8)
    out = ck.gemm_q(i8_dev(codes), torch.from_numpy(scales).to(DEV), u8_dev(inp["packed"]),
                    bf16_dev(inp["w_scales"]), per_group, bias=bf16_dev(inp["bias"]))
    ref = oracle.gemm_q(codes, scales, inp["packed"], inp["w_scales"], per_group, bias=inp["bias"])
    assert_output_close(host(out), ref)
    lin = ck.linear(bf16_dev(inp["x"]), 64, 8, u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), per_group,
                    bias=bf16_dev(inp["bias"]))
    c2, s2 = ck.rotate_quant(bf16_dev(inp["x"]), 64, 8)
    two = ck.gemm_q(c2, s2, u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), per_group, bias=bf16_dev(inp["bias"]))
    assert torch.equal(lin, two)


@pytest.mark.parametrize("per_group", [True, False])
def test_gemv_entry_matches_oracle(per_group):
    K, N = 3840, 1024
    for M in (1, 4, 8):
        inp = workloads.linear_inputs(M, K, N, seed=11, outliers=8, scale="group" if per_group else "channel")
        codes, scales = oracle.rotate_quant(inp["x"], 64, 8)
        out = ck.gemv(i8_dev(codes), torch.from_numpy(scales).to(DEV), u8_dev(inp["packed"]),
                      bf16_dev(inp["w_scales"]), per_group)
        ref = oracle.gemm_q(codes, scales, inp["packed"], inp["w_scales"], per_group)
        assert_output_close(host(out), ref)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("per_group", [True, False])
@pytest.mark.parametrize("G", [16, 64, 256])
@pytest.mark.parametrize("M", [1, 2, 3, 7, 40, 64, 300])
def test_linear_end_to_end(M, G, per_group, bits):
    K, N = 1536, 144
    inp = workloads.linear_inputs(M, K, N, seed=G + M, outliers=15, scale="group" if per_group else "channel",
                                  zero_rows=(1,) if M > 1 else (), with_bias=True)
    xd = bf16_dev(inp["x"])
    wd, sd, bd = u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), bf16_dev(inp["bias"])
    out = host(ck.linear(xd, G, bits, wd, sd, per_group, bias=bd))
    codes, scales = ck.rotate_quant(xd, G, bits)
    codes, scales = host(codes), host(scales)
    # codes against the oracle's own rotation (tolerance of the fp32 transform)
    ref_codes, _ = oracle.rotate_quant(inp["x"], G, bits)
    assert_codes_close(codes, ref_codes)
    # output against the oracle epilogue on the GPU's own codes and scales
    ref = oracle.gemm_q(codes, scales, inp["packed"], inp["w_scales"], per_group, bias=inp["bias"])
    assert_output_close(out, ref)
    if M > 1:
        assert np.array_equal(out[1], workloads.bf16_bits_to_f32(inp["bias"]))  # zero row -> bias


FUSED_CASES = [(1, 3840), (2, 3840), (3, 3840), (4, 3840), (1, 64), (4, 64), (2, 256), (3, 2112), (1, 8192),
               (4, 8192), (1, 16384), (2, 16384), (3, 16384)]


def mfma_one_launch(M, K, N):
    """The whole linear runs the one-launch MFMA kernel (5 to 8 rows, K <= 4096, N >= 8192)."""
    return 5 <= M <= 8 and K <= 4096 and N >= 8192


def padded_two_launch(xd, G, bits, wd, sd, per_group, bd, x_scale):
    """rotate-quant + the few-row MFMA kernel on codes (ck_w4_gemm_q takes it from 6 rows
    on), with x padded by zero rows to at least 6: rows are independent on that path, so
    its first M rows are what the one-launch MFMA kernel must give bit for bit."""
    M = xd.shape[0]
    xp = torch.cat([xd, torch.zeros((max(0, 6 - M), xd.shape[1]), dtype=xd.dtype, device=xd.device)])
    codes, scales = ck.rotate_quant(xp, G, bits)
    return ck.gemm_q(codes, scales * np.float32(x_scale), wd, sd, per_group, bias=bd)[:M]


@pytest.mark.parametrize("M,K", FUSED_CASES)
@pytest.mark.parametrize("G", [16, 64, 256])
def test_fused_decode_linear_equals_two_step_path(M, K, G):
    """The one-launch decode linear gives the two-launch outputs bit for bit, for both
    bit widths and scale kinds, with a zero row and an input scale.  The VALU form
    (one row, or more rows beyond K = 4096; one workgroup per CU) equals
    ck_rotate_quant followed by ck_w4_gemv: one K slice with 2 active lanes, partial
    and full slices, up to eight slices.  The MFMA form (2 to 8 rows) equals
    rotate-quant followed by the few-row kernel, and on per-channel scales (exact
    integer sums) the GEMV too.  N = 16 and 48 (two and six workgroups), 1024, 4112
    (the last workgroup partly empty) and 10240."""
    if K % G:
        pytest.skip("K must be a multiple of G")
    for N in (16, 48, 1024, 4112, 10240):
        for bits in (8, 4):
            for per_group in (True, False):
                inp = workloads.linear_inputs(M, K, N, seed=G + M + bits, outliers=min(8, K // 8),
                                              scale="group" if per_group else "channel",
                                              zero_rows=(1,) if M > 1 else (), with_bias=True)
                xd, wd = bf16_dev(inp["x"]), u8_dev(inp["packed"])
                sd, bd = bf16_dev(inp["w_scales"]), bf16_dev(inp["bias"])
                fused = ck.linear(xd, G, bits, wd, sd, per_group, bias=bd, x_scale=0.3)
                codes, scales = ck.rotate_quant(xd, G, bits)
                two = ck.gemv(codes, scales * np.float32(0.3), wd, sd, per_group, bias=bd)
                if mfma_one_launch(M, K, N):
                    assert torch.equal(fused, padded_two_launch(xd, G, bits, wd, sd, per_group, bd, 0.3)), \
                        (N, bits, per_group)
                    if per_group:
                        continue
                assert torch.equal(fused, two), (N, bits, per_group)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("K,G", [(64, 16), (64, 64), (256, 256), (2048, 64), (2112, 64), (3840, 16),
                                 (3840, 64), (3840, 256), (4096, 256)])
def test_mfma_decode_linear_launch_shapes(M, K, G):
    """The one-launch MFMA linear (through its test entry point, which runs it for any
    N) over its workgroup shapes: one or two K slices (the second with 1 to 32 groups),
    workgroups of 8 to 48 weight rows (a half tile of 8 at N = 16, 48, 10240; a last
    workgroup with 8 of its 24 rows at N = 4112; 342 workgroups of 48 rows, more than
    the CUs, at N = 16384), both bit widths and scale kinds, a zero row, bias and an
    input scale: bit for bit against rotate-quant + the few-row kernel, and against the
    oracle's epilogue on the same codes.  Where the linear's own plan picks this kernel
    (5 to 8 rows, N >= 8192), ck_w4a8_linear / ck_w4a4_linear give the same bits."""
    Ns = [16, 48, 4112] + ([10240] if (K, G) == (3840, 64) else []) + ([16384] if K == 4096 else [])
    for N in Ns:
        for bits in (8, 4):
            for per_group in (True, False):
                inp = workloads.linear_inputs(M, K, N, seed=3 * M + K + bits, outliers=min(8, K // 8),
                                              scale="group" if per_group else "channel",
                                              zero_rows=(M - 1,) if M > 1 else (),
                                              with_bias=True)
                xd, wd = bf16_dev(inp["x"]), u8_dev(inp["packed"])
                sd, bd = bf16_dev(inp["w_scales"]), bf16_dev(inp["bias"])
                out = ck.linear_mfma_one_launch(xd, G, bits, wd, sd, per_group, bias=bd, x_scale=0.75)
                ref = padded_two_launch(xd, G, bits, wd, sd, per_group, bd, 0.75)
                assert torch.equal(out, ref), (N, bits, per_group)
                if mfma_one_launch(M, K, N):
                    assert torch.equal(ck.linear(xd, G, bits, wd, sd, per_group, bias=bd, x_scale=0.75), out)
                if N <= 4112:
                    codes, scales = ck.rotate_quant(xd, G, bits)
                    ref = oracle.gemm_q(host(codes), host(scales) * np.float32(0.75), inp["packed"],
                                        inp["w_scales"], per_group, bias=inp["bias"])
                    assert_output_close(host(out), ref)
                    if M > 1:
                        h = host(out)
                        assert np.array_equal(h[M - 1], workloads.bf16_bits_to_f32(inp["bias"]))  # zero row -> bias


@pytest.mark.parametrize("G", [16, 64, 256])
@pytest.mark.parametrize("M,K", [(6, 3840), (8, 3840), (13, 1024), (16, 3840), (17, 3840), (24, 2048),
                                 (32, 3840), (33, 3840), (48, 1024), (64, 3840)])
def test_linear_tiled_codes_equal_row_major_path(M, K, G):
    """From 6 to 64 rows the whole linear stores its codes in the few-row kernel's
    tiled operand layout.  Its outputs are bit-identical to ck_rotate_quant
    (row-major codes) followed by ck_w4_gemm_q, which runs the same kernel on
    row-major codes: both bit widths and scale kinds, full and partial last tiles,
    a zero row, and the input scale."""
    N = 272
    for bits in (8, 4):
        for per_group in (True, False):
            inp = workloads.linear_inputs(M, K, N, seed=G + M + bits, outliers=8,
                                          scale="group" if per_group else "channel", zero_rows=(1,),
                                          with_bias=True)
            xd, wd = bf16_dev(inp["x"]), u8_dev(inp["packed"])
            sd, bd = bf16_dev(inp["w_scales"]), bf16_dev(inp["bias"])
            lin = ck.linear(xd, G, bits, wd, sd, per_group, bias=bd)
            codes, scales = ck.rotate_quant(xd, G, bits)
            two = ck.gemm_q(codes, scales, wd, sd, per_group, bias=bd)
            assert torch.equal(lin, two), (bits, per_group)
            # the input scale multiplies the row scales on both paths
            lin3 = ck.linear(xd, G, bits, wd, sd, per_group, bias=bd, x_scale=3.0)
            two3 = ck.gemm_q(codes, scales * 3.0, wd, sd, per_group, bias=bd)
            assert torch.equal(lin3, two3), (bits, per_group)


def test_fused_decode_linear_strided_input_ignores_padding():
    """Row stride > K: the fused kernel reads only the K columns (the padding is NaN)."""
    K, N, ld = 3840, 512, 4096
    inp = workloads.linear_inputs(1, K, N, seed=9, outliers=8, scale="group", with_bias=False)
    padded = workloads.activations(1, K, seed=9, outliers=8, ld=ld)
    assert np.array_equal(padded[:, :K], inp["x"])
    wd, sd = u8_dev(inp["packed"]), bf16_dev(inp["w_scales"])
    xs = bf16_dev(padded)[:, :K]
    assert xs.stride(0) == ld
    out = ck.linear(xs, 64, 8, wd, sd, True)
    ref = ck.linear(bf16_dev(inp["x"]), 64, 8, wd, sd, True)
    assert not torch.isnan(out).any()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("M", [1, 3, 8, 300])
def test_graph_replay_matches_eager(M):
    """Captured into a HIP graph, the linear gives the eager result on every replay."""
    K, N = 1024, 272
    inp = workloads.linear_inputs(M, K, N, seed=M, outliers=5, scale="group", with_bias=True)
    xd, wd, sd, bd = bf16_dev(inp["x"]), u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), bf16_dev(inp["bias"])
    ws = torch.empty((ck.workspace_bytes(M, K, N),), dtype=torch.uint8, device=DEV)
    eager = ck.linear(xd, 64, 8, wd, sd, True, bias=bd)
    out = torch.zeros_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ck.linear(xd, 64, 8, wd, sd, True, bias=bd, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ck.linear(xd, 64, 8, wd, sd, True, bias=bd, out=out, workspace=ws)
    for _ in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        ck.rotate_quant(xd, 256, 4)  # unrelated eager work between replays


def _graph_replays_equal_eager(fn, out):
    """Capture fn (writing into out) in a HIP graph; every replay equals the eager result."""
    eager = fn().clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        torch.mm(torch.ones(64, 64, device=DEV), torch.ones(64, 64, device=DEV))  # unrelated eager work


def test_mfma_one_launch_in_the_linear_graph_strided_noalloc():
    """Where the linear itself takes the one-launch MFMA kernel (5 to 8 rows, N >= 8192):
    a HIP graph replays it bit-identically with eager work between replays; a strided x
    (NaN padding past K) gives the dense result; and the allocation-free W4A4 entry,
    which needs no scratch on this path, equals the workspace entry."""
    M, K, N = 7, 3840, 8192
    inp = workloads.linear_inputs(M, K, N, seed=77, outliers=8, scale="group", zero_rows=(2,), with_bias=True)
    xd, wd, sd, bd = bf16_dev(inp["x"]), u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), bf16_dev(inp["bias"])
    ref = padded_two_launch(xd, 64, 8, wd, sd, True, bd, 1.0)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty((ck.workspace_bytes(M, K, N),), dtype=torch.uint8, device=DEV)
    _graph_replays_equal_eager(lambda: ck.linear(xd, 64, 8, wd, sd, True, bias=bd, out=out, workspace=ws), out)
    assert torch.equal(out, ref)
    padded = workloads.activations(M, K, seed=77, outliers=8, ld=K + 256)
    xs = bf16_dev(padded)
    xs[:, K:] = float("nan")
    assert torch.equal(ck.linear(xs[:, :K], 64, 8, wd, sd, True, bias=bd), ck.linear(bf16_dev(padded[:, :K]), 64, 8,
                                                                                     wd, sd, True, bias=bd))
    lin4 = ck.linear(xd, 64, 4, wd, sd, True, bias=bd)
    assert torch.equal(ck.w4a4_linear_noalloc(xd, 64, wd, sd, True, bias=bd), lin4)
    assert torch.equal(lin4, padded_two_launch(xd, 64, 4, wd, sd, True, bd, 1.0))


@pytest.mark.parametrize("K,G,N", [(3840, 64, 10240), (3840, 16, 4112), (16384, 256, 4112)])
@pytest.mark.parametrize("bits", [8, 4])
def test_per_channel_rows_same_bits_for_every_batch_size(K, G, N, bits):
    """Per-channel scales: every kernel applies one epilogue, acc * (s_w * r) + b with
    the exact integer sum acc, so a row's output does not depend on the batch it came
    in, that is on which kernel the batch size picked.  On the same codes: the tiled
    GEMM (72 rows) against the VALU GEMV (1 to 5 rows), the few-row MFMA kernel (6 to
    32 rows at K = 3840; the GEMV at K = 16384).  Through the whole linear: 72 rows (the
    tiled GEMM; W4A4 on packed codes) against the one-launch VALU linear (1 to 4 rows),
    the one-launch MFMA linear (5 to 8 rows at N = 10240), the two-launch forms and the
    few-row kernel on tiled codes (32 rows).  Per-group scales are folded in a different
    order by each kernel and are held to the oracle's bar instead."""
    Mbig = 72
    inp = workloads.linear_inputs(Mbig, K, N, seed=K + G + bits, outliers=min(8, K // 8), scale="channel",
                                  zero_rows=(2, 70), with_bias=True)
    xd, wd = bf16_dev(inp["x"]), u8_dev(inp["packed"])
    sd, bd = bf16_dev(inp["w_scales"]), bf16_dev(inp["bias"])
    codes, scales = ck.rotate_quant(xd, G, bits)
    rs = scales * np.float32(0.3)
    ref = ck.gemm_q(codes, rs, wd, sd, False, bias=bd)
    for m in (1, 2, 4, 5, 6, 8, 32):
        sub = ck.gemm_q(codes[:m], rs[:m], wd, sd, False, bias=bd)
        assert torch.equal(sub, ref[:m]), ("codes", m)
        if m <= 8:
            assert torch.equal(ck.gemv(codes[:m], rs[:m], wd, sd, False, bias=bd), sub), ("gemv", m)
    lin = ck.linear(xd, G, bits, wd, sd, False, bias=bd, x_scale=0.3)
    for m in (1, 3, 4, 5, 7, 8, 32):
        assert torch.equal(ck.linear(xd[:m], G, bits, wd, sd, False, bias=bd, x_scale=0.3), lin[:m]), ("linear", m)
    assert_output_close(host(lin[:8]), oracle.gemm_q(host(codes[:8]), host(scales[:8]), inp["packed"], inp["w_scales"],
                                                      False, bias=inp["bias"], x_scale=0.3))


def test_graph_replay_packed_w4a4_and_awq_gemm():
    """The packed W4A4 path (M > 64), the weight producer and the AWQ prefill GEMM
    replay from a HIP graph bit-identically."""
    M, K, N = 300, 1024, 272
    inp = workloads.linear_inputs(M, K, N, seed=8, outliers=5, scale="channel", with_bias=True)
    xd, wd, sd, bd = bf16_dev(inp["x"]), u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), bf16_dev(inp["bias"])
    ws = torch.empty((ck.workspace_bytes(M, K, N),), dtype=torch.uint8, device=DEV)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    _graph_replays_equal_eager(lambda: ck.linear(xd, 256, 4, wd, sd, False, bias=bd, out=out, workspace=ws),
                               out)
    x, packed, s, z, bias = _awq_inputs(M, K, N, seed=9)
    args = (bf16_dev(x), u8_dev(packed), bf16_dev(s), bf16_dev(z))
    bias_d = bf16_dev(bias)
    out2 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    _graph_replays_equal_eager(lambda: ck.w4a16_gemm(*args, bias=bias_d, out=out2), out2)
    w = bf16_dev(_weights_bf16(N, K, seed=10))
    pk = torch.empty((N, K // 2), dtype=torch.uint8, device=DEV)
    sc = torch.empty((K // 64, N), dtype=torch.bfloat16, device=DEV)
    _graph_replays_equal_eager(lambda: ck.quantize_weights(w, 64, True, pk, sc)[0], pk)


def test_awq_gemm_deterministic():
    x, packed, s, z, bias = _awq_inputs(1000, 768, 528, seed=12)
    args = (bf16_dev(x), u8_dev(packed), bf16_dev(s), bf16_dev(z))
    a = [ck.w4a16_gemm(*args, bias=bf16_dev(bias)) for _ in range(2)]
    assert torch.equal(a[0].view(torch.int16), a[1].view(torch.int16))


def test_linear_x_scale_power_of_two_is_exact():
    inp = workloads.linear_inputs(20, 512, 64, seed=2, outliers=4, scale="channel")
    xd, wd, sd = bf16_dev(inp["x"]), u8_dev(inp["packed"]), bf16_dev(inp["w_scales"])
    a = host(ck.linear(xd, 64, 8, wd, sd, False))
    b = host(ck.linear(xd, 64, 8, wd, sd, False, x_scale=4.0))
    assert np.array_equal(b, 4.0 * a)


@pytest.mark.parametrize("alpha", [0.3, 3.0, 4.0])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M", [1, 4, 20, 300])
def test_linear_x_scale_matches_oracle(M, bits, alpha):
    """Input scale against the oracle's reading (the linear of alpha * x: codes of x,
    row scale times alpha, bias unscaled), on every kernel path: the fused decode
    launch, the VALU GEMV, the few-row MFMA kernel and the tiled GEMM."""
    K, N = 1536, 272
    for per_group in (True, False):
        inp = workloads.linear_inputs(M, K, N, seed=M + bits, outliers=15, scale="group" if per_group else "channel",
                                      with_bias=True)
        xd = bf16_dev(inp["x"])
        out = host(ck.linear(xd, 64, bits, u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), per_group,
                             bias=bf16_dev(inp["bias"]), x_scale=alpha))
        codes, scales = ck.rotate_quant(xd, 64, bits)
        a32 = float(np.float32(alpha))   # the C ABI takes the scale as fp32
        ref = oracle.gemm_q(host(codes), host(scales), inp["packed"], inp["w_scales"], per_group,
                            bias=inp["bias"], x_scale=a32)
        assert_output_close(out, ref)


def test_linear_int8_weight_tensor_and_strided_weights():
    """Packed weights given as an int8 tensor, and as a strided view, give the same bytes."""
    M, K, N = 10, 512, 48
    inp = workloads.linear_inputs(M, K, N, seed=4, outliers=3, scale="group")
    wide = workloads.packed_weights(N, K, seed=4, ld=K // 2 + 64)
    assert np.array_equal(wide[:, :K // 2], inp["packed"])
    xd, sd = bf16_dev(inp["x"]), bf16_dev(inp["w_scales"])
    ref = host(ck.linear(xd, 64, 8, u8_dev(inp["packed"]), sd, True))
    as_i8 = u8_dev(inp["packed"]).view(torch.int8)
    strided = u8_dev(wide)[:, :K // 2]
    assert np.array_equal(host(ck.linear(xd, 64, 8, as_i8, sd, True)), ref)
    assert np.array_equal(host(ck.linear(xd, 64, 8, strided, sd, True)), ref)


def test_empty_batch_is_noop():
    inp = workloads.linear_inputs(1, 256, 32, seed=1, outliers=0, scale="channel")
    x = bf16_dev(inp["x"])[:0]
    out = ck.linear(x, 64, 8, u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), False)
    assert out.shape == (0, 32)


def test_matmul_deterministic():
    inp = workloads.linear_inputs(300, 1024, 528, seed=8, outliers=10, scale="group")
    args = (bf16_dev(inp["x"]), 64, 4, u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), True)
    assert torch.equal(ck.linear(*args), ck.linear(*args))
    inp = workloads.linear_inputs(8, 1024, 528, seed=8, outliers=10, scale="group")
    args = (bf16_dev(inp["x"]), 64, 8, u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), True)
    assert torch.equal(ck.linear(*args), ck.linear(*args))


def test_errors_raise():
    x = bf16_dev(workloads.activations(4, 512, seed=0))
    with pytest.raises(ck.CKError):
        ck.rotate_quant(x, 32, 8)          # unsupported G
    with pytest.raises(ck.CKError):
        ck.rotate_quant(x[:, :96], 16, 8)  # K % 64: unsupported
    with pytest.raises(ValueError):
        ck.rotate_quant(x[:, :320], 256, 8)  # K % G: invalid


def test_binding_rejects_mis_sized_tensors():
    """Outputs and auxiliary operands are checked against M, N and K before any launch."""
    M, K, N = 4, 512, 64
    inp = workloads.linear_inputs(M, K, N, seed=3, outliers=0, scale="group", with_bias=True)
    x, wd, sd = bf16_dev(inp["x"]), u8_dev(inp["packed"]), bf16_dev(inp["w_scales"])
    codes, rs = ck.rotate_quant(x, 64, 8)
    with pytest.raises(ValueError):   # output one row short
        ck.linear(x, 64, 8, wd, sd, True, out=torch.empty((M - 1, N), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):   # row scales of the wrong length
        ck.gemm_q(codes, rs[:-1], wd, sd, True)
    with pytest.raises(ValueError):   # per-group scales given as a transposed view
        ck.gemm_q(codes, rs, wd, sd.t().contiguous().t(), True)
    with pytest.raises(ValueError):   # per-channel scales of the per-group shape
        ck.gemm_q(codes, rs, wd, sd, False)
    with pytest.raises(ValueError):   # bias of the wrong length
        ck.linear(x, 64, 8, wd, sd, True, bias=bf16_dev(inp["bias"])[:-16])
    with pytest.raises(ValueError):   # workspace of the wrong dtype
        ck.linear(x, 64, 8, wd, sd, True, workspace=torch.empty((1 << 16,), dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):   # codes output too short for K
        ck.rotate_quant(x, 64, 8, codes=torch.empty((M, K - 64), dtype=torch.int8, device=DEV))
    with pytest.raises(ValueError):   # AWQ zero points with one group missing
        ck.w4a16_gemv(x, wd, sd, sd[:-1].contiguous())


# ----------------------------------------------------------------- AWQ W4A16


@pytest.mark.parametrize("M,K,N", [(1, 3072, 1024), (3, 1024, 272), (8, 4096, 64), (1, 64, 16),
                                   (2, 10240, 48), (5, 3072, 32), (7, 16384, 16), (4, 2112, 80),
                                   (2, 7168, 32), (6, 1088, 48)])
def test_awq_gemv_matches_oracle(M, K, N):
    """Both lane widths: 16-column lanes where they leave fewer lanes past K (K = 64,
    1024, 1088, 2112, 3072, 7168), 32-column lanes otherwise (K = 4096, 10240, 16384)."""
    d = workloads.awq_inputs(M, K, N, seed=K + N, with_bias=(M == 3))
    out = ck.w4a16_gemv(bf16_dev(d["x"]), u8_dev(d["packed"]), bf16_dev(d["scales"]), bf16_dev(d["zeros"]),
                        bias=None if d["bias"] is None else bf16_dev(d["bias"]))
    ref = oracle.awq_gemv(d["x"], d["packed"], d["scales"], d["zeros"], bias=d["bias"])
    assert_output_close(host(out), ref)


# ------------------------------------------------------ weight producer


def _weights_bf16(N, K, seed, zero_rows=()):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K)) * rng.uniform(0.005, 0.05, size=(N, 1))
    w[:, rng.choice(K, max(1, K // 100), replace=False)] *= 8.0   # a few heavy input channels
    for r in zero_rows:
        w[r] = 0.0
    return workloads.to_bf16_bits(w)


@pytest.mark.parametrize("per_group", [False, True])
@pytest.mark.parametrize("G", [16, 64, 256])
def test_quantize_weights_bit_exact_given_rotation(G, per_group):
    """Packed codes and bf16 scales equal the oracle's quantiser applied to the
    kernel's own rotated values (ck_test_rotate_f32 runs the same rotation)."""
    N, K = 272, 3840
    w = _weights_bf16(N, K, seed=G + per_group, zero_rows=(5,))
    wd = bf16_dev(w)
    packed, scales = ck.quantize_weights(wd, G, per_group)
    wr = host(ck.rotated_f32(wd, G))
    ref_p, ref_s = oracle.quantize_weights(wr, per_group)
    assert np.array_equal(host(packed), ref_p)
    assert np.array_equal(host(scales.view(torch.int16)).view(np.uint16), ref_s)
    assert (host(packed)[5] == 0x88).all()


@pytest.mark.parametrize("per_group", [False, True])
@pytest.mark.parametrize("G", [16, 64, 256])
def test_quantize_weights_matches_oracle(G, per_group):
    """Against the oracle's exact rotation: codes agree to the rotation-codes bar, scales
    within one bf16 step (the absmax can differ by an fp32 rounding)."""
    N, K = 300, 2304
    w = _weights_bf16(N, K, seed=3 * G + per_group)
    packed, scales = ck.quantize_weights(bf16_dev(w), G, per_group)
    ref_p, ref_s = oracle.rotate_quantize_weights(w, G, per_group)
    assert_codes_close(oracle.unpack(host(packed)), oracle.unpack(ref_p))
    s = host(scales.view(torch.int16)).view(np.uint16).astype(np.int32)
    assert np.abs(s - ref_s.astype(np.int32)).max() <= 1
    assert (s == ref_s).mean() >= 0.99


def test_quantize_weights_strided_input_and_small_shapes():
    K, ld = 256, 320                       # padding columns hold NaN
    w = np.full((17, ld), 0x7FC0, dtype=np.uint16)
    w[:, :K] = _weights_bf16(17, K, seed=1)
    wd = bf16_dev(w)[:, :K]
    for G in (16, 64, 256):
        for pg in (False, True):
            p1, s1 = ck.quantize_weights(wd, G, pg)
            p2, s2 = ck.quantize_weights(bf16_dev(np.ascontiguousarray(w[:, :K])), G, pg)
            assert torch.equal(p1, p2) and torch.equal(s1.view(torch.int16), s2.view(torch.int16))
    p, s = ck.quantize_weights(bf16_dev(_weights_bf16(3, 64, seed=2)), 16, True)
    assert tuple(p.shape) == (3, 32) and tuple(s.shape) == (1, 3)


@pytest.mark.parametrize("per_group", [False, True])
def test_produced_weights_run_the_linear(per_group):
    """Weights from the producer feed the linear unchanged: the GPU linear matches the
    oracle epilogue on them, and approximates the unquantised x . W^T."""
    M, N, K, G = 96, 400, 1536, 64
    w = _weights_bf16(N, K, seed=9)
    x = workloads.activations(M, K, seed=9, outliers=15)
    packed, scales = ck.quantize_weights(bf16_dev(w), G, per_group)
    xd = bf16_dev(x)
    out = host(ck.linear(xd, G, 8, packed, scales, per_group))
    codes, rs = ck.rotate_quant(xd, G, 8)
    ref = oracle.gemm_q(host(codes), host(rs), host(packed), host(scales.view(torch.int16)).view(np.uint16),
                        per_group)
    assert_output_close(out, ref)
    # quantisation error of the whole path: as small as with the oracle's own weights
    exact = workloads.bf16_bits_to_f32(x).astype(np.float64) @ workloads.bf16_bits_to_f32(w).astype(np.float64).T
    ref_p, ref_s = oracle.rotate_quantize_weights(w, G, per_group)
    oracle_out, _, _ = oracle.linear(x, G, 8, ref_p, ref_s, per_group)
    err_gpu = np.linalg.norm(out - exact)
    err_oracle = np.linalg.norm(oracle_out - exact)
    assert err_oracle / np.linalg.norm(exact) < 0.3
    assert err_gpu <= 1.05 * err_oracle


# ------------------------------------------------------- AWQ prefill GEMM


def _awq_inputs(M, K, N, seed):
    rng = np.random.default_rng(seed)
    x = workloads.to_bf16_bits(rng.standard_normal((M, K)))
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = workloads.to_bf16_bits(rng.uniform(0.002, 0.02, size=(K // 64, N)))
    z = workloads.to_bf16_bits(rng.normal(0, 0.01, size=(K // 64, N)))
    bias = workloads.to_bf16_bits(rng.standard_normal(N))
    return x, packed, s, z, bias


@pytest.mark.parametrize("M,K,N", [
    (9, 64, 16), (64, 256, 272), (300, 1152, 400), (513, 3072, 256), (257, 128, 528), (1, 640, 48),
])
def test_awq_gemm_matches_oracle(M, K, N):
    x, packed, s, z, bias = _awq_inputs(M, K, N, seed=M + K + N)
    out = host(ck.w4a16_gemm(bf16_dev(x), u8_dev(packed), bf16_dev(s), bf16_dev(z), bias=bf16_dev(bias)))
    ref = oracle.awq_gemm(x, packed, s, z, bias=bias)
    assert_output_close(out, ref)


def test_awq_gemm_without_bias_strided_and_near_the_gemv():
    """No bias, a strided input with NaN padding, and agreement with the exact-weight
    GEMV within W's bf16 rounding at a size both accept."""
    M, K, N, ld = 8, 3072, 512, 3200
    x, packed, s, z, _ = _awq_inputs(M, K, N, seed=3)
    xp = np.full((M, ld), 0x7FC0, dtype=np.uint16)
    xp[:, :K] = x
    xd = bf16_dev(xp)[:, :K]
    g = host(ck.w4a16_gemm(xd, u8_dev(packed), bf16_dev(s), bf16_dev(z)))
    assert np.isfinite(g).all()
    assert_output_close(g, oracle.awq_gemm(x, packed, s, z))
    v = host(ck.w4a16_gemv(xd, u8_dev(packed), bf16_dev(s), bf16_dev(z)))
    wmax = np.abs(workloads.bf16_bits_to_f32(oracle.awq_dequantize(packed, s, z))).max()
    bound = 2 * 2.0 ** -8 * np.abs(workloads.bf16_bits_to_f32(x)).sum(1, keepdims=True) * wmax
    assert (np.abs(g - v) <= bound + 2.0 ** -7 * np.abs(v)).all()


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M,K,N", [(8200, 320, 3856), (1000, 448, 3856)])
def test_gemm_tile_choice_ragged_sampled_rows(M, K, N, bits):
    """Per-channel tiled GEMM on both tile sizes with ragged M and N: 8200 x 3856 takes
    the 256 x 256 tiles (three rounds), 1000 x 3856 the 128 x 128 ones; byte codes
    (ck_w4_gemm_q) and packed W4A4 codes (the whole linear).  Checked on sampled rows
    that include the last tile's against the oracle, and the two code forms against
    each other bit for bit."""
    inp = workloads.linear_inputs(M, K, N, seed=M + N + bits, outliers=4, scale="channel", zero_rows=(M - 1,))
    xd, wd, sd = bf16_dev(inp["x"]), u8_dev(inp["packed"]), bf16_dev(inp["w_scales"])
    codes, scales = ck.rotate_quant(xd, 64, bits)
    out = ck.gemm_q(codes, scales, wd, sd, False)
    rows = np.unique(np.concatenate([np.arange(0, M, 131), np.arange(M - 8, M), [127, 128, 255, 256]]))
    ref = oracle.gemm_q(host(codes)[rows], host(scales)[rows], inp["packed"], inp["w_scales"], False)
    assert_output_close(host(out)[rows], ref)
    if bits == 4:
        assert torch.equal(ck.linear(xd, 64, 4, wd, sd, False), out)


@pytest.mark.parametrize("M,K,N", [(4096, 512, 4096), (4100, 320, 18448), (1024, 320, 18448)])
def test_awq_gemm_large_tiles_sampled_rows(M, K, N):
    """Shapes that fill the chip: 256 x 256 tiles (the prefill configuration; one
    round, and five rounds ragged in M and N) and 128 x 128 tiles where the large
    ones would leave most of their second round idle (1024 x 18448), checked on
    sampled rows that include the last tile's."""
    x, packed, s, z, bias = _awq_inputs(M, K, N, seed=M + N)
    out = host(ck.w4a16_gemm(bf16_dev(x), u8_dev(packed), bf16_dev(s), bf16_dev(z), bias=bf16_dev(bias)))
    rows = np.unique(np.concatenate([np.arange(0, M, 97), np.arange(M - 8, M), [255, 256]]))
    ref = oracle.awq_gemm(x[rows], packed, s, z, bias=bias)
    assert_output_close(out[rows], ref)


# ------------------------------------------------------------ edge shapes


@pytest.mark.parametrize("M,K,N,G", [
    (65, 64, 16, 16),        # first tiled M, a single K step (stage tail of one step)
    (129, 320, 48, 64),      # five K steps: one full stage of four, then a partial one
    (300, 448, 32, 64),      # seven K steps
    (257, 512, 32, 16),      # two full stages: the second stage's DMA is issued whole up front
    (96, 768, 64, 64),       # three stages: the third is issued in parts during the second
    (200, 1088, 48, 64),     # four full stages and a one-step tail
    (70, 32768, 32, 256),    # longest K
])
def test_w4a4_packed_path_edge_shapes(M, K, N, G):
    """The packed W4A4 tiled path at K tails that do not fill a 4-step stage and at the
    longest K, against the oracle epilogue on the GPU's own codes."""
    inp = workloads.linear_inputs(M, K, N, seed=M + K, outliers=3, scale="channel", with_bias=True)
    xd = bf16_dev(inp["x"])
    out = host(ck.linear(xd, G, 4, u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), False,
                         bias=bf16_dev(inp["bias"])))
    codes, scales = ck.rotate_quant(xd, G, 4)
    ref = oracle.gemm_q(host(codes), host(scales), inp["packed"], inp["w_scales"], False, bias=inp["bias"])
    assert_output_close(out, ref)
    codes4, rs = ck.rotate_quant_packed4(xd, G)
    acc = host(ck.accumulators_i32_a4(codes4, K, u8_dev(inp["packed"])))
    assert np.array_equal(acc.astype(np.int64), oracle.int_gemm(host(codes), oracle.unpack(inp["packed"])))


@pytest.mark.parametrize("M,K,N", [
    (33, 64, 16),            # a single K step: only the short last stage
    (20, 32768, 16),         # longest K
    (300, 192, 784),         # one two-step stage, then a short one
    (200, 448, 96),          # three two-step stages, then a short one
])
def test_awq_gemm_edge_shapes(M, K, N):
    x, packed, s, z, bias = _awq_inputs(M, K, N, seed=K + N)
    out = host(ck.w4a16_gemm(bf16_dev(x), u8_dev(packed), bf16_dev(s), bf16_dev(z), bias=bf16_dev(bias)))
    assert_output_close(out, oracle.awq_gemm(x, packed, s, z, bias=bias))


def test_quantize_weights_longest_rows():
    w = _weights_bf16(5, 32768, seed=13, zero_rows=(2,))
    wd = bf16_dev(w)
    for G in (16, 256):
        for pg in (False, True):
            packed, scales = ck.quantize_weights(wd, G, pg)
            ref_p, ref_s = oracle.quantize_weights(host(ck.rotated_f32(wd, G)), pg)
            assert np.array_equal(host(packed), ref_p)
            assert np.array_equal(host(scales.view(torch.int16)).view(np.uint16), ref_s)
