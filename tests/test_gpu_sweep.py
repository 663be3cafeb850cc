"""Seeded sweep over random shapes within the documented limits: every matmul entry
point against the oracle, the same acceptance as the parity tests.  The shapes come
from one fixed generator, so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_codes_close, assert_output_close, bf16_dev, host, i8_dev, u8_dev

pytestmark = pytest.mark.gpu

ck = pytest.importorskip("packed_int4_convrot_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """uint8 [M, K/2] two's-complement nibble pairs -> int8 [M, K] (column 2j low)."""
    lo = (b & 0x0F).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    out = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int16)
    out[:, 0::2] = lo - 16 * (lo >= 8)
    out[:, 1::2] = hi - 16 * (hi >= 8)
    return out.astype(np.int8)


def _cases(n, seed):
    """n random (M, K, N, G, bits, per_group, bias) with K % G == 0 and N % 16 == 0.  M
    spans every kernel the shape rules pick (GEMV, few-row MFMA, tiled GEMM)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        G = int(rng.choice([16, 64, 256]))
        K = 64 * int(rng.integers(1, 48))
        K = max(K // G, 1) * G if K % G else K
        M = int(rng.choice([1, 2, 3, 5, 6, 8, 9, 17, 33, 64, 65, 129, 200, 257, 300]))
        N = 16 * int(rng.integers(1, 40))
        out.append((M, K, N, G, int(rng.choice([8, 4])), bool(rng.integers(0, 2)), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("M,K,N,G,bits,per_group,with_bias", _cases(24, seed=2026))
def test_linear_random_shapes(M, K, N, G, bits, per_group, with_bias):
    inp = workloads.linear_inputs(M, K, N, seed=M * 7 + K + N, outliers=max(1, K // 200),
                                  scale="group" if per_group else "channel",
                                  zero_rows=(M - 1,) if M > 3 else (), with_bias=with_bias)
    xd = bf16_dev(inp["x"])
    bias = bf16_dev(inp["bias"]) if with_bias else None
    out = host(ck.linear(xd, G, bits, u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), per_group, bias=bias))
    codes, scales = ck.rotate_quant(xd, G, bits)
    codes, scales = host(codes), host(scales)
    ref_codes, _ = oracle.rotate_quant(inp["x"], G, bits)
    # at least 99.99% equal, i.e. one code off by 1 allowed below 10^4 codes
    assert_codes_close(codes, ref_codes, min_equal=1.0 - max(1.0, 1e-4 * codes.size) / codes.size)
    ref = oracle.gemm_q(codes, scales, inp["packed"], inp["w_scales"], per_group, bias=inp["bias"])
    assert_output_close(out, ref)
    # the integer accumulators of the kernel that serves this M, exactly
    acc = host(ck.accumulators_i32(i8_dev(codes), u8_dev(inp["packed"])))
    assert np.array_equal(acc.astype(np.int64), oracle.int_gemm(codes, oracle.unpack(inp["packed"])))


@pytest.mark.parametrize("M,K,N,G,bits,per_group,with_bias", _cases(12, seed=7))
def test_packed_w4a4_random_shapes(M, K, N, G, bits, per_group, with_bias):  # bits: always 4 here
    """The packed-code half-steps on random shapes: codes equal the byte codes, and the
    tiled GEMM on them equals the oracle epilogue."""
    inp = workloads.linear_inputs(M, K, N, seed=M + 3 * K + N, outliers=2, scale="group" if per_group else "channel",
                                  with_bias=with_bias)
    xd = bf16_dev(inp["x"])
    c8, s8 = ck.rotate_quant(xd, G, 4)
    c4, s4 = ck.rotate_quant_packed4(xd, G)
    assert np.array_equal(_unpack_nibbles(host(c4)), host(c8))
    assert np.array_equal(host(s4), host(s8))
    bias = bf16_dev(inp["bias"]) if with_bias else None
    out = host(ck.gemm_packed4(c4, s4, u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), per_group, bias=bias))
    ref = oracle.gemm_q(host(c8), host(s8), inp["packed"], inp["w_scales"], per_group, bias=inp["bias"])
    assert_output_close(out, ref)


def _awq_cases(n, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.choice([1, 2, 4, 8, 9, 40, 130, 257])), 64 * int(rng.integers(1, 40)), 16 * int(rng.integers(1, 40)),
             bool(rng.integers(0, 2))) for _ in range(n)]


@pytest.mark.parametrize("M,K,N,with_bias", _awq_cases(12, seed=11))
def test_awq_random_shapes(M, K, N, with_bias):
    d = workloads.awq_inputs(M, K, N, seed=M + K + N, with_bias=with_bias)
    args = (bf16_dev(d["x"]), u8_dev(d["packed"]), bf16_dev(d["scales"]), bf16_dev(d["zeros"]))
    bias = bf16_dev(d["bias"]) if with_bias else None
    g = host(ck.w4a16_gemm(*args, bias=bias))
    assert_output_close(g, oracle.awq_gemm(d["x"], d["packed"], d["scales"], d["zeros"], bias=d["bias"]))
    if M <= 8 and K <= 16384:
        v = host(ck.w4a16_gemv(*args, bias=bias))
        assert_output_close(v, oracle.awq_gemv(d["x"], d["packed"], d["scales"], d["zeros"], bias=d["bias"]))
