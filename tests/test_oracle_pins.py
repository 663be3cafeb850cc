"""Pins for the CPU oracle (no GPU).

The oracle is trusted only through these checks, none of which re-types its
formulas: closed forms of the Hadamard matrix, scipy's Sylvester
construction, a fast Walsh-Hadamard transform written here as a different
algorithm, the hand-worked examples in tests/golden/ (each citing the page it
follows), brute-force numpy products on tiny inputs, and invariants of
rounding (sign symmetry, power-of-two scale invariance, monotonicity).
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16(vals):
    return workloads.to_bf16_bits(np.asarray(vals, dtype=np.float64))


def _f32(bits):
    return workloads.bf16_bits_to_f32(bits)


# ---------------------------------------------------------------- Hadamard


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_matches_scipy_sylvester(G):
    H = oracle.hadamard(G).astype(np.int64)
    assert np.array_equal(H, scipy.linalg.hadamard(G))


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_closed_form(G):
    H = oracle.hadamard(G).astype(np.int64)
    assert np.array_equal(H @ H, G * np.eye(G, dtype=np.int64))  # H_G . H_G = G I
    assert np.array_equal(H, H.T)
    assert set(np.unique(H)) <= {-1, 1}
    assert (H[0] == 1).all() and (H[:, 0] == 1).all()


def test_hadamard_h4_golden():
    assert np.array_equal(oracle.hadamard(4), np.array(_golden("rotate_quant.json")["H4"]))


# ---------------------------------------------------------------- rotation


def _fwht(v):
    """Iterative fast Walsh-Hadamard transform (natural order), fp64."""
    v = np.array(v, dtype=np.float64)
    h = 1
    n = v.shape[-1]
    while h < n:
        v = v.reshape(v.shape[:-1] + (n // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        v = v.reshape(v.shape[:-3] + (n,))
        h *= 2
    return v


@pytest.mark.parametrize("G", [16, 64, 256])
def test_rotate_unit_vectors_give_hadamard_rows(G):
    H = scipy.linalg.hadamard(G)
    for i in (0, 1, 5, G // 2 + 3, G - 1):
        x = np.zeros((1, 3 * G))
        x[0, G + i] = 1.0  # unit vector inside the second group
        xr = oracle.rotate(_bf16(x), G)
        assert np.array_equal(xr[0, :G], np.zeros(G, np.float32))
        assert np.array_equal(xr[0, 2 * G:], np.zeros(G, np.float32))
        assert np.array_equal(xr[0, G:2 * G], (H[i] / np.sqrt(G)).astype(np.float32))


@pytest.mark.parametrize("G", [16, 64, 256])
def test_rotate_constant_group_is_single_spike(G):
    x = np.full((2, G), 1.5)
    x[1] = -0.375
    xr = oracle.rotate(_bf16(x), G)
    assert xr[0, 0] == np.float32(1.5 * np.sqrt(G)) and xr[1, 0] == np.float32(-0.375 * np.sqrt(G))
    assert not xr[:, 1:].any()


def test_rotate_g1_is_identity():
    x = workloads.activations(3, 40, seed=11, outliers=2)
    assert np.array_equal(oracle.rotate(x, 1), _f32(x))


@pytest.mark.parametrize("G", [16, 64, 256])
def test_rotate_matches_block_diagonal_scipy_product(G):
    K = 4 * G
    x = workloads.activations(5, K, seed=G, outliers=3)
    ref = _f32(x).astype(np.float64) @ scipy.linalg.block_diag(*[scipy.linalg.hadamard(G)] * 4)
    ref = (ref / np.sqrt(G)).astype(np.float32)
    assert np.array_equal(oracle.rotate(x, G), ref)


@pytest.mark.parametrize("G", [16, 64, 256])
def test_rotate_matches_fast_transform(G):
    K = 3 * G
    x = workloads.activations(4, K, seed=100 + G, outliers=2)
    xf = _f32(x).astype(np.float64).reshape(4, K // G, G)
    ref = (_fwht(xf) / np.sqrt(G)).reshape(4, K).astype(np.float32)
    assert np.array_equal(oracle.rotate(x, G), ref)


@pytest.mark.parametrize("G", [16, 64, 256])
def test_rotate_preserves_group_norms(G):
    x = workloads.activations(6, 2 * G, seed=7, outliers=1)
    xr = oracle.rotate(x, G).astype(np.float64).reshape(6, 2, G)
    xf = _f32(x).astype(np.float64).reshape(6, 2, G)
    np.testing.assert_allclose((xr ** 2).sum(-1), (xf ** 2).sum(-1), rtol=1e-6)


def test_rotate_strided_rows_ignore_padding():
    x = workloads.activations(3, 128, seed=5, outliers=1, ld=192)  # NaN padding columns
    xr = oracle.rotate(x, 64, K=128)
    assert np.isfinite(xr).all()
    assert np.array_equal(xr, oracle.rotate(np.ascontiguousarray(x[:, :128]), 64))


# ------------------------------------------------------------ quantisation


def _golden_case_x(case):
    if "x_constant" in case:
        return np.full((1, case["K"]), case["x_constant"])
    return np.asarray([case["x"]], dtype=np.float64)


@pytest.mark.parametrize("case", _golden("rotate_quant.json")["cases"], ids=lambda c: c["name"])
def test_rotate_quant_golden(case):
    x = _bf16(_golden_case_x(case))
    assert np.array_equal(_f32(x), _golden_case_x(case).astype(np.float32))  # inputs exact in bf16
    xr = oracle.rotate(x, case["G"])
    codes, scales = oracle.quantize(xr, case["bits"])
    if "xr" in case:
        assert np.array_equal(xr[0], np.asarray(case["xr"], dtype=np.float32))
        assert np.array_equal(codes[0], np.asarray(case["codes"], dtype=np.int8))
    else:
        assert xr[0, 0] == case["xr_first"] and (xr[0, 1:] == case["xr_rest"]).all()
        assert codes[0, 0] == case["codes_first"] and (codes[0, 1:] == case["codes_rest"]).all()
    expect = case["scale_num"] / case["scale_den"]
    assert abs(float(scales[0]) - expect) <= 2 ** -23 * expect


@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_properties(bits):
    qmax = oracle.QMAX[bits]
    x = workloads.activations(64, 512, seed=21, outliers=5, zero_rows=(3, 40))
    xr = oracle.rotate(x, 64)
    codes, s = oracle.quantize(xr, bits)
    nz = np.abs(xr).max(1) > 0
    assert (np.abs(codes[nz]).max(1) == qmax).all()          # the absmax maps to +-qmax
    assert (np.abs(codes.astype(int)) <= qmax).all()
    # each code is the nearest integer to xr/s (up to fp32 rounding)
    err = np.abs(xr[nz] / s[nz, None] - codes[nz])
    assert err.max() <= 0.5 + 1e-4
    # zero rows: codes 0 and the positive placeholder scale
    assert not codes[~nz].any() and (s[~nz] == 1.0).all()
    # rounding is symmetric, monotone and invariant under power-of-two scaling
    c2, s2 = oracle.quantize(-xr, bits)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, s)
    c3, s3 = oracle.quantize(xr * np.float32(8.0), bits)
    assert np.array_equal(c3, codes) and np.array_equal(s3[nz], s[nz] * np.float32(8.0))
    order = np.argsort(xr[1])
    assert (np.diff(codes[1][order].astype(int)) >= 0).all()


# -------------------------------------------------------------------- codec


def test_codec_golden_bytes():
    g = _golden("codec.json")
    for e in g["bytes"]:
        w = oracle.unpack(np.array([[e["byte"]]], dtype=np.uint8))
        assert w.tolist() == [[e["col_even_value"], e["col_odd_value"]]]
    for r in g["rows"]:
        assert oracle.unpack(np.array([r["packed"]], dtype=np.uint8)).tolist() == [r["values"]]


def test_codec_round_trip_all_bytes():
    allb = np.arange(256, dtype=np.uint8).reshape(1, 256)
    w = oracle.unpack(allb).astype(np.int64) + 8
    assert w.min() == 0 and w.max() == 15
    repacked = (w[:, 0::2] | (w[:, 1::2] << 4)).astype(np.uint8)  # independent packer
    assert np.array_equal(repacked, allb)


def test_codec_random_matrix_and_stride():
    p = workloads.packed_weights(7, 96, seed=3, ld=64)   # 48 data bytes + 16 padding bytes
    w = oracle.unpack(p, 96)
    assert w.shape == (7, 96)
    lo = (p[:, :48] & 0xF).astype(int) - 8
    hi = (p[:, :48] >> 4).astype(int) - 8
    assert np.array_equal(w[:, 0::2], lo) and np.array_equal(w[:, 1::2], hi)


# ----------------------------------------------------- integer matmul + epilogue


def test_int_gemm_matches_numpy_matmul():
    rng = np.random.default_rng(0)
    codes = rng.integers(-127, 128, size=(5, 192), dtype=np.int8)
    w = rng.integers(-8, 8, size=(9, 192), dtype=np.int8)
    ref = codes.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(oracle.int_gemm(codes, w), ref)
    per_g = oracle.int_gemm(codes, w, 64)
    assert per_g.shape == (5, 9, 3)
    assert np.array_equal(per_g.sum(-1), ref)
    assert np.array_equal(per_g[:, :, 1], codes[:, 64:128].astype(np.int64) @ w[:, 64:128].astype(np.int64).T)


def test_linear_golden():
    g = _golden("linear.json")
    x = _bf16([g["x"]])
    codes, sx = oracle.rotate_quant(x, g["G"], g["bits"])
    packed = np.array(g["packed"], dtype=np.uint8)
    w = oracle.unpack(packed)
    assert oracle.int_gemm(codes, w)[0].tolist() == g["acc"]
    assert oracle.int_gemm(codes, w, g["per_group"]["Gw"])[0].tolist() == g["per_group"]["acc_groups"]
    expect_sx = g["sx_num"] / g["sx_den"]
    assert abs(float(sx[0]) - expect_sx) <= 2 ** -23 * expect_sx
    pc = oracle.gemm_q(codes, sx, packed, _bf16(g["per_channel"]["w_scales"]), per_group=False)
    np.testing.assert_allclose(pc[0], float(sx[0]) * np.array(g["per_channel"]["out_over_sx"]), rtol=1e-15)
    pg = oracle.gemm_q(codes, sx, packed, _bf16(g["per_group"]["w_scales"]), per_group=True,
                       Gw=g["per_group"]["Gw"])
    np.testing.assert_allclose(pg[0], float(sx[0]) * np.array(g["per_group"]["out_over_sx"]), rtol=1e-15)


@pytest.mark.parametrize("per_group", [False, True])
def test_epilogue_equals_dequantised_fp64_matmul(per_group):
    """Integer path scaled by s_x * s_w equals dequantise-then-matmul in fp64."""
    M, K, N, Gw = 6, 256, 10, 64   # K/Gw = 4 != N, so a transposed scale index fails
    inp = workloads.linear_inputs(M, K, N, seed=9, outliers=3, scale="group" if per_group else "channel",
                                  with_bias=True)
    out, codes, sx = oracle.linear(inp["x"], 64, 8, inp["packed"], inp["w_scales"], per_group,
                                   bias=inp["bias"])
    w = oracle.unpack(inp["packed"]).astype(np.float64)
    s_w = _f32(inp["w_scales"]).astype(np.float64)
    if per_group:
        w_deq = w * np.repeat(s_w.T, Gw, axis=1)   # W[n,k] = (q-8) * s_w[k // Gw, n]
    else:
        w_deq = w * s_w[:, None]
    a_deq = codes.astype(np.float64) * sx.astype(np.float64)[:, None]
    ref = a_deq @ w_deq.T + _f32(inp["bias"]).astype(np.float64)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_x_scale_golden():
    """Input scale (hand-worked, tests/golden/x_scale.json): the row scale is multiplied
    by x_scale and the bias is added unscaled."""
    g = _golden("x_scale.json")
    x = np.zeros((1, g["K"]))
    x[0, g["x_nonzero"]["index"]] = g["x_nonzero"]["value"]
    x = _bf16(x)
    packed = np.array([[b] * (g["K"] // 2) for b in g["packed_row_bytes"]], dtype=np.uint8)
    sx_exact = sum(2.0 ** e for e in g["sx_f32_terms_pow2"])
    ws, bias = _bf16(g["w_scales"]), _bf16(g["bias"])
    for case in g["cases"]:
        out, codes, sx = oracle.linear(x, g["G"], g["bits"], packed, ws, False, bias=bias,
                                       x_scale=case["x_scale"])
        assert (codes == 127).all() and float(sx[0]) == sx_exact
        assert oracle.int_gemm(codes, oracle.unpack(packed))[0].tolist() == g["acc"]
        if "out" in case:
            np.testing.assert_allclose(out[0], case["out"], rtol=1e-15)
        else:
            assert out[0].tolist() == [4 * sx_exact * 4064 + 1, -4 * sx_exact * 1016 - 2]


@pytest.mark.parametrize("alpha", [0.25, 4.0, 64.0])
def test_x_scale_power_of_two_equals_linear_of_scaled_input(alpha):
    """For a power-of-two input scale, alpha * x is exact in bf16 and the linear of it
    (computed from that input, scale 1) is bit-identical to the linear of x at scale alpha."""
    M, K, N = 5, 512, 24
    for per_group in (False, True):
        inp = workloads.linear_inputs(M, K, N, seed=11, outliers=3, scale="group" if per_group else "channel",
                                      zero_rows=(2,), with_bias=True)
        scaled = _bf16(_f32(inp["x"]).astype(np.float64) * alpha)
        assert np.array_equal(_f32(scaled), _f32(inp["x"]) * np.float32(alpha))
        for bits in (8, 4):
            a = oracle.linear(inp["x"], 64, bits, inp["packed"], inp["w_scales"], per_group, bias=inp["bias"],
                              x_scale=alpha)
            b = oracle.linear(scaled, 64, bits, inp["packed"], inp["w_scales"], per_group, bias=inp["bias"])
            assert np.array_equal(a[1], b[1]) and np.array_equal(a[0], b[0])


@pytest.mark.parametrize("alpha", [0.3, 3.0, 1.7e-3])
def test_x_scale_equals_dequantised_product_of_scaled_activations(alpha):
    """Any positive scale: the output equals (alpha * s_x * codes) . (s_w * w)^T + bias by
    a dequantise-then-matmul route in numpy, and approximates (alpha * x) . W^T."""
    M, K, N = 7, 256, 10
    inp = workloads.linear_inputs(M, K, N, seed=5, outliers=2, scale="group", with_bias=True)
    out, codes, sx = oracle.linear(inp["x"], 64, 8, inp["packed"], inp["w_scales"], True, bias=inp["bias"],
                                   x_scale=alpha)
    w = oracle.unpack(inp["packed"]).astype(np.float64) * np.repeat(_f32(inp["w_scales"]).T, 64, axis=1)
    a_deq = alpha * codes.astype(np.float64) * sx.astype(np.float64)[:, None]
    np.testing.assert_allclose(out, a_deq @ w.T + _f32(inp["bias"]).astype(np.float64), rtol=1e-12, atol=1e-12)
    # against the unquantised linear of the scaled input (rotation undone on the
    # dequantised activations): the error is the activation quantisation error, scaled by alpha
    H = scipy.linalg.hadamard(64) / 8.0
    x_rot = _f32(inp["x"]).astype(np.float64).reshape(M, K // 64, 64) @ H
    exact = alpha * x_rot.reshape(M, K) @ w.T + _f32(inp["bias"]).astype(np.float64)
    bound = alpha * (sx.astype(np.float64)[:, None] / 2 * (1 + 2.0 ** -20)) @ np.abs(w).sum(1)[None, :]
    bound += alpha * 2.0 ** -24 * np.abs(x_rot.reshape(M, K)) @ np.abs(w).T   # fp32 rounding of the rotation
    assert (np.abs(out - exact) <= bound + 1e-12).all()


def test_x_scale_rejects_non_positive():
    inp = workloads.linear_inputs(1, 64, 2, seed=1, outliers=0, scale="channel")
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            oracle.linear(inp["x"], 64, 8, inp["packed"], inp["w_scales"], False, x_scale=bad)


def test_linear_zero_rows_give_bias_only():
    inp = workloads.linear_inputs(4, 128, 16, seed=1, outliers=0, scale="group", zero_rows=(2,),
                                  with_bias=True)
    out, codes, sx = oracle.linear(inp["x"], 64, 4, inp["packed"], inp["w_scales"], True, bias=inp["bias"])
    assert sx[2] == 1.0 and not codes[2].any()
    assert np.array_equal(out[2], _f32(inp["bias"]).astype(np.float64))


# --------------------------------------------------------------------- AWQ


def test_awq_golden():
    g = _golden("awq.json")
    args = (_bf16([g["x"]]), np.array(g["packed"], dtype=np.uint8), _bf16(g["scales"]), _bf16(g["zeros"]))
    assert oracle.awq_gemv(*args, Gw=g["Gw"])[0].tolist() == g["y"]
    assert oracle.awq_gemv(*args, Gw=g["Gw"], bias=_bf16(g["bias"]))[0].tolist() == g["y_bias"]


def test_awq_unit_vectors_return_dequantised_columns():
    d = workloads.awq_inputs(1, 256, 24, seed=5)
    q = oracle.unpack(d["packed"]).astype(np.float64)
    s = _f32(d["scales"]).astype(np.float64)
    z = _f32(d["zeros"]).astype(np.float64)
    for k in (0, 1, 63, 64, 130, 255):
        e = np.zeros((1, 256))
        e[0, k] = 1.0
        col = oracle.awq_gemv(_bf16(e), d["packed"], d["scales"], d["zeros"])[0]
        np.testing.assert_array_equal(col, q[:, k] * s[k // 64] + z[k // 64])


def test_awq_matches_numpy_brute_force():
    d = workloads.awq_inputs(3, 192, 20, seed=8, with_bias=True)
    q = oracle.unpack(d["packed"]).astype(np.float64)
    W = q * np.repeat(_f32(d["scales"]).T, 64, 1) + np.repeat(_f32(d["zeros"]).T, 64, 1)
    ref = _f32(d["x"]).astype(np.float64) @ W.T + _f32(d["bias"])
    np.testing.assert_allclose(oracle.awq_gemv(d["x"], d["packed"], d["scales"], d["zeros"], bias=d["bias"]),
                               ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- weight quantiser


def _impulse_rows(d):
    w = np.zeros((len(d["impulses"]), d["K"]), dtype=np.float64)
    for r, c, v in d["impulses"]:
        w[r, c] = v
    return _bf16(w)


@pytest.mark.parametrize("per_group", [False, True])
def test_weight_quant_golden(per_group):
    d = _golden("weight_quant.json")
    packed, scales = oracle.rotate_quantize_weights(_impulse_rows(d), d["G"], per_group)
    want = np.array([list(bytes.fromhex(h)) for h in d["packed_rows_hex"]], dtype=np.uint8)
    assert np.array_equal(packed, want)
    ref = d["scales_per_group"] if per_group else d["scales_per_channel"]
    assert np.array_equal(scales, np.array([[int(v, 16) for v in r] for r in ref] if per_group
                                           else [int(v, 16) for v in ref], dtype=np.uint16))


def _unpacked(packed):
    return oracle.unpack(packed).astype(np.int64)


@pytest.mark.parametrize("per_group", [False, True])
def test_weight_quant_exact_round_trip(per_group):
    """Rotated weights that are exactly code * s (s a bf16 value, every group holding a
    +-7) come back as those codes and that scale."""
    rng = np.random.default_rng(5)
    N, K, Gw = 7, 256, 64
    ng = K // Gw if per_group else 1
    glen = Gw if per_group else K
    codes = rng.integers(-7, 8, size=(N, K))
    codes[:, ::glen] = np.where(rng.random((N, K // glen)) < 0.5, -7, 7)  # the absmax in every group
    s_bits = _bf16(rng.uniform(1e-3, 3.0, size=(N, ng)))
    s = _f32(s_bits).astype(np.float64)
    wr = (codes * np.repeat(s, glen, axis=1)).astype(np.float32)
    assert np.array_equal(wr.astype(np.float64), codes * np.repeat(s, glen, axis=1))  # exact in fp32
    packed, scales = oracle.quantize_weights(wr, per_group, Gw)
    assert np.array_equal(_unpacked(packed), codes)
    assert np.array_equal(scales, s_bits.T if per_group else s_bits[:, 0])


@pytest.mark.parametrize("per_group", [False, True])
def test_weight_quant_error_bound_and_range(per_group):
    """Every value lands within half a step of code * s; the group absmax maps to +-7;
    stored codes are 1..15 (never 0); an all-zero group gets scale 0 and code 0."""
    rng = np.random.default_rng(11)
    N, K, Gw = 9, 512, 64
    wr = (rng.standard_normal((N, K)) * rng.uniform(0.01, 10.0, size=(N, 1))).astype(np.float32)
    wr[3] = 0.0
    wr[4, :Gw] = 0.0
    packed, scales = oracle.quantize_weights(wr, per_group, Gw)
    q = oracle.unpack(packed).astype(np.int64) + 8
    assert q.min() >= 1 and q.max() <= 15
    glen = Gw if per_group else K
    s = _f32(scales.T if per_group else scales[:, None]).astype(np.float64)
    s_full = np.repeat(s, glen, axis=1)
    codes = q - 8
    err = np.abs(wr.astype(np.float64) - codes * s_full)
    assert (err <= 0.5 * s_full * (1 + 1e-6) + 1e-30).all()
    a = np.abs(wr).reshape(N, K // glen, glen).max(-1)
    c = np.abs(codes).reshape(N, K // glen, glen).max(-1)
    assert (c[a > 0] == 7).all() and (c[a == 0] == 0).all()
    assert (s[a == 0] == 0).all() and (s[a > 0] > 0).all()
    # scale is the bf16 rounding of a / 7: within half a bf16 step
    assert (np.abs(s[a > 0] - a[a > 0] / 7.0) <= 2.0 ** -8 * a[a > 0] / 7.0 * 1.0001).all()


@pytest.mark.parametrize("G", [16, 64, 256])
@pytest.mark.parametrize("per_group", [False, True])
def test_weight_producer_gives_the_linear_of_w(G, per_group):
    """Rotating both sides by the same H_G leaves x . W^T unchanged, so the linear with
    produced weights approximates the unquantised product; pairing weights rotated
    with one G and activations rotated with another does not."""
    rng = np.random.default_rng(G)
    M, N, K = 6, 48, 512
    x = _bf16(rng.standard_normal((M, K)))
    W = _bf16(rng.standard_normal((N, K)) * 0.05)
    ref = _f32(x).astype(np.float64) @ _f32(W).astype(np.float64).T
    packed, scales = oracle.rotate_quantize_weights(W, G, per_group)
    out, _, _ = oracle.linear(x, G, 8, packed, scales, per_group)
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 0.15, rel
    other = 16 if G != 16 else 64
    bad, _, _ = oracle.linear(x, other, 8, packed, scales, per_group)
    assert np.linalg.norm(bad - ref) / np.linalg.norm(ref) > 0.5


# ------------------------------------------------ AWQ dequantise (prefill)


def _hexes(rows):
    return np.array([[int(v, 16) for v in r] for r in rows], dtype=np.uint16)


def test_awq_dequantize_golden():
    d = _golden("awq_dequantize.json")
    w = oracle.awq_dequantize(np.array(d["packed"], dtype=np.uint8), _hexes(d["scales"]), _hexes(d["zeros"]),
                              d["Gw"])
    assert np.array_equal(w, _hexes(d["W"]))
    y = oracle.awq_gemm(_bf16([d["x"]]), np.array(d["packed"], dtype=np.uint8), _hexes(d["scales"]),
                        _hexes(d["zeros"]), d["Gw"])
    assert np.array_equal(y[0], np.array(d["y"]))


def test_awq_dequantize_is_the_rounded_exact_weight():
    """Every dequantised weight is within one bf16 rounding of each step of the exact
    (q - 8) s + z, and equals it whenever the exact value is a bf16 number."""
    rng = np.random.default_rng(21)
    N, K, Gw = 16, 256, 64
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = _bf16(rng.uniform(0.002, 0.02, size=(K // Gw, N)))
    z = _bf16(rng.normal(0, 0.01, size=(K // Gw, N)))
    w = _f32(oracle.awq_dequantize(packed, s, z, Gw)).astype(np.float64)
    q = oracle.unpack(packed).astype(np.float64)
    S = np.repeat(_f32(s).astype(np.float64).T, Gw, axis=1)
    Z = np.repeat(_f32(z).astype(np.float64).T, Gw, axis=1)
    exact = q * S + Z
    # two roundings of at most half a bf16 step each (relative 2^-8 of the value rounded)
    bound = 2.0 ** -8 * (np.abs(q * S) + np.abs(exact)) * 1.0001 + 1e-30
    assert (np.abs(w - exact) <= bound).all()
    # zero scale and zero point -> exact products
    z0 = np.zeros_like(z)
    s1 = _bf16(np.full((K // Gw, N), 0.25))
    assert np.array_equal(_f32(oracle.awq_dequantize(packed, s1, z0, Gw)).astype(np.float64), q * 0.25)


def test_awq_gemm_brute_force_and_near_the_exact_product():
    rng = np.random.default_rng(22)
    M, N, K, Gw = 5, 12, 128, 64
    x = _bf16(rng.standard_normal((M, K)))
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = _bf16(rng.uniform(0.002, 0.02, size=(K // Gw, N)))
    z = _bf16(rng.normal(0, 0.01, size=(K // Gw, N)))
    bias = _bf16(rng.standard_normal(N))
    y = oracle.awq_gemm(x, packed, s, z, Gw, bias=bias)
    w = _f32(oracle.awq_dequantize(packed, s, z, Gw)).astype(np.float64)
    ref = _f32(x).astype(np.float64) @ w.T + _f32(bias).astype(np.float64)
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)
    exact = oracle.awq_gemv(x, packed, s, z, Gw, bias=bias)
    wmax = np.abs(w).max()
    assert np.abs(y - exact).max() <= 2 * 2.0 ** -8 * np.abs(_f32(x)).sum(1).max() * wmax
