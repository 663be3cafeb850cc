"""Parity at the benchmark workloads' full sizes, through the same entry points
and launch configurations the benchmark times.  Where the oracle cannot
redo the whole product in seconds, it checks sampled rows (always including the
first, last and all-zero rows) exactly as the small-size tests do.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import DEV, assert_codes_close, assert_output_close, bf16_dev, host, u8_dev

pytestmark = pytest.mark.gpu

ck = pytest.importorskip("packed_int4_convrot_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _rows(M, extra=(), n=24, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(n, M), replace=False).tolist()) | {0, M - 1} | set(extra)
    return np.array(sorted(r for r in rows if r < M))


def _linear_case(name, M=None, full=False):
    w = workloads.WORKLOADS[name]
    inp = workloads.workload_inputs(name, M=M)
    per_group = w["scale"] == "group"
    xd = bf16_dev(inp["x"])
    wd, sd = u8_dev(inp["packed"]), bf16_dev(inp["w_scales"])
    out = host(ck.linear(xd, w["G"], w["bits"], wd, sd, per_group))
    codes, scales = ck.rotate_quant(xd, w["G"], w["bits"])
    M_ = inp["x"].shape[0]
    rows = np.arange(M_) if full else _rows(M_, w.get("zero_rows", ()))
    codes_h, scales_h = host(codes)[rows], host(scales)[rows]
    ref_codes, ref_scales = oracle.rotate_quant(inp["x"][rows], w["G"], w["bits"])
    assert_codes_close(codes_h, ref_codes)
    assert np.all(np.abs(scales_h - ref_scales) <= 2.0 ** -20 * ref_scales)
    ref = oracle.gemm_q(codes_h, scales_h, inp["packed"], inp["w_scales"], per_group)
    assert_output_close(out[rows], ref)
    for r in w.get("zero_rows", ()):
        assert not out[r].any()
    return inp, codes, rows


def test_w4a8_linear_m32_k3840_n3840_g64_full():
    _linear_case("w4a8_linear_m32_k3840_n3840_g64", full=True)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_w4a8_decode_gemv_k3840_n10240(M):
    _linear_case("w4a8_decode_gemv_k3840_n10240_g64", M=M, full=True)


def _accumulators_both_layouts(name, inp, codes, rows):
    """int32 accumulators of the tiled GEMM on byte codes and on the packed codes that
    ck_w4a4_linear actually multiplies at this size, exact on the sampled rows."""
    w = workloads.WORKLOADS[name]
    ref = oracle.int_gemm(host(codes)[rows], oracle.unpack(inp["packed"]))
    acc = host(ck.accumulators_i32(codes, u8_dev(inp["packed"])))
    assert np.array_equal(acc[rows].astype(np.int64), ref)
    codes4, _ = ck.rotate_quant_packed4(bf16_dev(inp["x"]), w["G"])
    acc4 = host(ck.accumulators_i32_a4(codes4, w["K"], u8_dev(inp["packed"])))
    assert np.array_equal(acc4[rows].astype(np.int64), ref)


def test_w4a4_linear_m8192_k3840_n3840_g64_sampled():
    name = "w4a4_linear_m8192_k3840_n3840_g64"
    inp, codes, rows = _linear_case(name)
    _accumulators_both_layouts(name, inp, codes, rows)


def test_w4a4_linear_m8192_k10240_n3840_g256_sampled():
    name = "w4a4_linear_m8192_k10240_n3840_g256"
    inp, codes, rows = _linear_case(name)
    assert set(workloads.WORKLOADS[name]["zero_rows"]) <= set(rows.tolist())
    _accumulators_both_layouts(name, inp, codes, rows)


@pytest.mark.parametrize("G", [16, 64, 256])
def test_rotate_quant_m8192_k10240_ld10752_sampled(G):
    name = "rotate_quant_m8192_k10240_ld10752"
    w = workloads.WORKLOADS[name]
    x = workloads.workload_inputs(name)["x"]
    K = w["K"]
    xd = bf16_dev(x)[:, :K]
    assert xd.stride(0) == w["ld"]
    codes, scales = ck.rotate_quant(xd, G, w["bits"])
    rows = _rows(w["M"], n=16, seed=G)
    ref_codes, ref_scales = oracle.rotate_quant(x[rows], G, w["bits"], K=K)
    assert_codes_close(host(codes)[rows], ref_codes)
    s = host(scales)
    assert np.isfinite(s).all() and (s > 0).all()
    assert np.all(np.abs(s[rows] - ref_scales) <= 2.0 ** -20 * ref_scales)
    # given identical rotated inputs the codes are bit-exact (sampled rows)
    xr = host(ck.rotated_f32(xd[torch.from_numpy(rows).to(DEV)], G))
    c2, s2 = oracle.quantize(xr, w["bits"])
    assert np.array_equal(host(codes)[rows], c2) and np.array_equal(s[rows], s2)


def test_awq_w4a16_gemv_m1_k3072_n18432_full():
    d = workloads.workload_inputs("awq_w4a16_gemv_m1_k3072_n18432")
    out = ck.w4a16_gemv(bf16_dev(d["x"]), u8_dev(d["packed"]), bf16_dev(d["scales"]), bf16_dev(d["zeros"]))
    ref = oracle.awq_gemv(d["x"], d["packed"], d["scales"], d["zeros"])
    assert_output_close(host(out), ref)
