"""The allocation-free W4A4 linear (ck_w4a4_linear_noalloc) against ck_w4a4_linear.

Both run the same kernels; the only difference is where the codes and row scales
live (the library's static per-GPU scratch instead of a caller workspace), so the
outputs must be bit-identical.  Two calls in a row, the second with a smaller
input, check that the shared scratch carries nothing over from one call to the
next; the results are also held to the oracle's bar.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import DEV, assert_output_close, bf16_dev, host, u8_dev

pytestmark = pytest.mark.gpu

ck = pytest.importorskip("packed_int4_convrot_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(M, K, N, G, per_group, seed):
    inp = workloads.linear_inputs(M, K, N, seed=seed, outliers=max(1, K // 200),
                                  scale="group" if per_group else "channel", zero_rows=(M - 1,) if M > 2 else (),
                                  with_bias=True)
    args = (bf16_dev(inp["x"]), G, u8_dev(inp["packed"]), bf16_dev(inp["w_scales"]), per_group)
    return inp, args


@pytest.mark.parametrize("per_group", [False, True])
def test_noalloc_equals_workspace_linear_two_calls(per_group):
    # first call: tiled GEMM on packed codes (M > 64); second, smaller: the few-row
    # kernel on byte codes; third: the fused decode launch (no scratch at all)
    for i, (M, K, N, G) in enumerate([(300, 2304, 400, 256), (40, 1024, 272, 64), (1, 3840, 256, 64)]):
        inp, args = _case(M, K, N, G, per_group, seed=100 + i)
        bias = bf16_dev(inp["bias"])
        print("noalloc case M=%d K=%d N=%d G=%d per_group=%s" % (M, K, N, G, per_group), flush=True)
        a = ck.w4a4_linear_noalloc(*args, bias=bias)
        b = ck.linear(args[0], G, 4, *args[2:], bias=bias)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        codes, scales = ck.rotate_quant(args[0], G, 4)
        ref = oracle.gemm_q(host(codes), host(scales), inp["packed"], inp["w_scales"], per_group, bias=inp["bias"])
        assert_output_close(host(a), ref)


def test_noalloc_workload_size_and_back():
    """The K = 3840, M = 8192 W4A4 workload (15.7 MB of packed codes) fits the scratch;
    a later small call on the same scratch is still exact."""
    name = "w4a4_linear_m8192_k3840_n3840_g64"
    w = workloads.WORKLOADS[name]
    inp = workloads.workload_inputs(name)
    xd, wd, sd = bf16_dev(inp["x"]), u8_dev(inp["packed"]), bf16_dev(inp["w_scales"])
    print("noalloc workload %s" % name, flush=True)
    a = ck.w4a4_linear_noalloc(xd, w["G"], wd, sd, False)
    b = ck.linear(xd, w["G"], 4, wd, sd, False)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    small = xd[:70]
    a2 = ck.w4a4_linear_noalloc(small, w["G"], wd, sd, False)
    assert torch.equal(a2.view(torch.int16), b[:70].view(torch.int16))


def test_noalloc_rejects_beyond_scratch():
    x = torch.zeros((8192, 32768), dtype=torch.bfloat16, device=DEV)
    packed = torch.zeros((16, 16384), dtype=torch.uint8, device=DEV)
    with pytest.raises(ck.CKError, match="static scratch"):
        ck.w4a4_linear_noalloc(x, 64, packed, torch.ones(16, dtype=torch.bfloat16, device=DEV), False)
