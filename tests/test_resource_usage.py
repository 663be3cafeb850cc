"""Register budget of the gfx950 kernels, from the compiler's resource-usage
remarks that the build records (packed_int4_convrot_amd/_build/resource_usage.json):
no kernel may use scratch memory or spill registers, since a spill puts a
round trip to memory into every iteration of the loop it sits in."""
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORT = os.path.join(ROOT, "packed_int4_convrot_amd", "_build", "resource_usage.json")


def _report():
    if not os.path.exists(REPORT):
        pytest.skip("library not built (python -m packed_int4_convrot_amd.build)")
    import importlib.util
    spec = importlib.util.spec_from_file_location("_ck_build", os.path.join(ROOT, "packed_int4_convrot_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with open(REPORT) as f:
        rep = json.load(f)
    assert rep["sources_sha"] == mod.sources_sha(), "resource report is older than the sources: rebuild"
    return rep


def test_every_hot_kernel_is_reported():
    names = " ".join(k["kernel"] for k in _report()["kernels"])
    for kernel in ("rotate_quant_kernel", "w4_gemv_kernel", "w4_skinny_kernel", "w4_gemm_kernel",
                   "w4a16_gemv_kernel", "awq_gemm_kernel", "w4_gemv_fused_kernel", "w4_skinny_fused_kernel"):
        assert kernel in names, kernel


def test_no_scratch_and_no_spills():
    bad = [(k["source"], k["kernel"], k.get("scratch"), k.get("vgpr_spill"), k.get("sgpr_spill"))
           for k in _report()["kernels"]
           if k.get("scratch", 0) or k.get("vgpr_spill", 0) or k.get("sgpr_spill", 0)]
    assert not bad, bad


def test_register_counts_within_the_file():
    for k in _report()["kernels"]:
        assert k["vgpr"] + k.get("agpr", 0) <= 512, k
        assert k["lds"] <= 160 * 1024, k
