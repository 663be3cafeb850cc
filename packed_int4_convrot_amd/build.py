"""Build libck.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m packed_int4_convrot_amd.build

Kernels are compiled with hipcc for gfx950 only.  Packed-fp32 VALU forms are
switched off (-Xclang -target-feature -Xclang -packed-fp32-ops) and
floating-point contraction is off, so every fp32 rounding step in the kernels
is the one written in the source.  The C ABI layer (ck_api.cpp) is plain host
C++ compiled with g++.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import json
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libck.so")

HIP_SOURCES = ["rotate_quant.hip", "w4_gemv.hip", "w4_gemv_fused.hip", "w4_skinny.hip", "w4_skinny_fused.hip", "w4_gemm.hip", "w4a16_gemv.hip",
               "awq_gemm.hip", "static_scratch.hip"]
CXX_SOURCES = ["ck_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed: %s\n%s" % (" ".join(cmd), out))
    return out


RESOURCE_REPORT = os.path.join(BUILD, "resource_usage.json")
_FIELDS = {"VGPRs": "vgpr", "AGPRs": "agpr", "SGPRs": "sgpr", "ScratchSize [bytes/lane]": "scratch",
           "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill", "LDS Size [bytes/block]": "lds",
           "Occupancy [waves/SIMD]": "occupancy"}


def _resource_usage(src, text):
    """Per-kernel records from the compiler's kernel-resource-usage remarks."""
    recs, cur = [], None
    for line in text.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].split("[-Rpass", 1)[0].strip()
        if body.startswith("Function Name:"):
            cur = {"source": src, "kernel": body.split(":", 1)[1].strip()}
            recs.append(cur)
        elif cur is not None and ":" in body:
            key, val = (t.strip() for t in body.split(":", 1))
            if key in _FIELDS:
                cur[_FIELDS[key]] = int(val)
    return recs


def sources_sha() -> str:
    h = hashlib.sha256()
    for src in HIP_SOURCES + CXX_SOURCES + sorted(f for f in os.listdir(CSRC) if f.endswith(".h")):
        with open(os.path.join(CSRC, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([HIPCC, *HIP_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src),
                     "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        objs.append(obj)
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    usage = []
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        for src, out in zip(HIP_SOURCES + CXX_SOURCES, ex.map(_run, jobs)):
            usage += _resource_usage(src, out)
            text = "\n".join(l for l in out.splitlines() if "remark:" not in l)
            if verbose and text.strip():
                print(text)
    with open(RESOURCE_REPORT, "w") as f:
        json.dump({"sources_sha": sources_sha(), "kernels": usage}, f, indent=1)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
