"""Benchmark of the ConvRot packed-INT4 linear on one MI355X.

Headline step: the W4A8 ConvRot decode linear at M = 1, K = 3840, N = 10240,
G = 64, per-group (64) bf16 weight scales, through ck_w4a8_linear -- one
launch in which the activation row is rotated and quantised while the packed
weights stream in.  The metric is packed-weight bandwidth: N * K / 2 bytes per
step over the step time.  Inputs are resident in HBM before timing starts; the
steps cycle through enough weight copies (> 512 MiB) that every step reads its
weights from HBM, not from the 256 MiB Infinity Cache.  The K timed steps are
captured in one HIP graph and replayed between two synchronisations, so the
figure is the GPU's and not the Python launch path's (reported separately as
eager_us_per_step).

After the timed region the other metric figures are measured the same way
(ConvRot linear microseconds and int8 TOPS at M = 8192, the decode GEMV at
M = 4 and 8, M = 32, standalone rotate-quant, the AWQ W4A16 GEMV) and reported
under "also"; the CPU oracle is timed on a bounded sample under "cpu_baseline".

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu-baseline]

HBM traffic of the headline kernel comes from two rocprofv3 counter passes
(FETCH_SIZE, then WRITE_SIZE) over this script, scaled by what the same
counters read for a plain copy of known size (`--calibration-copy`);
`--write-traffic` turns the four counter CSVs into the record that
`roofline.traffic` is read from.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
INT8_PEAK_TOPS = 5000.0          # MI355X dense int8 MFMA, published (5.0 POPS)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w4a8_decode_gemv_m1_k3840_n10240_traffic.txt")
GEMV_SOURCES = ["packed_int4_convrot_amd/csrc/w4_gemv_fused.hip", "packed_int4_convrot_amd/csrc/gemv_reduce.h",
                "packed_int4_convrot_amd/csrc/rotate_rows.h", "packed_int4_convrot_amd/csrc/ck_device.h",
                "packed_int4_convrot_amd/csrc/launch.h"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 2000 headline steps are about 13 ms: long enough that a stall of a few hundred
    # microseconds in one replay (seen once, at 1.3 ms per timed region, while the
    # next 20 replays agreed to 1%) moves the result by a few percent at most.
    ap.add_argument("--steps", type=int, default=2000)
    # 30000 warm-up steps are about 0.2 s of the headline step: the clocks of a chip
    # coming out of idle keep rising for tens of milliseconds under load.
    ap.add_argument("--warmup", type=int, default=30000)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the secondary measurements and the clock readings")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-oracle-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--copies", type=int, default=32, help="weight copies cycled through (cold cache)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="only run a plain elementwise copy of CALIB_BYTES (counter calibration)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="write the traffic record from rocprofv3 counter_collection CSVs and exit")
    ap.add_argument("--profile-workload", choices=sorted(PROFILE_WORKLOADS),
                    help="only run one kernel of the extras a few times (for rocprofv3 counter passes)")
    ap.add_argument("--write-counters", nargs="+", metavar="ARG",
                    help="WORKLOAD CSV...: write profiles/WORKLOAD_counters.txt from the counter passes")
    return ap.parse_args()


def sources_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


CALIB_BYTES = 256 << 20        # bytes read and bytes written by the calibration copy
CALIB_KERNEL = "neg_kernel"    # torch's elementwise negation: one read and one write per element
HEADLINE_KERNEL = "w4_gemv_fused_kernel<1,"


def calibration_copy():
    """A plain elementwise copy of known size (int32 negation, CALIB_BYTES in and out),
    run a few times, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.neg(src, out=dst)
        torch.neg(dst, out=src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes_each_way": CALIB_BYTES, "dispatches": 8}), flush=True)


def _counter_per_dispatch(path, kernel_substring, counter):
    """Mean over dispatches of a kernel of one counter (summed over its instances) in a
    rocprofv3 counter_collection CSV, with the dispatch count."""
    import csv
    per = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if kernel_substring in row["Kernel_Name"] and row["Counter_Name"] == counter:
                per[row["Dispatch_Id"]] = per.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit("no %s dispatches of %r in %s" % (counter, kernel_substring, path))
    return sum(per.values()) / len(per), len(per)


def write_traffic(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, alg_bytes):
    fetch_kib, nf = _counter_per_dispatch(fetch_csv, HEADLINE_KERNEL, "FETCH_SIZE")
    write_kib, nw = _counter_per_dispatch(write_csv, HEADLINE_KERNEL, "WRITE_SIZE")
    cal_fetch_kib, ncf = _counter_per_dispatch(cal_fetch_csv, CALIB_KERNEL, "FETCH_SIZE")
    cal_write_kib, ncw = _counter_per_dispatch(cal_write_csv, CALIB_KERNEL, "WRITE_SIZE")
    f_scale = CALIB_BYTES / (cal_fetch_kib * 1024.0)
    w_scale = CALIB_BYTES / (cal_write_kib * 1024.0)
    hbm = fetch_kib * 1024.0 * f_scale + write_kib * 1024.0 * w_scale
    rec = {"kernel": HEADLINE_KERNEL, "sources_sha": sources_sha(GEMV_SOURCES),
           "fetch_kib_per_dispatch": round(fetch_kib, 1), "write_kib_per_dispatch": round(write_kib, 1),
           "dispatches": [nf, nw], "calibration_fetch_kib": round(cal_fetch_kib, 1),
           "calibration_write_kib": round(cal_write_kib, 1), "calibration_dispatches": [ncf, ncw],
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "hbm_bytes_per_launch": int(round(hbm)), "algorithmic_bytes_per_launch": alg_bytes,
           "traffic_over_algorithmic": round(hbm / alg_bytes, 4)}
    text = ("HBM traffic of the fused W4A8 decode linear kernel (M=1, K=3840, N=10240, G=64, per-group scales)\n"
            "from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by the same counter\n"
            "on a plain copy of %d bytes each way (torch int32 negation).\n\n"
            "Commands (repository root, TMPDIR=/tmp):\n"
            "  rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o run -- python3 bench.py --steps 20 --warmup 2 --no-extras --no-cpu-baseline\n"
            "  rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o run -- python3 bench.py --steps 20 --warmup 2 --no-extras --no-cpu-baseline\n"
            "  rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_cal_fetch -o run -- python3 bench.py --calibration-copy\n"
            "  rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_cal_write -o run -- python3 bench.py --calibration-copy\n"
            "  python3 bench.py --write-traffic <the four run_counter_collection.csv files>\n\n"
            "JSON: %s\n" % (CALIB_BYTES, json.dumps(rec)))
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        f.write(text)
    print(text)


# Kernels of the extras that the counter summaries under profiles/ cover: the
# kernel-name substring, the MFMA op counter, and the algorithmic bytes per launch.
PROFILE_WORKLOADS = {
    "w4a4_gemm_m8192_k3840_n3840": dict(
        kernel="w4_gemm_kernel", M=8192, K=3840, N=3840, mops="SQ_INSTS_VALU_MFMA_MOPS_I8",
        alg_bytes=8192 * 3840 // 2 + 8192 * 4 + 3840 * 3840 // 2 + 3840 * 2 + 8192 * 3840 * 2),
    "w4a4_gemm_m8192_k10240_n3840": dict(
        kernel="w4_gemm_kernel", M=8192, K=10240, N=3840, mops="SQ_INSTS_VALU_MFMA_MOPS_I8",
        alg_bytes=8192 * 10240 // 2 + 8192 * 4 + 3840 * 10240 // 2 + 3840 * 2 + 8192 * 3840 * 2),
    "awq_w4a16_gemm_m4096_k3072_n18432": dict(
        kernel="awq_gemm_kernel", M=4096, K=3072, N=18432, mops="SQ_INSTS_VALU_MFMA_MOPS_BF16",
        alg_bytes=4096 * 3072 * 2 + 18432 * 3072 // 2 + 2 * 2 * 48 * 18432 + 4096 * 18432 * 2),
    "rotate_quant_m8192_k10240_ld10752_g64": dict(
        kernel="rotate_quant_kernel", M=8192, K=10240, N=0, mops=None,
        alg_bytes=8192 * 10240 * 2 + 8192 * 10240 + 8192 * 4),
    "awq_w4a16_gemv_m1_k3072_n18432": dict(
        kernel="w4a16_gemv_kernel", M=1, K=3072, N=18432, mops=None,
        alg_bytes=18432 * 3072 // 2 + 2 * 2 * 48 * 18432 + 3072 * 2 + 18432 * 2),
    # The one-launch decode linear at M = 1 (the headline step), M = 4: packed
    # weights, group scales, bf16 x, bf16 output.
    "w4a8_decode_linear_m1_k3840_n10240_g64": dict(
        kernel="w4_gemv_fused_kernel", M=1, K=3840, N=10240, mops=None,
        alg_bytes=10240 * 3840 // 2 + 60 * 10240 * 2 + 1 * 3840 * 2 + 1 * 10240 * 2),
    "w4a8_decode_linear_m4_k3840_n10240_g64": dict(
        kernel="w4_gemv_fused_kernel", M=4, K=3840, N=10240, mops=None,
        alg_bytes=10240 * 3840 // 2 + 60 * 10240 * 2 + 4 * 3840 * 2 + 4 * 10240 * 2),
    # The one-launch MFMA linear at M = 8 (same bytes as above; its MFMAs cover 16
    # activation rows and 48 weight rows per 40-row workgroup).
    "w4a8_decode_linear_m8_k3840_n10240_g64": dict(
        kernel="w4_skinny_fused_kernel", M=8, K=3840, N=10240, mops="SQ_INSTS_VALU_MFMA_MOPS_I8",
        alg_bytes=10240 * 3840 // 2 + 60 * 10240 * 2 + 8 * 3840 * 2 + 8 * 10240 * 2),
    # The matmul half of the M = 32 W4A8 linear: packed weights, group scales, the
    # tiled codes and row scales, the bf16 output.
    "w4a8_skinny_m32_k3840_n3840_g64": dict(
        kernel="w4_skinny_kernel", M=32, K=3840, N=3840, mops=None,
        alg_bytes=3840 * 3840 // 2 + 60 * 3840 * 2 + 32 * 3840 + 32 * 4 + 32 * 3840 * 2),
}
_COMMON = ["packed_int4_convrot_amd/csrc/ck_device.h", "packed_int4_convrot_amd/csrc/launch.h"]
KERNEL_SOURCES = {
    "w4_gemm_kernel": ["packed_int4_convrot_amd/csrc/w4_gemm.hip"] + _COMMON,
    "awq_gemm_kernel": ["packed_int4_convrot_amd/csrc/awq_gemm.hip"] + _COMMON,
    "rotate_quant_kernel": ["packed_int4_convrot_amd/csrc/rotate_quant.hip"] + _COMMON,
    "w4a16_gemv_kernel": ["packed_int4_convrot_amd/csrc/w4a16_gemv.hip",
                          "packed_int4_convrot_amd/csrc/gemv_reduce.h"] + _COMMON,
    "w4_skinny_kernel": ["packed_int4_convrot_amd/csrc/w4_skinny.hip"] + _COMMON,
    "w4_gemv_fused_kernel": ["packed_int4_convrot_amd/csrc/w4_gemv_fused.hip",
                             "packed_int4_convrot_amd/csrc/gemv_reduce.h",
                             "packed_int4_convrot_amd/csrc/rotate_rows.h"] + _COMMON,
    "w4_skinny_fused_kernel": ["packed_int4_convrot_amd/csrc/w4_skinny_fused.hip",
                               "packed_int4_convrot_amd/csrc/gemv_reduce.h",
                               "packed_int4_convrot_amd/csrc/rotate_rows.h"] + _COMMON,
}


def counter_passes(name):
    """The --pmc argument of each counter pass (within one pass's hardware limits)."""
    w = PROFILE_WORKLOADS[name]
    if w["mops"] is None:
        return ["FETCH_SIZE", "WRITE_SIZE", "SQ_INSTS_VALU SQ_INSTS_LDS SQ_WAVES"]
    return [w["mops"] + " SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAVES",
            "FETCH_SIZE", "WRITE_SIZE"]


def profile_workload(name, reps=5):
    """Run one kernel of the extras reps + 1 times, synchronising after each call, so that
    counter passes see whole dispatches of it alone."""
    import torch
    import packed_int4_convrot_amd as ck
    import workloads
    dev = torch.device("cuda:0")

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    if name.startswith("w4a4_gemm"):
        wl = "w4a4_linear_m8192_k3840_n3840_g64" if "k3840" in name else "w4a4_linear_m8192_k10240_n3840_g256"
        inp = workloads.workload_inputs(wl)
        x = bf16(inp["x"])
        packed = torch.from_numpy(inp["packed"]).to(dev)
        scl = bf16(inp["w_scales"])
        codes4, rs = ck.rotate_quant_packed4(x, workloads.WORKLOADS[wl]["G"])
        out = torch.empty((x.shape[0], packed.shape[0]), dtype=torch.bfloat16, device=dev)

        def fn():
            ck.gemm_packed4(codes4, rs, packed, scl, False, out=out)
    elif name.startswith("w4a8_skinny"):
        wl = "w4a8_linear_m32_k3840_n3840_g64"
        w = workloads.WORKLOADS[wl]
        inp = workloads.workload_inputs(wl)
        x = bf16(inp["x"])
        packed = torch.from_numpy(inp["packed"]).to(dev)
        scl = bf16(inp["w_scales"])
        out = torch.empty((w["M"], w["N"]), dtype=torch.bfloat16, device=dev)
        work = torch.empty((ck.workspace_bytes(w["M"], w["K"], w["N"]),), dtype=torch.uint8, device=dev)

        def fn():
            ck.linear(x, w["G"], 8, packed, scl, True, out=out, workspace=work)
    elif name.startswith("w4a8_decode_linear"):
        wl = "w4a8_decode_gemv_k3840_n10240_g64"
        w = workloads.WORKLOADS[wl]
        M = PROFILE_WORKLOADS[name]["M"]
        inp = workloads.workload_inputs(wl, M=M)
        x = bf16(inp["x"])
        packed = torch.from_numpy(inp["packed"]).to(dev)
        scl = bf16(inp["w_scales"])
        out = torch.empty((M, w["N"]), dtype=torch.bfloat16, device=dev)
        work = torch.empty((ck.workspace_bytes(M, w["K"], w["N"]),), dtype=torch.uint8, device=dev)

        def fn():
            ck.linear(x, w["G"], 8, packed, scl, True, out=out, workspace=work)
    elif name.startswith("awq_w4a16_gemv"):
        d = workloads.workload_inputs("awq_w4a16_gemv_m1_k3072_n18432")
        xv = bf16(d["x"])
        pk = torch.from_numpy(d["packed"]).to(dev)
        s, z = bf16(d["scales"]), bf16(d["zeros"])
        out = torch.empty((xv.shape[0], pk.shape[0]), dtype=torch.bfloat16, device=dev)

        def fn():
            ck.w4a16_gemv(xv, pk, s, z, out=out)
    elif name.startswith("awq"):
        d = workloads.workload_inputs("awq_w4a16_gemv_m1_k3072_n18432")
        rng = torch.Generator(device=dev).manual_seed(1)
        xs = torch.randn((4096, 3072), generator=rng, device=dev).to(torch.bfloat16)
        pk = torch.from_numpy(d["packed"]).to(dev)
        s, z = bf16(d["scales"]), bf16(d["zeros"])
        out = torch.empty((4096, 18432), dtype=torch.bfloat16, device=dev)

        def fn():
            ck.w4a16_gemm(xs, pk, s, z, out=out)
    else:
        wl = "rotate_quant_m8192_k10240_ld10752"
        x = bf16(workloads.workload_inputs(wl)["x"])
        K = workloads.WORKLOADS[wl]["K"]
        codes = torch.empty((x.shape[0], K), dtype=torch.int8, device=dev)
        rs = torch.empty((x.shape[0],), dtype=torch.float32, device=dev)

        def fn():
            ck.rotate_quant(x[:, :K], 64, 8, codes, rs)
    for _ in range(reps + 1):
        fn()
        torch.cuda.synchronize()
    print(json.dumps({"profile_workload": name, "dispatches": reps + 1}), flush=True)


def write_counters(name, csvs, out_dir=None):
    """Summarise the counter passes of one profile workload: each counter's mean per
    dispatch of the workload's kernel, and what follows from them."""
    import csv
    w = PROFILE_WORKLOADS[name]
    per = {}        # counter -> {(file, dispatch): value}
    for path in csvs:
        with open(path) as f:
            for row in csv.DictReader(f):
                if w["kernel"] in row["Kernel_Name"]:
                    key = (path, row["Dispatch_Id"])
                    per.setdefault(row["Counter_Name"], {})[key] = float(row["Counter_Value"])
    if not per:
        raise SystemExit("no dispatches of %r in the given files" % w["kernel"])
    mean = {c: sum(v.values()) / len(v) for c, v in per.items()}
    rec = {"workload": name, "kernel": w["kernel"], "sources_sha": sources_sha(KERNEL_SOURCES[w["kernel"]]),
           "dispatches_per_pass": min(len(v) for v in per.values()),
           "counters_mean_per_dispatch": {c: round(v, 1) for c, v in sorted(mean.items())},
           "algorithmic_bytes_per_launch": w["alg_bytes"]}
    lines = []
    try:
        with open(TRAFFIC_FILE) as f:
            cal = json.loads(f.read().split("JSON:", 1)[1])
        fs, ws = cal["fetch_scale"], cal["write_scale"]
    except (OSError, IndexError, ValueError, KeyError):
        fs = ws = None
    if fs is not None and "FETCH_SIZE" in mean and "WRITE_SIZE" in mean:
        hbm = mean["FETCH_SIZE"] * 1024.0 * fs + mean["WRITE_SIZE"] * 1024.0 * ws
        rec["fabric_bytes_per_launch"] = int(round(hbm))
        rec["fabric_over_algorithmic"] = round(hbm / w["alg_bytes"], 4)
        lines.append("Bytes between the L2s and the fabric per launch: FETCH_SIZE x %.4f + WRITE_SIZE x %.4f "
                     "(the calibration factors of the headline traffic record) = %.1f MB, %.3f x the algorithmic "
                     "%.1f MB.  FETCH_SIZE counts L2 misses, which the Infinity Cache serves in part: operands "
                     "that several XCDs read each come from there, not from HBM, once per XCD."
                     % (fs, ws, hbm / 1e6, hbm / w["alg_bytes"], w["alg_bytes"] / 1e6))
    if w["mops"] and w["mops"] in mean:
        ops = mean[w["mops"]] * 512.0
        alg_ops = 2.0 * w["M"] * w["N"] * w["K"]
        rec["mfma_ops_per_launch"] = ops
        rec["mfma_ops_over_2MNK"] = round(ops / alg_ops, 4)
        lines.append("MFMA ops per launch: %s x 512 = %.4g, %.4f x 2*M*N*K" % (w["mops"], ops, ops / alg_ops))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            per_simd = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024.0
            rec["mfma_busy_cycles_per_simd"] = round(per_simd, 1)
            lines.append("MFMA busy cycles per SIMD (1024 SIMDs): %.0f" % per_simd)
    text = ("rocprofv3 counters of %s (kernel %s), mean per dispatch over the counter passes.\n\n"
            "Commands (repository root, TMPDIR=/tmp; one pass per line):\n" % (name, w["kernel"]))
    for i, pmc in enumerate(counter_passes(name)):
        text += ("  rocprofv3 --pmc %s --output-format csv -d gpurun_out/pmc_%s_%d -o run -- "
                 "python3 bench.py --profile-workload %s\n" % (pmc, name, i, name))
    text += "  python3 bench.py --write-counters %s <the run_counter_collection.csv files>\n\n" % name
    text += "".join("%s\n" % line for line in lines)
    text += "\nJSON: %s\n" % json.dumps(rec)
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), "%s_counters.txt" % name)
    with open(path, "w") as f:
        f.write(text)
    print(text)


def headline_alg_bytes(M, K, N):
    """Bytes the fused M = 1 step must move: packed weights, group scales, the bf16
    activation row and the bf16 output row."""
    return N * K // 2 + (K // 64) * N * 2 + M * K * 2 + M * N * 2


def measured_traffic(bytes_per_launch_alg):
    """HBM bytes per GEMV launch from the committed rocprofv3 counter summary, or None
    when the kernel sources changed after the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.loads(f.read().split("JSON:", 1)[1])
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("sources_sha") != sources_sha(GEMV_SOURCES):
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.cpu_oracle_child:
        oracle_child()
        return
    if args.write_traffic:
        write_traffic(*args.write_traffic, alg_bytes=headline_alg_bytes(1, 3840, 10240))
        return
    if args.write_counters:
        if len(args.write_counters) < 2 or args.write_counters[0] not in PROFILE_WORKLOADS:
            raise SystemExit("--write-counters WORKLOAD CSV...; workloads: %s" % ", ".join(sorted(PROFILE_WORKLOADS)))
        write_counters(args.write_counters[0], args.write_counters[1:])
        return
    if args.steps < 1 or args.warmup < 0:
        raise SystemExit("--steps must be >= 1 and --warmup >= 0")
    if args.gpus != 1:
        print("bench.py measures one MI355X: this build has no multi-GPU path, run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibration_copy:
        calibration_copy()
        return
    if args.profile_workload:
        profile_workload(args.profile_workload)
        return

    import packed_int4_convrot_amd as ck
    import workloads
    sys.path.insert(0, os.path.join(ROOT, "tests"))

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ------------------------------------------------------------ headline
    name = "w4a8_decode_gemv_k3840_n10240_g64"
    w = workloads.WORKLOADS[name]
    M, K, N, G = 1, w["K"], w["N"], w["G"]
    inp = workloads.workload_inputs(name, M=M)
    log("bench: generating %d weight copies of %.1f MB" % (args.copies, N * K / 2 / 1e6))
    x = bf16(inp["x"])
    packed0 = u8(inp["packed"])
    scales0 = bf16(inp["w_scales"])
    packs = [packed0] + [packed0.clone() for _ in range(args.copies - 1)]
    scls = [scales0] + [scales0.clone() for _ in range(args.copies - 1)]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((ck.workspace_bytes(M, K, N),), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        ck.linear(x, G, 8, packs[i % args.copies], scls[i % args.copies], True, out=out, workspace=ws)

    # Warm-up: at least W steps, as whole replays of the timed graph itself (at least
    # one), so that the timed replay is never that graph's first: a graph's first
    # replay measured 3-5% slower than the next ones (with --steps 20, about 0.4 us
    # per step).  warmup_steps_run in the result is the number of steps this ran.
    g_steps = capture(torch, step, args.steps)
    warm_replays = max(1, -(-args.warmup // args.steps))
    for _ in range(warm_replays):
        g_steps.replay()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t_start.record(stream)
    g_steps.replay()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    packed_bytes = N * K // 2
    value = packed_bytes / (ms_step * 1e-3) / 1e9
    # The step is one launch (rotate-quant fused into the GEMV), so the
    # average launch duration is the timed region over the steps.
    alg_bytes = headline_alg_bytes(M, K, N)
    achieved = alg_bytes / (ms_step * 1e-3) / 1e9
    traffic = measured_traffic(alg_bytes)
    # Spread: the same graph replayed again, each replay's mean step time.
    reps = []
    for _ in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g_steps.replay()
        b.record(stream)
        torch.cuda.synchronize()
        reps.append(a.elapsed_time(b) / args.steps * 1e3)
    reps.sort()
    spread = {"replays": len(reps), "steps_each": args.steps, "p10_us": round(reps[1], 3),
              "median_us": round((reps[9] + reps[10]) / 2, 3), "p90_us": round(reps[17], 3)}
    eager_us = _time_eager(torch, step, stream, min(args.steps, 100)) * 1.0
    log("bench: step %.3f us (wall %.2f us), %.0f GB/s packed, eager %.2f us/step" %
        (ms_step * 1e3, wall / args.steps * 1e6, value, eager_us))

    result = {
        "metric": "ConvRot linear us + int8 TOPS (M=8192) and packed-weight GB/s (M=1 GEMV)",
        "value": round(value, 1),
        "unit": "GB/s (packed weight, M=1 W4A8 ConvRot decode linear)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_replays * args.steps,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded N(0,1) activations with x20 outlier columns, uniform uint4 codes, "
                "uniform [0.002,0.02] bf16 group scales)",
        "config": {"workload": "w4a8_convrot_decode_linear", "M": M, "K": K, "N": N, "G": G,
                   "weight_scales": "per-group (64), bf16", "weight_copies_cycled": args.copies,
                   "step": "ck_w4a8_linear (rotate-quant fused into the decode GEMV, one launch)",
                   "timing": "K steps captured in one HIP graph, replayed between synchronisations"},
        "roofline": {"bound": "hbm", "kernel": "w4_gemv_fused_kernel (rotate-quant + decode GEMV, one workgroup per CU)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg_bytes, "avg_launch_us": round(ms_step * 1e3, 3)},
        "eager_us_per_step": round(eager_us, 3),
        "us_per_step_over_replays": spread,
        "gfx_clock_mhz": None if args.no_extras else gfx_clock_mhz(torch, capture(torch, step, 2000)),
    }

    # ------------------------------------------------------------ extras
    if not args.no_extras:
        result["also"] = extras(ck, workloads, torch, dev, bf16, u8, stream)
        result["also"]["same_bytes_plain_copy"] = same_bytes_copy(torch, dev, stream, alg_bytes, args.copies)
        result["also"]["launch_floor"] = launch_floor(torch, dev, stream)

    # ------------------------------------------------------------ CPU oracle
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(packed_bytes, result.get("also"), ms_step * 1e3)

    print(json.dumps(result), flush=True)


def gfx_clock_mhz(torch, graph, seconds=1.5):
    """GFX clock (MHz, mean over the XCDs) read with amd-smi while `graph` is replayed
    back to back for about `seconds`; the median of the readings, or None where amd-smi
    is missing or prints something else."""
    import subprocess
    import threading
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True,
                                   text=True, timeout=10)
                d = json.loads(r.stdout)
                d = d["gpu_data"][0] if isinstance(d, dict) else d[0]
                vals = [v["clk"]["value"] for k, v in d["clock"].items() if k.startswith("gfx")]
                if vals:
                    samples.append(sum(vals) / len(vals))
            except Exception:
                return

    t = threading.Thread(target=poll, daemon=True)
    t0 = time.time()
    graph.replay()
    t.start()
    while time.time() - t0 < seconds:
        graph.replay()
        torch.cuda.synchronize()
    stop.set()
    t.join(timeout=15)
    if not samples:
        return None
    samples.sort()
    return round(samples[len(samples) // 2], 1)


def capture(torch, fn, n):
    """A HIP graph holding n calls fn(0..n-1) (the library allocates and syncs nothing)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    _upload(torch, g)
    return g


def _upload(torch, g):
    """Upload the instantiated graph to the device (hipGraphUpload) before its first
    replay.  Otherwise the first replay, which is the timed one, also carries that
    one-time setup: measured 0.03-0.18 us per headline step.  Skipped where the
    runtime or torch does not offer it."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        rc = hip.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    except (OSError, AttributeError, RuntimeError, TypeError):
        return False
    torch.cuda.synchronize()
    return rc == 0


def _time_eager(torch, fn, stream, iters, warmup=3):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(iters):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters * 1e3  # us


WARM_S = 0.2   # seconds of the same work before each secondary measurement


def _time(fn, stream, iters, warmup=3, warm_s=None, reps=5):
    """Microseconds per call: the median over `reps` timed replays of a HIP graph of
    `iters` calls, after a graph of `warmup` calls has been replayed for at least
    `warm_s` seconds (WARM_S by default).  Under sustained load the chip's clocks keep
    rising for tens of milliseconds: the M = 8192 GEMM at K = 3840 times 116 us per
    call after 3 warm-up calls, 107 us after 100 and 97 us from 300 on, so each
    measurement first runs long enough to reach that steady state; the median keeps
    one replay caught in a transient clock drop from setting the figure."""
    import torch
    g_w = capture(torch, fn, warmup)
    g = capture(torch, fn, iters)
    t0 = time.perf_counter()
    while True:
        g_w.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= (WARM_S if warm_s is None else warm_s):
            break
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per_call = []
    for _ in range(reps):
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        per_call.append(a.elapsed_time(b) / iters * 1e3)
    return sorted(per_call)[len(per_call) // 2]


def same_bytes_copy(torch, dev, stream, nbytes, copies):
    """A plain elementwise copy (torch int32 negation: one read and one write per
    element) moving the same HBM bytes as one headline step, from cold sources,
    timed like the headline: what one launch of this size can reach."""
    n = nbytes // 8
    srcs = [torch.ones(n, dtype=torch.int32, device=dev) for _ in range(copies)]
    dst = torch.empty(n, dtype=torch.int32, device=dev)
    us = _time(lambda i: torch.neg(srcs[i % copies], out=dst), stream, 100)
    return {"bytes": n * 8, "us": round(us, 3), "GBps": round(n * 8 / us / 1e3, 1),
            "frac_hbm": round(n * 8 / us / 1e3 / HBM_PEAK_GBS, 4)}


def launch_floor(torch, dev, stream):
    """Per-launch cost of a trivial kernel (256 elements), timed like the headline:
    the floor under every small-M figure."""
    a = torch.ones(256, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    return {"us": round(_time(lambda i: torch.neg(a, out=b), stream, 100), 3),
            "kernel": "torch elementwise negation of 256 int32"}


def extras(ck, workloads, torch, dev, bf16, u8, stream):
    res = {}
    # decode GEMV at M = 4, 5, 6, 8 (cold weights)
    name = "w4a8_decode_gemv_k3840_n10240_g64"
    w = workloads.WORKLOADS[name]
    K, N = w["K"], w["N"]
    base = workloads.workload_inputs(name, M=8)
    packs = [u8(base["packed"]) for _ in range(32)]
    scl = bf16(base["w_scales"])
    for M in (4, 5, 6, 8):
        x = bf16(base["x"][:M])
        codes, rs = ck.rotate_quant(x, 64, 8)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        us = _time(lambda i: ck.gemv(codes, rs, packs[i % 32], scl, True, out=out), stream, 100)
        ws = torch.empty((ck.workspace_bytes(M, K, N),), dtype=torch.uint8, device=dev)
        lin = _time(lambda i: ck.linear(x, 64, 8, packs[i % 32], scl, True, out=out, workspace=ws), stream, 100)
        # algorithmic bytes: packed weights, group scales, the activations (codes for the
        # GEMV, bf16 x for the whole linear) and the bf16 output
        wb = N * K // 2 + (K // 64) * N * 2 + 2 * M * N
        gemv_bytes, lin_bytes = wb + M * K + 4 * M, wb + 2 * M * K
        res["w4a8_decode_gemv_m%d" % M] = {
            "gemv_us": round(us, 3), "linear_us": round(lin, 3), "packed_GBps": round(N * K / 2 / us / 1e3, 1),
            "gemv_algorithmic_bytes": gemv_bytes, "gemv_frac_hbm": round(gemv_bytes / us / 1e3 / HBM_PEAK_GBS, 4),
            "linear_algorithmic_bytes": lin_bytes,
            "linear_frac_hbm": round(lin_bytes / lin / 1e3 / HBM_PEAK_GBS, 4)}
    del packs
    log("bench: decode extras done")

    # M = 32 W4A8 linear (per-group scales)
    name = "w4a8_linear_m32_k3840_n3840_g64"
    w = workloads.WORKLOADS[name]
    inp = workloads.workload_inputs(name)
    x = bf16(inp["x"])
    packs = [u8(inp["packed"]) for _ in range(64)]
    scl = bf16(inp["w_scales"])
    out = torch.empty((32, w["N"]), dtype=torch.bfloat16, device=dev)
    work = torch.empty((ck.workspace_bytes(32, w["K"], w["N"]),), dtype=torch.uint8, device=dev)
    us = _time(lambda i: ck.linear(x, 64, 8, packs[i % 64], scl, True, out=out, workspace=work), stream, 100)
    # x, codes written and read, row scales, packed weights, group scales, output
    alg = 368768 + 8202368
    res["w4a8_linear_m32_k3840_n3840_g64"] = {"linear_us": round(us, 3), "algorithmic_bytes": alg,
                                              "GBps": round(alg / us / 1e3, 1),
                                              "frac_hbm": round(alg / us / 1e3 / HBM_PEAK_GBS, 4)}
    del packs
    log("bench: M=32 done")

    # M = 8192 W4A4 linears (per-channel scales): rotate-quant + GEMM
    for name in ("w4a4_linear_m8192_k3840_n3840_g64", "w4a4_linear_m8192_k10240_n3840_g256"):
        w = workloads.WORKLOADS[name]
        inp = workloads.workload_inputs(name)
        M, K, N, G = w["M"], w["K"], w["N"], w["G"]
        x = bf16(inp["x"])
        # enough copies of x that the activations come from HBM (> 512 MB together,
        # twice the 256 MB Infinity Cache): the rotate-quant and whole-linear figures
        # below are cold; the GEMM's operands (packed codes and weights, 23-62 MB) stay
        # cache-resident, which an MFMA-bound kernel does not notice
        nx = max(2, -(-512 * 2 ** 20 // (M * K * 2)))
        xs = [x] + [x.clone() for _ in range(nx - 1)]
        packed = u8(inp["packed"])
        scl = bf16(inp["w_scales"])
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        work = torch.empty((ck.workspace_bytes(M, K, N),), dtype=torch.uint8, device=dev)  # held by the caller
        # the linear's own two launches: packed rotate-quant, then the GEMM on packed codes
        codes4, rs = ck.rotate_quant_packed4(x, G)
        lin = _time(lambda i: ck.linear(xs[i % nx], G, 4, packed, scl, False, out=out, workspace=work), stream, 20)
        rq = _time(lambda i: ck.rotate_quant_packed4(xs[i % nx], G, codes4, rs), stream, 20)
        rq_warm = _time(lambda i: ck.rotate_quant_packed4(x, G, codes4, rs), stream, 20)
        gm = _time(lambda i: ck.gemm_packed4(codes4, rs, packed, scl, False, out=out), stream, 20)
        # codes one per byte (ck_rotate_quant + ck_w4_gemm_q), for comparison
        codes, rs8 = ck.rotate_quant(x, G, 4)
        gm8 = _time(lambda i: ck.gemm_q(codes, rs8, packed, scl, False, out=out), stream, 20)
        ops = 2.0 * M * N * K
        rq_bytes = M * K * 2 + M * K // 2 + M * 4
        clk = gfx_clock_mhz(torch, capture(torch, lambda i: ck.gemm_packed4(codes4, rs, packed, scl, False, out=out), 40))
        res[name] = {"x_copies_cycled": nx, "linear_us": round(lin, 2), "rotate_quant_us": round(rq, 2),
                     "rotate_quant_warm_us": round(rq_warm, 2), "gemm_us": round(gm, 2),
                     "timing": "linear_us and rotate_quant_us cycle x_copies_cycled copies of x (cold); "
                               "rotate_quant_warm_us re-reads one x; gemm_us re-reads cache-resident operands",
                     "gemm_gfx_clock_mhz": clk,
                     "gemm_int8_TOPS": round(ops / gm / 1e6, 1),
                     "gemm_frac_int8_peak": round(ops / gm / 1e6 / INT8_PEAK_TOPS, 4),
                     "linear_int8_TOPS": round(ops / lin / 1e6, 1),
                     "rotate_quant_GBps": round(rq_bytes / rq / 1e3, 1),
                     "rotate_quant_frac_hbm": round(rq_bytes / rq / 1e3 / HBM_PEAK_GBS, 4),
                     "byte_codes_gemm_us": round(gm8, 2)}
        del x, xs, packed, out, codes, codes4, work
        log("bench: %s done" % name)

    # standalone rotate-quant, strided [8192, 10240] in [8192, 10752]
    name = "rotate_quant_m8192_k10240_ld10752"
    w = workloads.WORKLOADS[name]
    M, K = w["M"], w["K"]
    xs = [bf16(workloads.workload_inputs(name)["x"])]
    xs.append(xs[0].clone())  # two copies: 2 x 176 MB > the 256 MB Infinity Cache
    codes = torch.empty((M, K), dtype=torch.int8, device=dev)
    rs = torch.empty((M,), dtype=torch.float32, device=dev)
    rq_bytes = M * K * 2 + M * K + M * 4
    for G in w["Gs"]:
        us = _time(lambda i: ck.rotate_quant(xs[i % 2][:, :K], G, 8, codes, rs), stream, 20)
        clk = gfx_clock_mhz(torch, capture(torch, lambda i: ck.rotate_quant(xs[i % 2][:, :K], G, 8, codes, rs), 40),
                            seconds=1.0)
        res["rotate_quant_m8192_k10240_ld10752_g%d" % G] = {
            "us": round(us, 2), "GBps": round(rq_bytes / us / 1e3, 1),
            "frac_hbm": round(rq_bytes / us / 1e3 / HBM_PEAK_GBS, 4), "gfx_clock_mhz": clk}
    del xs
    log("bench: rotate-quant done")

    # offline weight producer: rotate + quantise + pack a bf16 [N, K] weight
    N, K = 10240, 3840
    rng = torch.Generator(device=dev).manual_seed(0)
    wsrc = [(torch.randn((N, K), generator=rng, device=dev) * 0.02).to(torch.bfloat16) for _ in range(4)]  # 315 MB > the 256 MB Infinity Cache
    pk = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    for pg in (False, True):
        sc = torch.empty((K // 64, N) if pg else (N,), dtype=torch.bfloat16, device=dev)
        us = _time(lambda i: ck.quantize_weights(wsrc[i % 4], 64, pg, pk, sc), stream, 20)
        nbytes = N * K * 2 + N * K // 2 + sc.numel() * 2
        res["quantize_weights_n%d_k%d_g64_%s" % (N, K, "per_group" if pg else "per_channel")] = {
            "us": round(us, 2), "GBps": round(nbytes / us / 1e3, 1),
            "frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
    del wsrc, pk
    log("bench: weight producer done")

    # AWQ W4A16 GEMV
    name = "awq_w4a16_gemv_m1_k3072_n18432"
    w = workloads.WORKLOADS[name]
    d = workloads.workload_inputs(name)
    x = bf16(d["x"])
    packs = [u8(d["packed"]) for _ in range(24)]
    s, z = bf16(d["scales"]), bf16(d["zeros"])
    out = torch.empty((1, w["N"]), dtype=torch.bfloat16, device=dev)
    us = _time(lambda i: ck.w4a16_gemv(x, packs[i % 24], s, z, out=out), stream, 100)
    pb = w["N"] * w["K"] // 2
    total = pb + 2 * 2 * (w["K"] // 64) * w["N"] + w["K"] * 2 + w["N"] * 2
    res[name] = {"us": round(us, 3), "packed_GBps": round(pb / us / 1e3, 1),
                 "total_GBps": round(total / us / 1e3, 1), "frac_hbm": round(total / us / 1e3 / HBM_PEAK_GBS, 4)}
    del packs
    log("bench: awq done")

    # AWQ prefill GEMM on the same layer at 4096 rows (bf16 MFMA, weights rebuilt in registers)
    M, K, N = 4096, w["K"], w["N"]
    rng = torch.Generator(device=dev).manual_seed(1)
    xs = (torch.randn((M, K), generator=rng, device=dev)).to(torch.bfloat16)
    pk = u8(d["packed"])
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    us = _time(lambda i: ck.w4a16_gemm(xs, pk, s, z, out=out), stream, 20)
    fl = 2.0 * M * N * K
    res["awq_w4a16_gemm_m%d_k%d_n%d" % (M, K, N)] = {
        "us": round(us, 1), "bf16_TFLOPS": round(fl / us / 1e6, 1),
        "frac_bf16_peak": round(fl / us / 1e6 / BF16_PEAK_TFLOPS, 4)}
    del xs, pk, out
    log("bench: awq prefill done")
    return res


def _host_cpu():
    """CPU model name and core counts of the host the oracle runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


# Rows of the M = 8192 workloads and of rotate-quant on which the oracle is timed
# (the same kind of sample the parity tests check); the oracle's work is linear in
# the rows, so its time for the whole workload is this time x M / rows.
ORACLE_SAMPLE_ROWS = {"w4a4_linear_m8192_k3840_n3840_g64": 8, "w4a4_linear_m8192_k10240_n3840_g256": 4,
                      "rotate_quant_m8192_k10240_ld10752": 16}


def oracle_child():
    """Time the oracle (single-threaded C) on every workload, pinned to one core.  Runs
    in its own process (bench.py --cpu-oracle-child) so that the pinning does not touch
    the GPU process; prints one JSON line."""
    cpu = min(os.sched_getaffinity(0))
    os.sched_setaffinity(0, {cpu})
    import oracle
    import workloads
    oracle.build()

    def stages(x, G, bits, packed, w_scales, per_group, K=None):
        t = {}
        t0 = time.perf_counter()
        xr = oracle.rotate(x, G, K)
        t["rotate"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        codes, sx = oracle.quantize(xr, bits)
        t["quantize"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        w = oracle.unpack(packed, codes.shape[1])
        t["unpack"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        acc = oracle.int_gemm(codes, w, 64 if per_group else None)
        t["int_gemm"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.epilogue(acc, sx, w_scales, per_group)
        t["epilogue"] = time.perf_counter() - t0
        return t

    res = {}
    name = "w4a8_decode_gemv_k3840_n10240_g64"
    w = workloads.WORKLOADS[name]
    for M in w["Ms"]:
        inp = workloads.workload_inputs(name, M=M)
        reps = 10 if M == 1 else 3
        tot = {}
        for _ in range(reps):
            for k, v in stages(inp["x"], w["G"], w["bits"], inp["packed"], inp["w_scales"], True).items():
                tot[k] = tot.get(k, 0.0) + v / reps
        res["%s_m%d" % (name, M)] = {"rows_timed": M, "rows": M, "stages_us": {k: round(v * 1e6, 1) for k, v in tot.items()},
                                     "us": round(sum(tot.values()) * 1e6, 1), "repeats": reps}
    for name in ("w4a8_linear_m32_k3840_n3840_g64", "w4a4_linear_m8192_k3840_n3840_g64",
                 "w4a4_linear_m8192_k10240_n3840_g256"):
        w = workloads.WORKLOADS[name]
        inp = workloads.workload_inputs(name)
        rows = ORACLE_SAMPLE_ROWS.get(name, w["M"])
        t = stages(inp["x"][:rows], w["G"], w["bits"], inp["packed"], inp["w_scales"], w["scale"] == "group")
        # every stage but the weight unpack is per row
        per_row = sum(v for k, v in t.items() if k != "unpack")
        res[name] = {"rows_timed": rows, "rows": w["M"], "stages_us": {k: round(v * 1e6, 1) for k, v in t.items()},
                     "us": round((per_row * w["M"] / rows + t["unpack"]) * 1e6, 1)}
    name = "rotate_quant_m8192_k10240_ld10752"
    w = workloads.WORKLOADS[name]
    x = workloads.workload_inputs(name)["x"]
    rows = ORACLE_SAMPLE_ROWS[name]
    for G in w["Gs"]:
        t0 = time.perf_counter()
        xr = oracle.rotate(x[:rows], G, w["K"])
        t1 = time.perf_counter()
        oracle.quantize(xr, w["bits"])
        t2 = time.perf_counter()
        res["%s_g%d" % (name, G)] = {"rows_timed": rows, "rows": w["M"],
                                     "stages_us": {"rotate": round((t1 - t0) * 1e6, 1), "quantize": round((t2 - t1) * 1e6, 1)},
                                     "us": round((t2 - t0) * w["M"] / rows * 1e6, 1)}
    name = "awq_w4a16_gemv_m1_k3072_n18432"
    d = workloads.workload_inputs(name)
    t0 = time.perf_counter()
    oracle.awq_gemv(d["x"], d["packed"], d["scales"], d["zeros"])
    res[name] = {"rows_timed": 1, "rows": 1, "us": round((time.perf_counter() - t0) * 1e6, 1)}
    print(json.dumps({"cpu": cpu, "host": _host_cpu(), "workloads": res}), flush=True)


# The GPU figure (microseconds of the whole step) that each oracle entry is set beside.
def _gpu_us(also, headline_us, key):
    if key == "w4a8_decode_gemv_k3840_n10240_g64_m1":
        return headline_us
    if key.startswith("w4a8_decode_gemv_k3840_n10240_g64_m"):
        return also.get("w4a8_decode_gemv_m%s" % key.rsplit("_m", 1)[1], {}).get("linear_us")
    if key.startswith("rotate_quant") or key.startswith("awq"):
        return also.get(key, {}).get("us")
    return also.get(key, {}).get("linear_us")


def cpu_baseline(packed_bytes, also, headline_us):
    """The oracle on every workload, single-threaded and pinned to one core, in a child
    process; the headline value is the packed-weight rate of the M = 1 decode step."""
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-oracle-child"], capture_output=True,
                       text=True, timeout=600)
    if r.returncode != 0:
        return {"error": r.stderr[-500:]}
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    per = {}
    for key, v in rec["workloads"].items():
        g = _gpu_us(also or {}, headline_us, key)
        per[key] = dict(v, gpu_us=g, speedup=round(v["us"] / g, 1) if g else None)
    head = per["w4a8_decode_gemv_k3840_n10240_g64_m1"]
    return {"value": round(packed_bytes / (head["us"] * 1e-6) / 1e9, 4), "unit": "GB/s (packed weight, M=1 step)",
            "cores": 1, "kind": "oracle", "host": rec["host"], "pinned_cpu": rec["cpu"],
            "sample": "each workload's oracle steps (rotation by explicit H_G product, quantisation, unpack, exact "
                      "integer sums, fp64 epilogue; AWQ: fp64 dequantised product) in one process pinned to one "
                      "core; decode M = 1 / 4 / 8, the M = 32 linear and AWQ whole, the M = 8192 linears and "
                      "rotate-quant on the first rows_timed rows, scaled by rows / rows_timed",
            "per_workload": per}


if __name__ == "__main__":
    main()
