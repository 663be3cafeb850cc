"""Host-side logic of bench.py: the one-GPU guard and the rocprofv3 counter summaries
(no GPU, no compute)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

# Hardware limits of one rocprofv3 counter pass on gfx950 (counters per block).
PASS_LIMITS = {"SQ_": 8, "TCC_": 4, "TCP_": 4, "TA_": 2, "TD_": 2, "GRBM_": 2}
# Derived counters in terms of the TCC counters they use.
DERIVED_TCC = {"FETCH_SIZE": 3, "WRITE_SIZE": 2}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one MI355X" in r.stderr


@pytest.mark.parametrize("name", sorted(bench.PROFILE_WORKLOADS))
def test_counter_passes_fit_one_pass(name):
    for pmc in bench.counter_passes(name):
        used = {}
        for c in pmc.split():
            if c in DERIVED_TCC:
                used["TCC_"] = used.get("TCC_", 0) + DERIVED_TCC[c]
                continue
            block = next(b for b in PASS_LIMITS if c.startswith(b))
            used[block] = used.get(block, 0) + 1
        for block, n in used.items():
            assert n <= PASS_LIMITS[block], (pmc, block, n)


def _csv(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_write_counters_means_and_derived_figures(tmp_path):
    name = "w4a4_gemm_m8192_k3840_n3840"
    M, K, N = 8192, 3840, 3840
    mfma_instr = 2 * M * N * K // (32 * 32 * 32 * 2)          # one v_mfma_i32_32x32x32_i8 = 65536 ops
    kern = "void ck::(anonymous namespace)::w4_gemm_kernel<2, 4, 4, 2, 4, false, false, true>(...)"
    other = "void ck::(anonymous namespace)::rotate_quant_kernel<64, 256, 2, 2>(...)"
    a, b, c = (str(tmp_path / n) for n in ("a.csv", "b.csv", "c.csv"))
    _csv(a, [(1, other, "SQ_INSTS_VALU_MFMA_MOPS_I8", 7, 0, 1)]
         + [(d, kern, "SQ_INSTS_VALU_MFMA_MOPS_I8", 2 * M * N * K / 512, 0, 100) for d in (2, 3)]
         + [(d, kern, "SQ_VALU_MFMA_BUSY_CYCLES", mfma_instr * 32, 0, 100) for d in (2, 3)])
    _csv(b, [(2, kern, "FETCH_SIZE", 1000.0, 0, 1), (3, kern, "FETCH_SIZE", 3000.0, 0, 1)])
    _csv(c, [(2, kern, "WRITE_SIZE", 61440.0, 0, 1), (3, kern, "WRITE_SIZE", 61440.0, 0, 1)])
    bench.write_counters(name, [a, b, c], out_dir=str(tmp_path))
    text = (tmp_path / ("%s_counters.txt" % name)).read_text()
    rec = json.loads(text.split("JSON:", 1)[1])
    assert rec["dispatches_per_pass"] == 2
    assert rec["counters_mean_per_dispatch"]["FETCH_SIZE"] == 2000.0
    assert rec["mfma_ops_over_2MNK"] == 1.0
    # every MFMA busy for 32 cycles, spread over 1024 SIMDs
    assert rec["mfma_busy_cycles_per_simd"] == pytest.approx(mfma_instr * 32 / 1024, rel=1e-6)
    with open(bench.TRAFFIC_FILE) as f:
        cal = json.loads(f.read().split("JSON:", 1)[1])
    want = 2000.0 * 1024 * cal["fetch_scale"] + 61440.0 * 1024 * cal["write_scale"]
    assert rec["fabric_bytes_per_launch"] == int(round(want))
    # the commands name committed entry points only
    for line in text.splitlines():
        if line.strip().startswith("rocprofv3 --pmc"):
            assert "python3 bench.py --profile-workload %s" % name in line


def test_write_counters_rejects_files_without_the_kernel(tmp_path):
    p = str(tmp_path / "x.csv")
    _csv(p, [(1, "some_other_kernel", "FETCH_SIZE", 1.0, 0, 1)])
    with pytest.raises(SystemExit):
        bench.write_counters("rotate_quant_m8192_k10240_ld10752_g64", [p], out_dir=str(tmp_path))


def test_traffic_is_null_once_the_kernel_changes(tmp_path, monkeypatch):
    rec = {"sources_sha": "0" * 16, "hbm_bytes_per_launch": 123}
    p = tmp_path / "traffic.txt"
    p.write_text("header\nJSON: %s\n" % json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.measured_traffic(1) is None
    rec["sources_sha"] = bench.sources_sha(bench.GEMV_SOURCES)
    p.write_text("header\nJSON: %s\n" % json.dumps(rec))
    assert bench.measured_traffic(1) == 123


def test_oracle_baseline_pairs_each_workload_with_its_gpu_figure():
    also = {"w4a8_decode_gemv_m4": {"linear_us": 11.0}, "w4a8_linear_m32_k3840_n3840_g64": {"linear_us": 12.0},
            "rotate_quant_m8192_k10240_ld10752_g64": {"us": 43.0}, "awq_w4a16_gemv_m1_k3072_n18432": {"us": 8.7},
            "w4a4_linear_m8192_k3840_n3840_g64": {"linear_us": 115.0}}
    assert bench._gpu_us(also, 6.8, "w4a8_decode_gemv_k3840_n10240_g64_m1") == 6.8
    assert bench._gpu_us(also, 6.8, "w4a8_decode_gemv_k3840_n10240_g64_m4") == 11.0
    assert bench._gpu_us(also, 6.8, "w4a8_linear_m32_k3840_n3840_g64") == 12.0
    assert bench._gpu_us(also, 6.8, "rotate_quant_m8192_k10240_ld10752_g64") == 43.0
    assert bench._gpu_us(also, 6.8, "awq_w4a16_gemv_m1_k3072_n18432") == 8.7
    assert bench._gpu_us(also, 6.8, "w4a4_linear_m8192_k3840_n3840_g64") == 115.0
    assert bench._gpu_us({}, 6.8, "w4a4_linear_m8192_k10240_n3840_g256") is None
    host = bench._host_cpu()
    assert host["nproc"] >= 1 and host["affinity_cpus"] >= 1
