"""Host-side logic of the measurement tools, without a GPU: bench.py's
single-GPU contract and committed-traffic lookup, and the rocprofv3 CSV
summaries of the profiling module on small synthetic CSV files."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_wise_int4_matmulnbits_amd import profiling  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       env=dict(os.environ, **env), capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_measured_traffic_needs_the_current_kernel(tmp_path, monkeypatch):
    f = tmp_path / "t.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("lm_head", 1, "bf16") is None          # no file
    entry = {"fetch_bytes": 100, "write_bytes": 23, "kernel_mean_us": 1.0}
    good = {"kernel_src_sha256_16": profiling.kernel_source_hash(),
            "configs": {"lm_head:1:bf16": entry}}
    f.write_text(json.dumps(good))
    assert bench.measured_traffic("lm_head", 1, "bf16") == 123
    assert bench.measured_traffic("lm_head", 1, "f16") is None           # other output type
    assert bench.measured_traffic("lm_head", 2, "bf16") is None          # other row count
    assert bench.measured_traffic("gate_up_bf16", 1, "bf16") is None     # other workload
    f.write_text(json.dumps(dict(good, kernel_src_sha256_16="0" * 16)))
    assert bench.measured_traffic("lm_head", 1, "bf16") is None          # sources changed since


def test_source_hash_covers_kernels_planner_and_header():
    names = {os.path.basename(p) for p in profiling.source_files()}
    assert {"mnb_gemv.hip", "mnb_gemv_mfma4.hip", "mnb_device.h", "mnb_api.cpp", "mnb.h"} <= names


def _write_counters(d, kernel, counter, values):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        for i, v in enumerate(values):
            w.writerow([i, kernel, counter, v, 1000 * i, 1000 * i + 500])


def _write_trace(d, kernel, durations_ns):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "VGPR_Count", "Accum_VGPR_Count",
                    "Grid_Size_X", "Workgroup_Size_X", "LDS_Block_Size"])
        t = 0
        for dur in durations_ns:
            w.writerow([kernel, t, t + dur, 84, 0, 1024 * 448, 448, 9216])
            t += dur + 100


def test_decode_summary_scales_by_the_copy(tmp_path):
    k = "void mnb::(anonymous namespace)::mnb_gemv_mfma4_kernel<1, 4, 1>(Params)"
    cfg = tmp_path / "down_rows_bf16:2:bf16"
    _write_trace(cfg / "trace", k, [50000] * 5 + [11000] * 500)      # warm-up, then the timed region
    _write_counters(cfg / "fetch", k, "FETCH_SIZE", [100.0, 102.0, 101.0])
    _write_counters(cfg / "write", k, "WRITE_SIZE", [10.0, 10.0, 10.0])
    (cfg / "trace" / "cmd.txt").write_text("trace cmd")
    # the copy runs: a small dispatch first, then the copy of 1 MiB
    _write_counters(tmp_path / "copy_fetch", "copyBuffer", "FETCH_SIZE", [3.0, 512.0])
    _write_counters(tmp_path / "copy_write", "copyBuffer", "WRITE_SIZE", [1.0, 1024.0])
    for kind in ("fetch", "write"):
        (tmp_path / ("copy_" + kind) / "bytes.txt").write_text(str(1 << 20))
    out = profiling.decode_summary(str(tmp_path), str(tmp_path / "t.json"), str(tmp_path / "t.md"))
    assert out["fetch_scale"] == 2.0 and out["write_scale"] == 1.0
    e = out["configs"]["down_rows_bf16:2:bf16"]
    assert e["kernel_mean_us"] == 11.0                      # the last 500 dispatches only
    assert e["kernel"] == "mnb_gemv_mfma4_kernel<1, 4, 1>" and e["vgprs_allocated"] == 168
    assert e["fetch_bytes"] == 101 * 1024 * 2                # median dispatch, scaled
    assert e["write_bytes"] == 10 * 1024
    assert e["algorithmic_bytes"] == 34021376
    assert abs(e["fetch_frac_of_8TBs"] - 101 * 2048 / 11e-6 / 8e12) < 1e-4
    assert e["cmd_trace"] == "trace cmd" and e["vgprs_traced"] == 84
    assert out["kernel_src_sha256_16"] == profiling.kernel_source_hash()
    saved = json.loads((tmp_path / "t.json").read_text())
    assert saved["configs"]["down_rows_bf16:2:bf16"]["fetch_bytes"] == 101 * 2048
