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
    assert bench.measured_traffic("lm_head", 1) is None          # no file
    good = {"kernel_src_sha256_16": profiling.kernel_source_hash(), "workload": "lm_head", "m": 1,
            "hbm_bytes_per_launch": 123}
    f.write_text(json.dumps(good))
    assert bench.measured_traffic("lm_head", 1) == 123
    assert bench.measured_traffic("lm_head", 2) is None          # other row count
    assert bench.measured_traffic("gate_up_bf16", 1) is None     # other workload
    f.write_text(json.dumps(dict(good, kernel_src_sha256_16="0" * 16)))
    assert bench.measured_traffic("lm_head", 1) is None          # kernel changed since


def _write_counters(d, kernel, counter, values):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        for i, v in enumerate(values):
            w.writerow([i, kernel, counter, v, 1000 * i, 1000 * i + 500])


def test_traffic_summary_scales_by_the_copy(tmp_path):
    k = "void mnb::(anonymous namespace)::mnb_gemv_kernel<1, 2, 2, 2>(Params)"
    _write_counters(tmp_path / "gf", k, "FETCH_SIZE", [100.0, 102.0, 101.0])
    _write_counters(tmp_path / "gw", k, "WRITE_SIZE", [10.0, 10.0, 10.0])
    # the copy run: a small dispatch first, then the copy of 1 MiB
    _write_counters(tmp_path / "cf", "copyBuffer", "FETCH_SIZE", [3.0, 512.0])
    _write_counters(tmp_path / "cw", "copyBuffer", "WRITE_SIZE", [1.0, 1024.0])
    out = profiling.traffic_summary(str(tmp_path / "gf"), str(tmp_path / "gw"), str(tmp_path / "cf"),
                                    str(tmp_path / "cw"), 1 << 20, "tiny_1k", 1,
                                    str(tmp_path / "t.json"), str(tmp_path / "t.md"), ["cmd"])
    assert out["fetch_scale"] == 2.0 and out["write_scale"] == 1.0
    assert out["fetch_bytes_per_launch"] == 101 * 1024 * 2      # median dispatch, scaled
    assert out["write_bytes_per_launch"] == 10 * 1024
    assert out["kernel_src_sha256_16"] == profiling.kernel_source_hash()
    assert json.loads((tmp_path / "t.json").read_text())["hbm_bytes_per_launch"] == (101 * 2 + 10) * 1024
