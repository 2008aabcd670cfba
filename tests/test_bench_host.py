"""Host-side checks of bench.py: the one-GPU refusal, the weight-copy rule
that keeps timed launches reading HBM, and the traffic calibration of the
counter summaries.  No GPU is used."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import vqsynth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("workload", ["mlp70b", "llama8b", "smollm", "tiny", "llama8b_rvq124"])
def test_each_linear_rotates_past_the_infinity_cache(workload):
    ws, _ = vqsynth.workload_weights(workload)
    n = bench.weight_copies(ws)
    for sw in ws:
        if n < bench.MAX_COPIES:
            assert n * bench.compressed_bytes(sw) >= bench.MALL_DEFEAT_BYTES, sw.name
    assert 2 <= n <= bench.MAX_COPIES


def test_traffic_summary_scales_by_the_copy(tmp_path):
    # two dispatches of the kernel and the 1 GiB copy, whose counters read
    # half (FETCH) and all (WRITE) of the bytes it moves
    def write(path, counter, vals):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for name, v in vals:
                w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})
    kib = bench.COPY_BYTES / 1024
    write(tmp_path / "f.csv", "FETCH_SIZE", [("k_gemv_cbs<4, 28>", 1000.0), ("k_gemv_cbs<4, 28>", 1002.0),
                                             ("copyBuffer", kib / 2)])
    write(tmp_path / "w.csv", "WRITE_SIZE", [("k_gemv_cbs<4, 28>", 10.0), ("k_gemv_cbs<4, 28>", 10.0),
                                             ("copyBuffer", kib)])
    out = tmp_path / "t.json"
    bench.traffic_summary("mlp70b:28672,8192", "k_gemv_cbs", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                          str(out))
    t = json.loads(out.read_text())
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    assert t["fetch_bytes_per_launch"] == pytest.approx(1001.0 * 1024 * 2)
    assert t["traffic_bytes_per_launch"] == pytest.approx(1001.0 * 1024 * 2 + 10.0 * 1024)
    assert t["shape"] == [28672, 8192] and t["tokens"] == 1
    assert t["source_hash"] == bench.kernel_source_hash("k_gemv_cbs")
