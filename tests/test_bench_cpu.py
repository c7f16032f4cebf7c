"""bench.py's host-side logic, without a GPU: the one-GPU guard, the kernel
code hash that ties the committed traffic counters to the kernel, the oracle
baseline's report, and the committed traffic profile's fields."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) {\n  return x + 1;  // one more\n}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["k.hip"])
    h0 = bench.kernel_hash()
    src.write_text("/* header */\nint f(int x) {\n\n    return x + 1;   // a different comment\n}\n")
    assert bench.kernel_hash() == h0
    src.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.kernel_hash() != h0


def test_cpu_baseline_report():
    pytest.importorskip("threadpoolctl")
    from workloads import get_workload, make_inputs

    wl = get_workload("tiny_fp32")
    rep = bench.cpu_baseline(wl, make_inputs(wl), 2.0, budget_s=0.0)  # stops after one head
    assert rep["kind"] == "oracle" and rep["cores"] >= 1 and rep["value"] > 0
    assert rep["unit"].startswith("TFLOP/s") and "1 of 2 heads" in rep["sample"]
    assert rep["ms_per_call"] > 0


def test_traffic_profile_fields():
    with open(bench.TRAFFIC_FILE) as f:
        tr = json.load(f)
    assert len(tr["kernel_hash"]) == 16
    assert tr["workload"] == "video_dit_32k" and tr["tau"] == 8.0
    assert tr["bytes_per_launch"] > 0
    cal = tr["calibration"]
    assert abs(cal["fetch_factor"] - 2.0) < 0.01 and abs(cal["write_factor"] - 1.0) < 0.01
