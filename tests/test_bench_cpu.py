"""bench.py's host-side logic, without a GPU: the one-GPU guard, the kernel
code hash that ties the committed traffic counters to the kernel, the oracle
baseline's report, and the committed traffic profile's fields."""
import json
import os
import subprocess
import sys

import numpy as np
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
    rep, par = bench.cpu_baseline(wl, make_inputs(wl), 2.0, budget_s=0.0)  # stops after one head
    assert par is None
    assert rep["kind"] == "oracle" and rep["cores"] >= 1 and rep["value"] > 0
    assert rep["cores"] == rep["usable_cores"] == bench.usable_cores()
    assert rep["unit"].startswith("TFLOP/s") and "1 of 2 heads" in rep["sample"]
    assert rep["ms_per_call"] > 0 and rep["host_cpu"]


def test_parity_witness_logic():
    """The bench's comparison of a GPU result with the oracle, fed results
    made on the CPU: the oracle's own output passes; a decision flipped away
    from the threshold, a wrong row or a NaN fails; a decision flipped
    inside the tie band is followed, not counted."""
    from oracle import attend_head
    from workloads import bf16_bits_to_f64, get_workload, make_inputs

    wl = get_workload("tiny_fp32")
    x = make_inputs(wl)
    q, k, v = (bf16_bits_to_f64(x[n][0, 0]) for n in "qkv")
    tau = 2.0
    ref = attend_head(q, k, v, 64, 64, tau)
    err, out_, in_ = bench.compare_head(ref["out"].copy(), ref["keep"].copy(), q, k, v, ref, 64, 64, tau)
    assert err == 0.0 and out_ == 0 and in_ == 0
    # flip the decision of the block farthest from the threshold
    gap = np.abs(ref["s"] - (ref["M"] - tau)[:, None])
    i, j = np.unravel_index(np.argmax(gap), gap.shape)
    keep = ref["keep"].copy()
    keep[i, j] = ~keep[i, j]
    _, out_, _ = bench.compare_head(ref["out"], keep, q, k, v, ref, 64, 64, tau)
    assert out_ == 1
    # a decision inside the band: the oracle follows the GPU there
    theta = ref["M"] - tau
    s2 = ref["s"].copy()
    i2, j2 = 3, int(np.argmin(np.abs(ref["s"][3] - theta[3]) + 1e9 * (np.arange(wl.Nk) == ref["s"][3].argmax())))
    s2[i2, j2] = theta[i2]  # on the threshold: kept by the oracle's rule
    ref2 = dict(ref, s=s2)
    keep2 = ref["keep"].copy()
    keep2[i2, j2] = ~keep2[i2, j2]
    gpu_out = attend_head(q, k, v, 64, 64, tau, keep_override=keep2)["out"]
    err, out_, in_ = bench.compare_head(gpu_out, keep2, q, k, v, ref2, 64, 64, tau)
    assert out_ == 0 and in_ == 1 and err < 1e-12
    bad = ref["out"].copy()
    bad[70, 5] += 0.05
    assert bench.compare_head(bad, ref["keep"], q, k, v, ref, 64, 64, tau)[0] > 0.04
    bad[70, 5] = np.nan
    assert bench.compare_head(bad, ref["keep"], q, k, v, ref, 64, 64, tau)[0] == float("inf")


def test_traffic_profile_fields():
    with open(bench.TRAFFIC_FILE) as f:
        tr = json.load(f)
    assert len(tr["kernel_hash"]) == 16
    assert tr["workload"] == "video_dit_32k" and tr["tau"] == 8.0
    assert tr["bytes_per_launch"] > 0
    cal = tr["calibration"]
    assert abs(cal["fetch_factor"] - 2.0) < 0.01 and abs(cal["write_factor"] - 1.0) < 0.01
