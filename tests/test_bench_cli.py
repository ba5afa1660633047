"""bench.py's host-side contract (CPU): one GPU only, and the committed
counter figures are used only while the kernel sources they were taken on
are unchanged."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_follows_the_committed_counters(monkeypatch):
    """The counter figure is reported while its source hash matches the
    kernel sources, and null as soon as they differ."""
    c = json.load(open(os.path.join(ROOT, "profiles", "greedy_counters.json")))
    assert abs(c["hbm_bytes_per_launch"] / (256 * 9 * 151936 * 2) - 1) < 0.01
    monkeypatch.setattr(bench, "source_hash", lambda paths: c["source_hash"])
    assert bench.load_traffic("greedy") == c["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "source_hash", lambda paths: "0" * 16)
    assert bench.load_traffic("greedy") is None


def test_metric_and_workload_names():
    assert bench.METRIC
    assert set(bench.LAUNCH_KERNELS) == {"greedy", "tree", "rejection"}
