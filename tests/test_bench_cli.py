"""bench.py's command-line contract and host-side helpers, on the host (no GPU is touched)."""
import os
import subprocess
import sys

import pytest

import bench
from token_level_sparse_kv_amd.perfmodel import step_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    # the step is measured on one GPU's share; --gpus N > 1 exits at once with a message
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_host_info_reports_the_pool_apart_from_the_core_counts():
    h = bench.host_info()
    assert h["os_cpu_count"] == os.cpu_count()
    assert 1 <= h["affinity_cpus"] <= os.cpu_count()
    assert 1 <= h["pool_threads"] <= min(16, h["affinity_cpus"])
    assert isinstance(h["cpu_model"], str)


def test_committed_scan_counters_match_the_byte_model():
    # the counter summary is used only while the scan's sources hash to the recorded
    # value; when it is, its bytes per launch lie just above the algorithmic bytes (the
    # prep's sample rows and the candidate writes are the excess) and never below them
    t = bench.traffic_from_profile()
    if t is None:
        pytest.skip("the scan's sources changed since the counters were taken (traffic is reported as null)")
    b = step_bytes(16, 8, 4, 128, 32, 131072, 4096)
    algorithmic = b["scan_kproj"] + b["q"] + b["M"] + b["append"]
    assert algorithmic <= t <= 1.05 * algorithmic
