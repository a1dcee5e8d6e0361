"""bench.py's command-line contract on the CPU (no GPU is touched)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                          text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr and proc.stdout == ""


def test_traffic_counters_apply_only_to_their_workload_and_source(tmp_path):
    sys.path.insert(0, ROOT)
    import bench
    assert bench.counted_traffic("480p") is None
    # a counter record whose source hash does not match reports nothing
    stale = dict(bench.HBM_COUNTERS, source_sha256="0" * 64)
    assert bench.counted_traffic("1344x768", stale) is None
    missing = dict(bench.HBM_COUNTERS, source="no/such/file.hip")
    assert bench.counted_traffic("1344x768", missing) is None
