"""Host-side contract of bench.py (no GPU): one GPU only, and the HBM-traffic
record names the headline workload and a kernel-source hash of the form the
benchmark compares against."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_and_kernel_hash():
    assert re.fullmatch(r"[0-9a-f]{16}", bench.kernel_hash())
    assert bench.kernel_hash() == bench.kernel_hash()
    t = bench.TRAFFIC
    assert t["workload"] == workloads.HEADLINE
    assert re.fullmatch(r"[0-9a-f]{16}", t["kernel_hash"])
    assert t["bytes"] > 0
