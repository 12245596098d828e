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


class _FakeCuda:
    """Stand-in for torch.cuda: each call of the timed case advances a GPU
    clock by a fixed number of milliseconds; events read that clock."""

    def __init__(self, ms_per_call):
        self.now = 0.0
        self.ms = ms_per_call

    class _Event:
        def __init__(self, cuda):
            self.cuda, self.t = cuda, None

        def record(self):
            self.t = self.cuda.now

        def elapsed_time(self, other):
            return other.t - self.t

    def Event(self, enable_timing=True):
        return _FakeCuda._Event(self)

    def synchronize(self):
        pass


class _FakeTorch:
    def __init__(self, ms_per_call):
        self.cuda = _FakeCuda(ms_per_call)


def _counting_case(torch_like):
    calls = []

    def case():
        calls.append(1)
        torch_like.cuda.now += torch_like.cuda.ms
    return case, calls


def test_warm_up_takes_the_step_count_then_batches_until_the_time_floor():
    t = _FakeTorch(ms_per_call=0.75)
    case, calls = _counting_case(t)
    bench.warm_up(case, 3, t)                        # no time floor: exactly 3 calls
    assert len(calls) == 3
    calls.clear()
    bench.warm_up(case, 3, t, warm_ms=50.0)          # 3, then batches of 5 past 50 ms
    # 2.25 ms after the 3 calls, then 13 batches of 3.75 ms reach 51 ms
    assert len(calls) == 3 + 5 * 13
    assert len(calls) * 0.75 >= 50.0 and (len(calls) - 5) * 0.75 < 50.0


def test_time_case_times_exactly_the_steps_after_the_warm_up():
    t = _FakeTorch(ms_per_call=2.0)
    case, calls = _counting_case(t)
    ms, _ = bench.time_case(case, 20, 60, t)
    assert len(calls) == 80 and ms == 2.0
