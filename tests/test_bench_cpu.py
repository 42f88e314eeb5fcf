"""Host logic of bench.py (no GPU): the one-GPU refusal, the settling loop and
the committed traffic counters' source check."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


class _CountingRun:
    def __init__(self):
        self.fused_calls = self.three_calls = 0

    def fused(self, att):
        self.fused_calls += 1

    def three(self, att):
        self.three_calls += 1


class _Torch:
    class cuda:
        @staticmethod
        def synchronize():
            pass


def test_settle_runs_both_forms_and_stops():
    run = _CountingRun()
    assert bench.settle(run, None, _Torch, 0.0) == 0
    n = bench.settle(run, None, _Torch, 0.01)
    assert n > 0 and n % 25 == 0
    assert run.fused_calls == run.three_calls == n


def test_traffic_counters_follow_the_kernel_source():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    entry = bench.traffic_entry(bench.FUSED_KERNEL)
    if t["source_hash"] == bench.source_hash():
        assert entry == t["kernels"][bench.FUSED_KERNEL]["hbm_bytes_per_launch"]
        # every K/V byte fetched once, plus a little (q, page table, partials)
        assert 1.0 <= t["kernels"][bench.FUSED_KERNEL]["read_over_algorithmic"] < 1.05
    else:
        assert entry is None
