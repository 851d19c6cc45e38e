"""bench.py's host-side contract, on the CPU: more than one GPU is refused with
a message, and the CPU baseline (the oracle, one thread and split over the
host's threads) runs on a small stand-in projection and reports its figures."""
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_matrix_vector_amd import inputs as I  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


class _Launch:
    """The fields cpu_baseline reads from a bench launch."""

    def __init__(self, R, K, seed):
        self.layer, self.dtc, self.n, self.m, self.K, self.B = 0, 0, 2, 4, K, 1
        self.x = I.activation_normal(1, K, torch.float16, seed)
        self.W = [I.weight(R, K, torch.float16, seed + 1)]
        self.R = [R]

    def part_bytes(self, i):
        return self.R[i] * self.K * 9 // 8


def test_cpu_baseline_reports_one_and_all_threads():
    out = bench.cpu_baseline([_Launch(96, 512, 3)], 0.05, torch, "stand-in")
    assert out["kind"] == "oracle" and out["cores"] == 1 and out["unit"] == "GB/s" and out["value"] > 0
    assert "1 thread" in out["sample"]
    at = out["all_threads"]
    if (os.cpu_count() or 1) > 1 and int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)) > 1:
        assert at["cores"] > 1 and at["value"] > 0
    else:
        assert at is None


def test_trials_statistics_order():
    calls = []

    class _Ev:
        def __init__(self, enable_timing=True):
            pass

        def record(self, s=None):
            pass

        def synchronize(self):
            pass

        def elapsed_time(self, other):
            calls.append(1)
            return [3.0, 1.0, 2.0][len(calls) - 1]

    class _Cuda:
        Event = _Ev

        @staticmethod
        def synchronize():
            pass

        @staticmethod
        def current_stream():
            return None

    class _Torch:
        cuda = _Cuda

    lo, med, hi = bench.trials_us(_Torch, lambda: None, 3, 1)
    assert (lo, med, hi) == (1000.0, 2000.0, 3000.0)


def test_config_steps_cover_every_other_workload():
    """The default line's extras.configs block covers the Qwen3-14B/32B MLP
    steps at 4:8 and 2:4, the Llama-3.3-70B layer sweep and the Qwen3-32B
    batches of 1/2/4/8, each over at least 8 weight instances per shape."""
    specs = bench.workloads(I)
    names = [n for n, _ in bench.CONFIG_STEPS]
    for n, layers in bench.CONFIG_STEPS:
        assert n in specs and layers >= 8, n
    for need in ("qwen3_14b_4of8", "qwen3_14b_2of4", "qwen3_32b_4of8", "qwen3_32b_2of4", "llama33_70b",
                 "qwen3_32b_b1", "qwen3_32b_b2", "qwen3_32b_b4", "qwen3_32b_b8"):
        assert need in names, need
