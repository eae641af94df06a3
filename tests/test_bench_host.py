"""Host-side checks of bench.py (no GPU): the one-GPU refusal and the byte accounting
behind `value` and `roofline.achieved`."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name,mb", [("long128k_b10", 69.0), ("long128k_b50", 337.2),
                                     ("uniform4k", 345.1)])
def test_algorithmic_bytes_per_call(name, mb):
    # 160 B per kept INT4 token and kv head, 264 B per INT8 token, plus queries,
    # outputs, mask words and block table: the per-call figures of the workload table
    w = W.WORKLOADS[name]
    L = w.lengths()
    got = bench.algorithmic_bytes(w, L, bench.kept_counts(w, L)) / 1e6
    assert abs(got - mb) / mb < 0.01, got


def test_dense_bytes_count_every_position():
    w = W.Workload("d", 4, 32, 8, 128, ctx=131072)
    L = w.lengths()
    got = bench.dense_bytes(w, L)
    kv = 4 * 8 * 131072 * 512
    assert kv <= got < kv * 1.001


def test_kept_counts_block_policy_is_a_lower_bound():
    w = W.WORKLOADS["long128k_blk_b50"]
    L = np.array([1000, 145, 144, 0])
    counts = bench.kept_counts(w, L)
    assert counts[2] == 0 and counts[3] == 0
    n4 = 1000 - 144
    assert counts[0] <= (n4 * 500 // 1000 + 16) * w.kv_heads
