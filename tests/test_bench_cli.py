"""bench.py command-line contract, checked without a GPU: it measures one
GPU and says so when asked for more, and its algorithmic work figures are
the per-token-head counts of the method."""
import os
import subprocess
import sys

import bench

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=REPO)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_work_per_token_head():
    # 4dm + 4F(d+1) flops per token-head: trig F = 2m, ReLU F = m
    B, H, L, d, m = 4, 8, 4096, 64, 256
    fl, nb = bench.path_total_work(B, H, L, d, m, "trig")
    assert fl == B * H * L * (4 * d * m + 4 * 2 * m * (d + 1))
    assert fl // (B * H * L) == 198656
    fl_relu, _ = bench.path_total_work(B, H, L, d, m, "relu")
    assert fl_relu // (B * H * L) == 132096
    # read q, k, v and write out, bf16
    assert nb == B * H * L * 4 * d * 2
