"""The benchmark's host-side contract: the one-GPU guard, the flop count of a step and the
roofline arithmetic (no GPU needed)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"] and msg["n_gpus"] == 2


def test_step_flops_are_the_sum_of_the_products():
    """fwd: x W^T, x A^T, u B^T; bwd: dy W, dy B, v A, v^T x, dy^T u (2 flops per multiply-add)."""
    T, N, K, r = 2048, 4096, 11008, 64
    products = [(T, N, K), (T, r, K), (T, N, r), (T, K, N), (T, r, N), (T, K, r), (r, K, T), (N, r, T)]
    assert bench.linear_flops(T, N, K, r) == sum(2 * m * n * k for m, n, k in products)
    assert bench.linear_flops(2048, 4096, 4096, 64) == 143_881_404_416


def test_roofline_takes_the_dominant_kernel_and_its_own_peak():
    T, N, K, r = 2048, 4096, 4096, 64
    timing = {"qgemm_fwd": (50, 4.0), "qgemm_dx": (50, 4.5), "gemv_fwd": (0, 0.0), "gemv_bwd": (0, 0.0),
              "adamw": (3, 9.0)}
    roof = bench.roofline_of(timing, T, N, K, r, 8_650_752)
    assert roof["kernel"] == "qgemm_dx" and roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s"
    flops = 2 * T * N * K + 2 * T * r * K
    avg_s = 4.5e-3 / 50
    assert roof["achieved"] == pytest.approx(flops / avg_s / 1e12)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 2516.6)
    assert set(roof["other_kernels"]) == {"qgemm_fwd"}
    few = bench.roofline_of({"qgemm_fwd": (0, 0.0), "qgemm_dx": (0, 0.0), "gemv_fwd": (200, 2.0),
                             "gemv_bwd": (200, 2.4)}, 1, N, K, r, 8_650_752)
    assert few["kernel"] == "gemv_bwd" and few["unit"] == "GB/s" and few["peak"] == 8000.0
