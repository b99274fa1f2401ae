"""Host-side checks of bench.py (no GPU work): the one-GPU contract and the
FLOP model's basic properties."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_flop_model():
    T, H, F, k = bench.TOKENS, bench.HIDDEN, bench.FFN, bench.K_RANK
    assert bench.dense_equiv_flops() == 3 * 6 * T * H * F
    # the split product costs the dense residual GEMM plus a small rank-k overhead
    for M, N, K in ((T, F, H), (T, H, F), (H, F, T)):
        f = bench.split_gemm_flops(M, N, K, k, k)
        assert 2 * M * N * K < f < 1.2 * 2 * M * N * K
    # the sketch is counted on refresh steps only
    assert bench.decompose_flops(T, H, k, 8, bench.L_K, True) > bench.decompose_flops(T, H, k, 8, bench.L_K, False) > 0
    assert bench.residual_flops(T, H, k) > 0
