"""The bench's host logic, on the CPU: the one-GPU guard, the algorithmic flop and byte
counts it prices kernels with, and the reading of recorded HBM traffic."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_flop_counts_at_the_flux_qkv_shape():
    M, K, N, r = 4608, 3072, 9216, 32
    # the 4-bit product, then the branches: T L2^T inside the GEMM, X L1^T beside it, and
    # the rank-1 term mu wbar^T
    assert bench.gemm_flops(M, K, N, r, True) == 2 * M * N * K + 2 * M * N * r + 2 * M * N
    assert bench.gemm_flops(M, K, N, 0, False) == 2 * M * N * K
    assert bench.layer_flops(M, K, N, r, True) - bench.gemm_flops(M, K, N, r, True) == 2 * M * K * r


def test_byte_counts_at_the_flux_qkv_shape():
    M, K, N, r = 4608, 3072, 9216, 32
    # fp16 in; a byte per two codes and one per 32-element block out; a fp16 mean per token
    assert bench.transform_bytes(M, K, True) == M * K * 2 + M * K // 2 + M * K // 32 + 2 * M
    assert bench.transform_bytes(M, K, True) / (M * K) == pytest.approx(2.53125, abs=1e-3)
    # packed operands with their scales, T and L2, mu and wbar, fp16 Y
    want = (M + N) * (K // 2 + K // 32) + 2 * r * (M + N) + 2 * (M + N) + 2 * M * N
    assert bench.gemm_bytes(M, K, N, r, True) == want


@pytest.mark.parametrize("kind", ["w4a4_gemm", "transform"])
def test_recorded_traffic_is_per_layer_or_absent(kind):
    """A record counts only for the kernel source it was taken on: either all three layers
    or nothing."""
    t = bench.recorded_traffic(kind)
    assert t is None or (set(t) == {"qkv", "fc1", "fc2"} and all(v > 0 for v in t.values()))


def test_composite_floor_prices_each_product_at_its_own_peak():
    """The linear's floor: the 4-bit product at the MXFP4 peak, both fp16 low-rank
    projections (X L1^T and T L2^T) at the fp16 peak."""
    M, K, N, r = 4608, 3072, 9216, 32
    want = 2 * M * N * K / 10.1e15 + 2 * M * r * (K + N) / 2.5e15
    assert bench.composite_floor_s(M, K, N, r) == pytest.approx(want, rel=1e-12)
    assert bench.composite_floor_s(M, K, N, 0) == pytest.approx(2 * M * N * K / 10.1e15, rel=1e-12)
