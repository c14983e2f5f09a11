"""Host logic of bench.py: the FLOP and byte counts behind the reported
rates, and the one-GPU contract (no GPU needed)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import workload  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_work(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_flops_without_a_window_are_4_and_10_times_b_h_n2_d():
    wl = workload("bf16_b2h32_n8192_d128_q3")
    fwd, bwd = bench.flops(wl)
    base = wl.B * wl.H * wl.n ** 2 * wl.d
    assert fwd == 4.0 * base and bwd == 10.0 * base
    assert abs((fwd + bwd) - 7.697e12) < 1e9  # the headline workload's 7.697 TFLOP per step


def test_flops_with_a_window_count_the_visible_pairs():
    wl = workload("bf16_b2h8_n16384_d256_w512")
    n, w = wl.n, wl.window
    pairs = n * (2 * w + 1) - w * (w + 1)  # |i - j| <= w inside [0, n)
    assert bench.flops(wl, pairs=True) == pairs
    fwd, bwd = bench.flops(wl)
    assert fwd == 4.0 * pairs * wl.B * wl.H * wl.d and bwd == 10.0 * pairs * wl.B * wl.H * wl.d
    assert abs(pairs / n ** 2 - 0.061583) < 1e-6


def test_algorithmic_bytes_read_inputs_once_and_write_outputs_once():
    wl = workload("bf16_b2h32_n8192_d128_q3")
    t = wl.B * wl.H * wl.n * wl.d * 2  # one bf16 [B, H, n, d] tensor
    r = wl.B * wl.H * wl.n * 4         # one fp32 [B, H, n] row array
    fwd, bwd = bench.hbm_bytes(wl)
    assert fwd == 4 * t + r            # Q, K, V in; O, LSE out
    assert bwd == 8 * t + 3 * r        # Q, K, V, O, dO, LSE in; dQ, dK, dV out; D written and read
