"""Host-side logic of bench.py (no GPU): the single-GPU contract, the
algorithmic work formulas behind the roofline figures, and the rule that
measured HBM traffic is reported only for the sources it was measured on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2 and "single GPU" in r.stderr


@pytest.mark.parametrize("B,H,T,D,W,C,gflop", [
    (8, 8, 1024, 64, 256, 64, 4.974),     # training-shape prefill
    (1, 12, 32768, 64, 1024, 128, 114.0),  # long prefill
])
def test_forward_flops(B, H, T, D, W, C, gflop):
    # band pairs W(W+1)/2 + (T-W)W at 4D flops each, plus 4D^2 + 2D(C+1) per evicted query
    assert abs(bench.fwd_flops(B, H, T, D, W, C) / 1e9 - gflop) < 0.001 * gflop


def test_forward_flops_small_cases_by_counting():
    B, H, T, D, W, C = 1, 1, 10, 4, 3, 2
    pairs = sum(min(W, t + 1) for t in range(T))
    evicted = sum(1 for t in range(T) if t >= W)
    assert bench.fwd_flops(B, H, T, D, W, C) == 4 * D * pairs + evicted * (4 * D * D + 2 * D * (C + 1))
    assert bench.fwd_flops(1, 1, 5, 4, 8, 2) == 4 * 4 * 15  # T < W: causal pairs only, nothing evicted


def test_backward_flops_and_decode_bytes():
    assert abs(bench.bwd_flops(4, 16, 8192, 128, 512, 64) / 1e9 - 429.8) < 0.1
    # decode step: the whole ring once, the slot write, A read + write, q/k/v in and y out
    assert bench.decode_bytes(64, 32, 128, 4096) == 64 * 32 * (2 * 4096 * 128 * 2 + 2 * 128 * 2 + 8 * 128 * 128
                                                                + 4 * 128 * 2)
    assert abs(bench.decode_bytes(64, 32, 128, 4096) / 1e9 - 4.5665) < 1e-3


def test_traffic_only_for_the_measured_sources(monkeypatch):
    real = bench.measured_traffic()
    monkeypatch.setattr(bench, "csrc_digest", lambda: "0" * 64)
    assert bench.measured_traffic() == {}
    if real:  # the committed summary carries every leg the bench reports
        assert {"prefill", "long", "decode", "backward", "train_forward", "continue"} <= set(real)


def test_roofline_chunk_never_exceeds_the_kernel_read_chunk():
    # bf16: 128-row query blocks read one 128-eviction chunk; float32: 64
    assert bench.roofline_chunk(128, 64) == 128      # long-context prefill: charged as configured
    assert bench.roofline_chunk(64, 64) == 64        # training-shape prefill: the configured, smaller chunk
    assert bench.roofline_chunk(64, 128) == 64       # D = 128 training forward: its configured C = 64
    assert bench.roofline_chunk(512, 128) == 128     # a larger C is charged at the kernel's chunk
    assert bench.roofline_chunk(512, 64) == 128
    assert bench.roofline_chunk(128, 64, "f32") == 64
