"""The benchmark's host side (no GPU): its one-GPU contract, its algorithmic byte accounting pinned
to the per-token figures of the hot path at the Zamba2-2.7B mixer shape (d_inner 5120 = 80 heads of
headdim 64, d_state 64, one B/C group, conv width 4: 5248 conv channels), and the rule that a
committed traffic or counter figure is reported only for the kernel sources it was measured on."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
H, P, N, G, W = 80, 64, 64, 1, 4
CD = H * P + 2 * G * N
STATE = H * P * N * 4          # one sequence's fp32 state: 1.31 MB


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_two_kernel_prefill_bytes_per_token():
    """conv: read xBC + write the activation, 4 bytes per channel and token (20,992 B); scan: read x, B,
    C, dt and write y (20,896 B); with the 32k prompt's final state, 41,928 B per token."""
    B, L = 1, 32768
    conv, scan = bench.prefill_bytes(B, L, H, P, N, G, W, CD, False, True)
    conv_params = CD * W * 4 + CD * 4 + B * W * CD * 2       # taps, bias, ring out
    scan_params = 3 * H * 4                                  # dt_bias, A, D
    assert (conv - conv_params) == 20992 * B * L
    assert (scan - scan_params - STATE) == 20896 * B * L
    assert (conv - conv_params + scan - scan_params) / (B * L) == pytest.approx(41928, abs=0.5)


def test_batched_prefill_bytes_with_state_in_and_out():
    """8 x 4096 with an initial state read and the final state written: 42,528 B per token."""
    B, L = 8, 4096
    conv, scan = bench.prefill_bytes(B, L, H, P, N, G, W, CD, True, True)
    conv_params = CD * W * 4 + CD * 4 + B * W * CD * 2
    per_tok = (conv - conv_params + scan - 3 * H * 4) / (B * L)
    assert per_tok == pytest.approx(42528, abs=0.5)


def test_one_pass_prefill_bytes_per_token():
    """The one-pass path reads the raw xBC rows and dt and writes y: the same 20,896 B per token as the
    scan alone (the conv output never reaches memory)."""
    B, L = 1, 32768
    f = bench.fused_bytes(B, L, H, P, N, G, W, CD, False, True)
    params = CD * (W + 1) * 4 + 3 * H * 4 + B * W * CD * 2
    assert (f - params - STATE) == 20896 * B * L


def test_decode_step_bytes_per_token():
    """One decode step of 256 sequences: the fp32 state read and written (2,621,440 B per sequence) plus
    the ring window, the new token, its ring slot, dt and y: 2,684,320 B per token."""
    B = 256
    s = bench.step_bytes(B, H, P, N, G, W, CD)
    params = CD * (W + 1) * 4 + 3 * H * 4
    assert (s - params) == 2684320 * B


def test_recorded_figures_follow_the_kernel_sources(monkeypatch):
    """traffic.json / counters.json figures are reported only while the sources hash as profiled."""
    for path in (bench.TRAFFIC_FILE, bench.COUNTERS_FILE):
        with open(path) as fh:
            kernels = json.load(fh)["kernels"]
        assert set(kernels) <= set(bench.KERNEL_SOURCES)
    for k, files in bench.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(ROOT, "selective_state_space_mixer_amd", "csrc", f)), (k, f)
    with open(bench.TRAFFIC_FILE) as fh:
        recorded = json.load(fh)["kernels"]["ssd_scan"]
    monkeypatch.setattr(bench, "source_digest", lambda kernel: recorded["source_sha256"])
    assert bench.measured_traffic("ssd_scan") == recorded["bytes_per_launch"]
    monkeypatch.setattr(bench, "source_digest", lambda kernel: "0" * 64)
    assert bench.measured_traffic("ssd_scan") is None
    assert bench.measured_mfma("ssd_scan") is None
