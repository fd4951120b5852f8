#!/usr/bin/env python3
"""Throughput of the Mamba-2 mixer hot path on one MI355X.

Headline (`value`): prefill tokens/s of one step = conv1d+SiLU and the chunked SSD scan over a
batch-1, 32768-token prompt at the Zamba2-2.7B mixer shape (d_model 2560, expand 2 -> 80 heads of
headdim 64, d_state 64, one B/C group, conv width 4), bf16 activations and fp32 state, inputs
resident in HBM, through the one-pass entry point m2_mixer_prefill_fwd (the conv output is never
written).  The same run times the two-kernel path (m2_conv1d_fwd then m2_ssd_scan_fwd) on the same
prompt, the same tokens as 8 packed prompts (two kernels, and one pass), the gated RMSNorm, the fused decode step on 256
sequences (the `decode` object) and the library's streaming copy (the attainable-bandwidth
reference).  Each entry point's average time comes from HIP events recorded on the stream it runs on,
around each of its calls in the order the path makes them, and is turned into a roofline fraction
with the algorithmic bytes it must move (the two-kernel path's entry points are also timed repeated
by themselves: `us_alone`).  The fp64 CPU oracle
is timed on a bounded sample of the same prefill on the host cores (`cpu_baseline`).

    python bench.py [--steps K] [--warmup W] [--decode-steps S] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD mixer tokens/s at 2.7B shape (32k prefill, decode) + % HBM roofline"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # untimed passes before each timed region: the device reaches its steady clocks after ~10 ms of
    # sustained work (3 warm-up passes left the 32k prefill 3-5% slower than 20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target length of the oracle sample")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "backward"], default="all")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (counter calibration) and exit")
    return ap.parse_args()


def prefill_bytes(B, L, H, P, N, G, W, Cd, with_state_in, with_state_out):
    """Algorithmic HBM bytes of one launch of each prefill kernel (bf16 activations)."""
    conv = B * L * Cd * 2 * 2 + Cd * W * 4 + Cd * 4 + B * W * Cd * 2  # read xBC, write act, params, ring out
    scan = B * L * (H * P * 2 + 2 * G * N * 2 + H * 2 + H * P * 2) + 3 * H * 4
    scan += (B * H * P * N * 4) * (int(with_state_in) + int(with_state_out))
    return conv, scan


def fused_bytes(B, L, H, P, N, G, W, Cd, with_state_in, with_state_out):
    """Algorithmic HBM bytes of one m2_mixer_prefill_fwd call: read the raw xBC and dt, write y, the
    parameters, the ring and the states (the conv output never leaves the chip)."""
    b = B * L * (Cd * 2 + H * 2 + H * P * 2) + Cd * (W + 1) * 4 + 3 * H * 4 + B * W * Cd * 2
    return b + (B * H * P * N * 4) * (int(with_state_in) + int(with_state_out))


def step_bytes(B, H, P, N, G, W, Cd):
    """Algorithmic HBM bytes of one decode-step launch: state read+write, ring W-1 reads + 1 write,
    the new token, dt, y, parameters."""
    return (B * H * P * N * 4 * 2 + B * (W - 1) * Cd * 2 + B * Cd * 2 + B * Cd * 2 + B * H * 2 + B * H * P * 2
            + Cd * (W + 1) * 4 + 3 * H * 4)


def bwd_bytes(B, L, H, P, N, G, with_state_in, with_dstate_out, with_dstate_in):
    """Algorithmic HBM bytes of one m2_ssd_scan_bwd launch (bf16 activations): read x, B, C, dt and dy,
    write dx, dB, dC and d(dt), the parameters and their gradients, and the states."""
    b = B * L * 2 * (2 * (H * P + 2 * G * N + H) + H * P) + 3 * H * 4 + 3 * H * 4
    return b + (B * H * P * N * 4) * (int(with_state_in) + int(with_dstate_out) + int(with_dstate_in))


def bwd_flops(B, L, H):
    """MFMA flops of one m2_ssd_scan_bwd launch at headdim 64 / d_state 64 as the kernels issue them
    (16,384 per v_mfma_f32_16x16x32_bf16): per head and 64-token chunk 128 for the chunk's state and
    adjoint contributions and 416 for the gradients, plus 32 per (sequence, group, chunk) for C.B."""
    nch = (L + 63) // 64
    return 16384 * (B * nch * H * (128 + 416))


def time_events(torch, fns, steps, warmup, alone=None):
    """Per-callable mean ms and the mean ms of one pass of all callables in order, over `steps` passes.

    The per-callable times come from an event pair around each call inside those passes, so every
    kernel is timed where the path runs it (the scan right after the conv whose output it reads).  The
    pass time comes from a second region of `steps` passes with no events inside; the wall ms of that
    region is returned too.  With `alone` (a list), the mean ms of `steps` back-to-back calls of each
    callable by itself is appended to it (a repeated conv runs slower: each call's output is still
    being written back from the caches when the next call starts)."""
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    if alone is not None:
        for f in fns:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                f()
            e1.record()
            torch.cuda.synchronize()
            alone.append(e0.elapsed_time(e1) / steps)
    marks = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
             for _ in range(steps)]
    for s in range(steps):
        for (e0, e1), f in zip(marks[s], fns):
            e0.record()
            f()
            e1.record()
    torch.cuda.synchronize()
    per = [sum(marks[s][i][0].elapsed_time(marks[s][i][1]) for s in range(steps)) / steps for i in range(len(fns))]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        for f in fns:
            f()
    end.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return per, start.elapsed_time(end), wall


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
_SCAN_SRC = ("ssd_scan.hip", "ssd_walk.hip", "ssd_common.h")
KERNEL_SOURCES = {"ssd_scan": _SCAN_SRC, "conv1d": ("conv1d.hip",), "ssd_step": ("ssd_step.hip",),
                  "mixer_prefill_packed": _SCAN_SRC + ("conv1d.hip",),
                  "gated_rmsnorm": ("gated_norm.hip",), "ssd_scan_packed": _SCAN_SRC, "conv1d_packed": ("conv1d.hip",),
                  "mixer_prefill": _SCAN_SRC + ("conv1d.hip",), "ssd_scan_bwd": ("ssd_bwd.hip", "ssd_common.h")}


def source_digest(kernel):
    """sha256 of the entry point's kernel sources and the shared device header (counters go stale when any
    of them changes)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ("m2_device.h",):
        with open(os.path.join(ROOT, "selective_state_space_mixer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, scaled by the
    plain-copy calibration; None if absent or taken on a different version of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
        e = t["kernels"][kernel]
        if e.get("source_sha256") != source_digest(kernel):
            return None
        return int(e["bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")


def measured_mfma(kernel):
    """MFMA utilisation of the entry point's main pass from the committed rocprofv3 SQ-counter summary
    (MFMA pipe busy fraction, achieved MFMA TFLOP/s and its fraction of the dense bf16 peak); None if
    absent or taken on a different version of the kernel source."""
    try:
        with open(COUNTERS_FILE) as fh:
            e = json.load(fh)["kernels"][kernel]
        if e.get("source_sha256") != source_digest(kernel):
            return None
        return {k: e[k] for k in ("kernel", "mfma_busy", "mfma_tflops", "mfma_frac_of_peak", "valu_per_wave",
                                  "mfma_per_wave")}
    except (OSError, KeyError, ValueError):
        return None


COPY_CEILING = [None]   # GB/s of the library's streaming copy, measured first in this run


def roofline(bytes_per_launch, ms, kernel=None):
    gbs = bytes_per_launch / (ms * 1e-3) / 1e9
    r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(kernel) if kernel else None}
    if r["traffic"] is not None:
        # the counters are not collected in this run: the figure is the committed rocprofv3 summary's, valid
        # while the kernel sources hash to what was profiled
        r["traffic_source"] = "profiles/traffic.json (rocprofv3 FETCH_SIZE/WRITE_SIZE, calibrated)"
    if COPY_CEILING[0]:
        r["frac_of_copy"] = round(gbs / COPY_CEILING[0], 4)
    return r


def bench_prefill(torch, m2, workloads, args):
    cfg = workloads.CONFIGS[3]
    d = cfg.dims
    inp = workloads.config_inputs(3)
    B, L, H, P, N, G, W, Cd = d.batch, d.seqlen, d.nheads, d.headdim, d.d_state, d.n_groups, d.d_conv, d.conv_dim
    dims = m2.make_dims(B, L, d.d_model, d.expand, P, N, G, W, d.chunk_size, d.io)
    bf = torch.bfloat16
    xbc = torch.from_numpy(inp.xbc).to("cuda", bf)
    dt = torch.from_numpy(inp.dt_raw).to("cuda", bf)
    cw, cb, dtb, A, D = (torch.from_numpy(a).cuda() for a in (inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D))
    act = torch.empty((B, L, Cd), device="cuda", dtype=bf)
    ring_out = torch.empty((B, W, Cd), device="cuda", dtype=bf)
    y = torch.empty((B, L, H * P), device="cuda", dtype=bf)
    s_out = torch.empty((B, H, P, N), device="cuda")
    nws = m2.m2_ssd_scan_workspace(dims)
    ws = torch.empty(max(nws, 1), device="cuda", dtype=torch.uint8) if nws else None
    xv, bv, cv = act[:, :, :H * P], act[:, :, H * P:H * P + G * N], act[:, :, H * P + G * N:]
    del inp

    nwf = m2.m2_mixer_prefill_workspace(dims)
    wsf = torch.empty(max(nwf, 1), device="cuda", dtype=torch.uint8)
    y2 = torch.empty_like(y)
    s_out2 = torch.empty_like(s_out)
    ring2 = torch.empty_like(ring_out)

    def fused():
        m2.m2_mixer_prefill_fwd(dims, xbc, cw, cb, dt, dtb, A, D, y2, None, 0, ring2, None, s_out2, workspace=wsf)

    def conv():
        m2.m2_conv1d_fwd(dims, xbc, cw, cb, act, None, 0, ring_out)

    def scan():
        m2.m2_ssd_scan_fwd(dims, xv, bv, cv, dt, dtb, A, D, y, None, s_out, workspace=ws)

    # one event-timed region of `steps` back-to-back calls gives both the step time and the entry
    # point's time (they are the same calls), so the roofline and ms_per_step agree
    _, fused_total, wall_ms = time_events(torch, [fused], args.steps, args.warmup)
    t_fused = fused_total / args.steps
    alone = []
    (t_conv, t_scan), two_total, _ = time_events(torch, [conv, scan], args.steps, args.warmup, alone)
    conv_b, scan_b = prefill_bytes(B, L, H, P, N, G, W, Cd, False, True)
    fused_b = fused_bytes(B, L, H, P, N, G, W, Cd, False, True)
    step_ms = fused_total / args.steps
    two_ms = two_total / args.steps
    tok = B * L
    # the two-kernel path's algorithmic bytes set the roofline tokens/s the prefill is judged against
    roof_tok_s = tok / ((conv_b + scan_b) / (HBM_PEAK_GBS * 1e9))
    return {
        "tokens_per_s": tok / (step_ms * 1e-3), "ms_per_step": step_ms, "wall_ms": wall_ms,
        "kernels": {"mixer_prefill": {"ms": t_fused, "bytes": fused_b,
                                      "roofline": roofline(fused_b, t_fused, "mixer_prefill")},
                    "conv1d": {"ms": t_conv, "bytes": conv_b, "roofline": roofline(conv_b, t_conv, "conv1d"),
                               "ms_alone": alone[0]},
                    "ssd_scan": {"ms": t_scan, "bytes": scan_b, "roofline": roofline(scan_b, t_scan, "ssd_scan"),
                                 "ms_alone": alone[1]}},
        "two_kernel": {"ms_per_step": round(two_ms, 4), "tokens_per_s": round(tok / (two_ms * 1e-3), 1),
                       "path_roofline_frac": round((conv_b + scan_b) / (two_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "path_roofline_frac": round(tok / (step_ms * 1e-3) / roof_tok_s, 4),
        "fused_min_roofline_frac": round(fused_b / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "config": {"workload": "zamba2-2.7b mixer prefill, batch 1 x 32768 tokens (conv1d+SiLU and SSD scan in one "
                               "pass: m2_mixer_prefill_fwd)",
                   "batch": B, "seqlen": L, "d_model": d.d_model, "expand": d.expand, "nheads": H,
                   "headdim": P, "d_state": N, "n_groups": G, "d_conv": W,
                   "chunk_size": d.chunk_size or "library default", "state": "fp32, zero initial, final returned"},
    }


VARLEN_LENS = (8192, 6144, 5120, 4096, 3584, 2560, 2048, 1024)  # 32768 tokens in 8 prompts


def bench_varlen(torch, m2, workloads, args):
    """The same 32768 tokens as eight prompts of different lengths, packed back to back
    (m2_conv1d_fwd_packed then m2_ssd_scan_fwd_packed, each prompt from a zero state)."""
    d1 = workloads.CONFIGS[3].dims
    lens = VARLEN_LENS
    T = sum(lens)
    inp = workloads.generate(d1.replace(seqlen=T), 1003, False)   # one row of T tokens, cut into prompts
    Bn, H, P, N, G, W, Cd = len(lens), d1.nheads, d1.headdim, d1.d_state, d1.n_groups, d1.d_conv, d1.conv_dim
    dims = m2.make_dims(Bn, max(lens), d1.d_model, d1.expand, P, N, G, W, d1.chunk_size, d1.io)
    bf = torch.bfloat16
    cu = torch.as_tensor([0] + list(itertools.accumulate(lens)), dtype=torch.int32, device="cuda")
    xbc = torch.from_numpy(inp.xbc[0]).to("cuda", bf)
    dt = torch.from_numpy(inp.dt_raw[0]).to("cuda", bf)
    cw, cb, dtb, A, D = (torch.from_numpy(a).cuda() for a in (inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D))
    act = torch.empty((T, Cd), device="cuda", dtype=bf)
    ring_out = torch.empty((Bn, W, Cd), device="cuda", dtype=bf)
    y = torch.empty((T, H * P), device="cuda", dtype=bf)
    s_out = torch.empty((Bn, H, P, N), device="cuda")
    nws = m2.m2_ssd_scan_workspace_packed(dims, T)
    ws = torch.empty(max(nws, 1), device="cuda", dtype=torch.uint8) if nws else None
    del inp

    def conv():
        m2.m2_conv1d_fwd_packed(dims, cu, xbc, cw, cb, act, None, 0, ring_out)

    def scan():
        m2.m2_ssd_scan_fwd_packed(dims, cu, act[:, :H * P], act[:, H * P:H * P + G * N], act[:, H * P + G * N:], dt,
                                  dtb, A, D, y, None, s_out, workspace=ws)

    (t_conv, t_scan), total_ms, _ = time_events(torch, [conv, scan], args.steps, args.warmup)
    conv_b, scan_b = prefill_bytes(1, T, H, P, N, G, W, Cd, False, True)
    conv_b += (Bn - 1) * W * Cd * 2           # one ring per prompt
    scan_b += (Bn - 1) * H * P * N * 4        # one final state per prompt
    step_ms = total_ms / args.steps

    # the same prompts through the one-pass path (the conv output of x never written)
    nwf = m2.m2_mixer_prefill_workspace_packed(dims, T)
    wsf = torch.empty(max(nwf, 1), device="cuda", dtype=torch.uint8)
    y2, s_out2, ring2 = torch.empty_like(y), torch.empty_like(s_out), torch.empty_like(ring_out)

    def fused():
        m2.m2_mixer_prefill_fwd_packed(dims, cu, xbc, cw, cb, dt, dtb, A, D, y2, None, 0, ring2, None, s_out2,
                                       workspace=wsf)

    (t_fused,), fused_ms, _ = time_events(torch, [fused], args.steps, args.warmup)
    fused_b = fused_bytes(1, T, H, P, N, G, W, Cd, False, True) + (Bn - 1) * (W * Cd * 2 + H * P * N * 4)
    fused_step = fused_ms / args.steps
    return {"value": round(T / (step_ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(step_ms, 4),
            "one_pass": {"value": round(T / (fused_step * 1e-3), 1), "unit": "tokens/s",
                         "ms_per_step": round(fused_step, 4),
                         "roofline": roofline(fused_b, t_fused, "mixer_prefill_packed")},
            "kernels": {"conv1d_packed": {"us": round(t_conv * 1e3, 2),
                                          "roofline": roofline(conv_b, t_conv, "conv1d_packed")},
                        "ssd_scan_packed": {"us": round(t_scan * 1e3, 2),
                                            "roofline": roofline(scan_b, t_scan, "ssd_scan_packed")}},
            "config": {"workload": "zamba2-2.7b mixer prefill, 8 prompts packed back to back (cu_seqlens)",
                       "lengths": list(lens), "tokens": T, "state": "fp32, zero initial, final returned per prompt"}}


def bench_norm(torch, m2, workloads, args):
    """Gated group RMSNorm on the 32k prefill output (2.7B shape: 32768 rows of d_inner 5120, one group)."""
    T, D = 32768, 5120
    y, z, w = workloads.norm_inputs(T, D, 3200, "bf16")
    bf = torch.bfloat16
    yt, zt = torch.from_numpy(y).to("cuda", bf), torch.from_numpy(z).to("cuda", bf)
    wt = torch.from_numpy(w).cuda()
    ot = torch.empty_like(yt)
    del y, z

    def norm():
        m2.m2_gated_rmsnorm(yt, zt, wt, ot, D, eps=1e-5)

    (t,), _, _ = time_events(torch, [norm], args.steps, args.warmup)
    nbytes = 3 * T * D * 2 + D * 4
    return {"us": round(t * 1e3, 2), "bytes": nbytes, "roofline": roofline(nbytes, t, "gated_rmsnorm"),
            "config": {"workload": "gated group RMSNorm of the 32k prefill output (gate first)", "rows": T,
                       "d_inner": D, "group_size": D, "eps": 1e-5}}


def bench_decode(torch, m2, workloads, args):
    cfg = workloads.CONFIGS[4]
    d = cfg.dims
    steps = args.decode_steps
    inp = workloads.generate(d, 1004, True, steps)
    B, H, P, N, G, W, Cd = d.batch, d.nheads, d.headdim, d.d_state, d.n_groups, d.d_conv, d.conv_dim
    dims = m2.make_dims(B, 1, d.d_model, d.expand, P, N, G, W, 0, d.io)
    bf = torch.bfloat16
    xt = torch.from_numpy(inp.xbc).to("cuda", bf)
    dtt = torch.from_numpy(inp.dt_raw).to("cuda", bf)
    cw, cb, dtb, A, D = (torch.from_numpy(a).cuda() for a in (inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D))
    ring = torch.from_numpy(inp.ring0).to("cuda", bf)
    state = torch.from_numpy(inp.state0).cuda()
    y = torch.empty((B, H * P), device="cuda", dtype=bf)
    del inp
    counter = [0]

    def step():
        t = counter[0] % steps
        m2.m2_ssd_step(dims, xt[t], dtt[t], cw, cb, dtb, A, D, ring, counter[0], state, y)
        counter[0] += 1

    warm = min(args.warmup, steps)
    (t_step,), total_ms, wall_ms = time_events(torch, [step], steps, warm)
    sb = step_bytes(B, H, P, N, G, W, Cd)
    step_ms = total_ms / steps
    return {
        "tokens_per_s": B / (step_ms * 1e-3), "ms_per_step": step_ms, "kernel_ms": t_step, "wall_ms": wall_ms,
        "steps": steps, "roofline": roofline(sb, t_step, "ssd_step"), "bytes_per_launch": sb,
        "config": {"workload": "zamba2-2.7b mixer decode, 256 sequences x %d chained tokens" % steps,
                   "batch": B, "nheads": H, "headdim": P, "d_state": N, "d_conv": W,
                   "state": "fp32 80x64x64 per sequence, N(0,0.1)", "ring": "bf16 4 x 5248, N(0,0.1)"},
    }


def bench_backward(torch, m2, workloads, args):
    """The scan's backward (m2_ssd_scan_bwd) on the 32k prompt at the 2.7B mixer shape: the gradients of
    a prefill's output and final state for all of its inputs (training path)."""
    cfg = workloads.CONFIGS[3]
    d = cfg.dims
    inp = workloads.config_inputs(3)
    B, L, H, P, N, G = d.batch, d.seqlen, d.nheads, d.headdim, d.d_state, d.n_groups
    dims = m2.make_dims(B, L, d.d_model, d.expand, P, N, G, d.d_conv, d.chunk_size, d.io)
    bf = torch.bfloat16
    dy_np, ds_np = workloads.grad_inputs(d, 1005)
    act = torch.from_numpy(inp.xbc).to("cuda", bf)
    dt = torch.from_numpy(inp.dt_raw).to("cuda", bf)
    dtb, A, D = (torch.from_numpy(a).cuda() for a in (inp.dt_bias, inp.A, inp.D))
    dy = torch.from_numpy(dy_np.reshape(B, L, H * P)).to("cuda", bf)
    ds = torch.from_numpy(ds_np).cuda()
    del inp, dy_np, ds_np
    xv, bv, cv = act[:, :, :H * P], act[:, :, H * P:H * P + G * N], act[:, :, H * P + G * N:]
    dx = torch.empty((B, L, H * P), device="cuda", dtype=bf)
    dBt = torch.empty((B, L, G * N), device="cuda", dtype=bf)
    dCt = torch.empty((B, L, G * N), device="cuda", dtype=bf)
    ddt = torch.empty((B, L, H), device="cuda", dtype=bf)
    dtb_g, dA, dD = (torch.empty(H, device="cuda") for _ in range(3))
    dsi = torch.empty((B, H, P, N), device="cuda")
    ws = torch.empty(m2.m2_ssd_scan_bwd_workspace(dims), device="cuda", dtype=torch.uint8)

    def bwd():
        m2.m2_ssd_scan_bwd(dims, xv, bv, cv, dt, dtb, A, D, dy, dx, dBt, dCt, ddt, dtb_g,
                           dA, dD, dstate_out=ds, dstate_in=dsi, workspace=ws)

    (t,), _, _ = time_events(torch, [bwd], args.steps, args.warmup)
    nb = bwd_bytes(B, L, H, P, N, G, False, True, True)
    fl = bwd_flops(B, L, H)
    r = roofline(nb, t, "ssd_scan_bwd")
    return {"value": round(B * L / (t * 1e-3), 1), "unit": "tokens/s", "us": round(t * 1e3, 2), "bytes": nb,
            "roofline": dict(r, kernel="ssd_scan_bwd"),
            "mfma": {"flops": fl, "achieved_TFLOPs": round(fl / (t * 1e-3) / 1e12, 1),
                     "peak_TFLOPs": 2500.0, "frac": round(fl / (t * 1e-3) / 2.5e15, 4)},
            "workspace_bytes": ws.numel(),
            "config": {"workload": "zamba2-2.7b scan backward, batch 1 x 32768 tokens (gradients of y and the final "
                                   "state for x, B, C, dt, dt_bias, A, D and the initial state)",
                       "batch": B, "seqlen": L, "nheads": H, "headdim": P, "d_state": N, "n_groups": G,
                       "chunk": 64}}


def copy_ceiling(torch, m2, mib=1024, reps=10):
    """GB/s (read + write bytes) of the library's streaming copy kernel over `mib` MiB: the attainable
    bandwidth reference beside the 8 TB/s vendor peak."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    m2.m2_stream_copy(dst, src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        m2.m2_stream_copy(dst, src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return round(2 * n / (ms * 1e-3) / 1e9, 1)


def cpu_baseline(workloads, seconds_target):
    """The fp64 oracle, untuned, on the same 32k prefill (conv1d+SiLU then the scan, all 80 heads), on
    the host cores.  Token prefixes double until one takes a quarter of `seconds_target` or the whole
    prompt is covered; the whole prompt is then repeated until `seconds_target` has passed."""
    cores = len(os.sched_getaffinity(0))
    os.environ["OMP_NUM_THREADS"] = str(cores)
    import oracle
    d = workloads.CONFIGS[3].dims
    H, P, N, G, L = d.nheads, d.headdim, d.d_state, d.n_groups, d.seqlen
    inp = workloads.config_inputs(3)

    def run(T):
        t0 = time.perf_counter()
        oracle.mixer_prefill(inp.xbc[:, :T], inp.dt_raw[:, :T], inp.conv_w, inp.conv_b, inp.dt_bias, inp.A,
                             inp.D, H, P, N, G)
        return time.perf_counter() - t0

    T = 512
    while True:
        dt = run(T)
        if dt >= seconds_target / 4 or T >= L:
            break
        T = min(2 * T, L)
    tokens, secs, reps = T, dt, 1
    if T >= L:
        while secs < seconds_target:
            secs += run(L)
            tokens += L
            reps += 1
    what = ("the whole prompt, %d run(s)" % reps) if T >= L else ("the first %d tokens" % T)
    return {"value": round(tokens / secs, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "batch-1 32768-token prefill at the Zamba2-2.7B mixer shape (conv1d+SiLU then scan, 80 "
                      "heads, fp64): %s, %.2f s" % (what, secs)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import selective_state_space_mixer_amd as m2
    import workloads
    if args.copy_probe_mib:
        # a plain copy of known size (the library's streaming copy), for scaling the FETCH_SIZE /
        # WRITE_SIZE counters
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            m2.m2_stream_copy(dst, src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}))
        return
    COPY_CEILING[0] = copy_ceiling(torch, m2)

    out = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": None}
    pre = dec = None
    if args.only in ("all", "prefill"):
        pre = bench_prefill(torch, m2, workloads, args)
        print("prefill: one pass %.3f ms/step, %.3e tok/s | conv %.1f us + scan %.1f us = %.3f ms/step" % (
            pre["ms_per_step"], pre["tokens_per_s"], pre["kernels"]["conv1d"]["ms"] * 1e3,
            pre["kernels"]["ssd_scan"]["ms"] * 1e3, pre["two_kernel"]["ms_per_step"]), file=sys.stderr, flush=True)
        out["value"] = round(pre["tokens_per_s"], 1)
        out["ms_per_step"] = round(pre["ms_per_step"], 4)
        out["config"] = pre["config"]
        k = pre["kernels"]
        # the headline step is the one-pass entry point: its roofline is the line's roofline
        out["roofline"] = dict(k["mixer_prefill"]["roofline"], kernel="mixer_prefill")
        out["prefill_kernels"] = {n: {"us": round(v["ms"] * 1e3, 2), "bytes": v["bytes"],
                                      "frac": v["roofline"]["frac"], "achieved_GBs": v["roofline"]["achieved"],
                                      "frac_of_copy": v["roofline"].get("frac_of_copy")}
                                  for n, v in k.items()}
        for n, v in k.items():
            if "ms_alone" in v:
                out["prefill_kernels"][n]["us_alone"] = round(v["ms_alone"] * 1e3, 2)
        for n in ("mixer_prefill", "ssd_scan"):
            out["prefill_kernels"][n]["mfma"] = measured_mfma(n)
        out["prefill_path_roofline_frac"] = pre["path_roofline_frac"]
        out["prefill_fused_min_roofline_frac"] = pre["fused_min_roofline_frac"]
        out["prefill_two_kernel"] = pre["two_kernel"]
    if args.only in ("all", "prefill"):
        vl = bench_varlen(torch, m2, workloads, args)
        print("packed prompts: %.3f ms/step, %.3e tok/s (one pass: %.3f ms/step)" % (
            vl["ms_per_step"], vl["value"], vl["one_pass"]["ms_per_step"]), file=sys.stderr,
              flush=True)
        out["varlen"] = vl
        nrm = bench_norm(torch, m2, workloads, args)
        print("gated rmsnorm: %.1f us (%.0f GB/s)" % (nrm["us"], nrm["roofline"]["achieved"]), file=sys.stderr,
              flush=True)
        out["epilogue"] = {"gated_rmsnorm": nrm}
    if args.only in ("all", "decode"):
        dec = bench_decode(torch, m2, workloads, args)
        print("decode: %.1f us/step, %.3e tok/s" % (dec["ms_per_step"] * 1e3, dec["tokens_per_s"]),
              file=sys.stderr, flush=True)
        out["decode"] = {"value": round(dec["tokens_per_s"], 1), "unit": "tokens/s",
                         "us_per_step": round(dec["ms_per_step"] * 1e3, 2), "kernel_us": round(dec["kernel_ms"] * 1e3, 2),
                         "steps": dec["steps"], "roofline": dict(dec["roofline"], kernel="ssd_step"),
                         "config": dec["config"]}
        if pre is None:
            out["value"] = round(dec["tokens_per_s"], 1)
            out["ms_per_step"] = round(dec["ms_per_step"], 4)
            out["config"] = dec["config"]
            out["roofline"] = out["decode"]["roofline"]
    if args.only in ("all", "backward"):
        bw = bench_backward(torch, m2, workloads, args)
        print("scan backward: %.1f us, %.3e tok/s (%.0f GB/s algorithmic, %.0f MFMA TFLOP/s)" % (
            bw["us"], bw["value"], bw["roofline"]["achieved"], bw["mfma"]["achieved_TFLOPs"]), file=sys.stderr,
            flush=True)
        out["backward"] = bw
        if pre is None and dec is None:
            out["value"] = bw["value"]
            out["ms_per_step"] = round(bw["us"] / 1e3, 4)
            out["config"] = bw["config"]
            out["roofline"] = bw["roofline"]
    out["copy_ceiling_GBs"] = COPY_CEILING[0]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(workloads, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
