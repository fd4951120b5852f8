"""More GPU parity against the fp64 oracle, each case printing its achieved error:

- a dt clamp (dt_min / dt_max set so both bounds bind) in the scan (a plan of several segments, on the
  walk kernel and on the general kernel), the packed scan, the decode step and the one-pass prefill;
- the 256-sequence decode workload over all of its 128 chained steps;
- a 32768-step decode chain on the 32k prompt, against the prefill's final state, ring and outputs
  (the Zamba2 article §七: the token-by-token path must agree with the chunked prefill);
- a bf16 decode step at headdim 64 / d_state 128 (the 130m-like shape);
- every channel of the full-size conv (32k prompt and the 8 x 4096 batch with history).
- plans of more segments than the segment chain loads at once (down to one chunk per segment).
Floored max-relative-error bar 2e-2 for bf16 activations with fp32 state; conv rings bit-exact."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import selective_state_space_mixer_amd as m2
    from gpu_util import dev, dev32, dims_of, host, nan_like, workspace

TOL = 2e-2
DT_MIN, DT_MAX = 0.03, 0.12


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")


def _softplus(v):
    return np.logaddexp(0.0, v)


def _clamp_hits(dt_raw, dt_bias):
    """How many dt values fall below DT_MIN and above DT_MAX (each bound must bind in these tests)."""
    dt = _softplus(np.asarray(dt_raw, np.float64) + np.asarray(dt_bias, np.float64))
    return int((dt < DT_MIN).sum()), int((dt > DT_MAX).sum())


def _split(d, inp):
    x, b, c = inp.split()
    lead = (d.batch, d.seqlen)
    return (x.reshape(lead + (d.nheads, d.headdim)), b.reshape(lead + (d.n_groups, d.d_state)),
            c.reshape(lead + (d.n_groups, d.d_state)))


@pytest.mark.parametrize("idx,over", [(3, dict(seqlen=8192)), (1, dict(batch=2, seqlen=2048))],
                         ids=["2.7b-walk-kernel", "130m-general-kernel"])
def test_dt_clamp_scan(idx, over):
    _need_gpu()
    d = workloads.CONFIGS[idx].dims.replace(**over)
    inp = workloads.generate(d, 6100 + idx, True)
    lo, hi = _clamp_hits(inp.dt_raw, inp.dt_bias)
    assert lo > 0 and hi > 0
    x, b, c = _split(d, inp)
    dims = dims_of(d)
    assert m2.m2_ssd_scan_workspace(dims) > 0, "expected a plan of several segments"
    y = nan_like((d.batch, d.seqlen, d.d_inner), "bf16")
    s = torch.full((d.batch, d.nheads, d.headdim, d.d_state), float("nan"), device="cuda")
    m2.m2_ssd_scan_fwd(dims, dev(x, "bf16"), dev(b, "bf16"), dev(c, "bf16"), dev(inp.dt_raw, "bf16"),
                       dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y, dev32(inp.state0), s, dt_min=DT_MIN,
                       dt_max=DT_MAX, workspace=workspace(dims))
    torch.cuda.synchronize()
    yr, sr = oracle.ssd_scan(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0, DT_MIN, DT_MAX)
    ey = oracle.max_rel_err(host(y).reshape(yr.shape), yr)
    es = oracle.max_rel_err(host(s), sr)
    # the clamp matters: without it the oracle's result is far from the clamped one
    y_free, _ = oracle.ssd_scan(x[:, :256], b[:, :256], c[:, :256], inp.dt_raw[:, :256], inp.dt_bias, inp.A, inp.D,
                                inp.state0)
    print("clamped scan %s (%d below, %d above): y %.2e state %.2e" % (over, lo, hi, ey, es))
    assert oracle.max_rel_err(y_free, yr[:, :256]) > 10 * TOL
    assert ey <= TOL and es <= TOL


def test_dt_clamp_packed_scan():
    _need_gpu()
    lens = [300, 1000, 37, 0, 2100]
    d1 = workloads.CONFIGS[2].dims
    T = sum(lens)
    inp = workloads.generate(d1.replace(batch=1, seqlen=T), 6200, False)
    H, P, N, G = d1.nheads, d1.headdim, d1.d_state, d1.n_groups
    x, b, c = inp.split()
    x, b, c = x[0].reshape(T, H, P), b[0].reshape(T, G, N), c[0].reshape(T, G, N)
    dt = inp.dt_raw[0]
    d = d1.replace(batch=len(lens), seqlen=max(lens))
    dims = dims_of(d)
    cu_np = np.concatenate([[0], np.cumsum(lens)])
    cu = torch.as_tensor(cu_np.astype(np.int32), device="cuda")
    y = nan_like((T, H * P), "bf16")
    s = torch.full((len(lens), H, P, N), float("nan"), device="cuda")
    m2.m2_ssd_scan_fwd_packed(dims, cu, dev(x, "bf16"), dev(b, "bf16"), dev(c, "bf16"), dev(dt, "bf16"),
                              dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y, None, s, dt_min=DT_MIN,
                              dt_max=DT_MAX, workspace=workspace(dims, T))
    torch.cuda.synchronize()
    yr, sr = oracle.ssd_scan_packed(x, b, c, dt, cu_np, inp.dt_bias, inp.A, inp.D, None, DT_MIN, DT_MAX)
    ey, es = oracle.max_rel_err(host(y).reshape(T, H, P), yr), oracle.max_rel_err(host(s), sr)
    print("clamped packed scan: y %.2e state %.2e" % (ey, es))
    assert ey <= TOL and es <= TOL


def test_dt_clamp_step():
    _need_gpu()
    d = workloads.CONFIGS[4].dims.replace(batch=4)
    steps = 6
    inp = workloads.generate(d, 6300, True, steps)
    lo, hi = _clamp_hits(inp.dt_raw, inp.dt_bias)
    assert lo > 0 and hi > 0
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    dims = dims_of(d)
    ring, state = dev(inp.ring0, "bf16"), dev32(inp.state0)
    w, cb, dtb, A, D = (dev32(a) for a in (inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D))
    r_ring, r_state = inp.ring0.astype(np.float64), inp.state0.astype(np.float64)
    worst = 0.0
    for t in range(steps):
        y = nan_like((d.batch, H * P), "bf16")
        m2.m2_ssd_step(dims, dev(inp.xbc[t], "bf16"), dev(inp.dt_raw[t], "bf16"), w, cb, dtb, A, D, ring, t, state, y,
                       dt_min=DT_MIN, dt_max=DT_MAX)
        yr, r_ring, r_state = oracle.ssd_step(inp.xbc[t], inp.dt_raw[t], inp.conv_w, inp.conv_b, inp.dt_bias, inp.A,
                                              inp.D, r_ring, t, r_state, H, P, N, G, DT_MIN, DT_MAX)
        torch.cuda.synchronize()
        worst = max(worst, oracle.max_rel_err(host(y), yr))
    es = oracle.max_rel_err(host(state), r_state)
    print("clamped decode steps: y %.2e state %.2e" % (worst, es))
    assert worst <= TOL and es <= TOL
    np.testing.assert_array_equal(host(ring), r_ring)


def test_dt_clamp_fused_prefill():
    _need_gpu()
    d = workloads.CONFIGS[2].dims.replace(batch=2, seqlen=1500)
    inp = workloads.generate(d, 6400, True)
    H, P, N, G, W, Cd = d.nheads, d.headdim, d.d_state, d.n_groups, d.d_conv, d.conv_dim
    dims = dims_of(d)
    y = nan_like((d.batch, d.seqlen, H * P), "bf16")
    s = torch.full((d.batch, H, P, N), float("nan"), device="cuda")
    ring = nan_like((d.batch, W, Cd), "bf16")
    ws = torch.empty(m2.m2_mixer_prefill_workspace(dims), device="cuda", dtype=torch.uint8)
    m2.m2_mixer_prefill_fwd(dims, dev(inp.xbc, "bf16"), dev32(inp.conv_w), dev32(inp.conv_b), dev(inp.dt_raw, "bf16"),
                            dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y, dev(inp.ring0, "bf16"), 0, ring,
                            dev32(inp.state0), s, dt_min=DT_MIN, dt_max=DT_MAX, workspace=ws)
    torch.cuda.synchronize()
    act, ringr = oracle.conv1d(inp.xbc, inp.conv_w, inp.conv_b, inp.ring0, 0)
    x, b, c = oracle.split_act(act, H, P, N, G)
    yr, sr = oracle.ssd_scan(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0, DT_MIN, DT_MAX)
    ey, es = oracle.max_rel_err(host(y).reshape(yr.shape), yr), oracle.max_rel_err(host(s), sr)
    print("clamped one-pass prefill: y %.2e state %.2e" % (ey, es))
    assert ey <= TOL and es <= TOL
    np.testing.assert_array_equal(host(ring), ringr)


def test_full_size_decode_b256_all_128_steps():
    """The decode workload as specified: 256 sequences, 128 chained steps; three sampled sequences
    against the oracle chain at every step."""
    _need_gpu()
    cfg = workloads.CONFIGS[4]
    d = cfg.dims
    steps = cfg.decode_steps
    inp = workloads.generate(d, 1004, True, steps)
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    dims = dims_of(d)
    ring, state = dev(inp.ring0, "bf16"), dev32(inp.state0)
    xt, dtt = dev(inp.xbc, "bf16"), dev(inp.dt_raw, "bf16")
    w, cb, dtb, A, D = (dev32(a) for a in (inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D))
    ys = torch.empty((steps, d.batch, H * P), device="cuda", dtype=torch.bfloat16)
    for t in range(steps):
        m2.m2_ssd_step(dims, xt[t], dtt[t], w, cb, dtb, A, D, ring, t, state, ys[t])
    torch.cuda.synchronize()
    ys_h, state_h, ring_h = host(ys), host(state), host(ring)
    worst_y = worst_s = 0.0
    for b in (0, 131, 255):
        r_ring = inp.ring0[b:b + 1].astype(np.float64)
        r_state = inp.state0[b:b + 1].astype(np.float64)
        for t in range(steps):
            yr, r_ring, r_state = oracle.ssd_step(inp.xbc[t, b:b + 1], inp.dt_raw[t, b:b + 1], inp.conv_w, inp.conv_b,
                                                  inp.dt_bias, inp.A, inp.D, r_ring, t, r_state, H, P, N, G)
            worst_y = max(worst_y, oracle.max_rel_err(ys_h[t, b:b + 1], yr))
        worst_s = max(worst_s, oracle.max_rel_err(state_h[b:b + 1], r_state))
        np.testing.assert_array_equal(ring_h[b:b + 1], r_ring)
    print("decode 256 x 128 steps (sampled sequences): y %.2e state %.2e" % (worst_y, worst_s))
    assert worst_y <= TOL and worst_s <= TOL


def test_decode_chain_of_32768_steps_equals_prefill():
    """The 32k prompt run token by token through m2_ssd_step (from a zero state and an empty conv
    history, as the prefill starts) against m2_ssd_scan_fwd's final state, the conv ring and sampled
    outputs, and against the oracle's final state."""
    _need_gpu()
    idx = 3
    d = workloads.CONFIGS[idx].dims
    inp = workloads.config_inputs(idx)
    Bn, L, H, P, N, G, W, Cd = d.batch, d.seqlen, d.nheads, d.headdim, d.d_state, d.n_groups, d.d_conv, d.conv_dim
    dims = dims_of(d)
    xbc, dt = dev(inp.xbc, "bf16"), dev(inp.dt_raw, "bf16")
    w, cb, dtb, A, D = (dev32(a) for a in (inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D))
    # prefill: conv -> scan
    act = torch.empty((Bn, L, Cd), device="cuda", dtype=torch.bfloat16)
    ring_p = torch.empty((Bn, W, Cd), device="cuda", dtype=torch.bfloat16)
    m2.m2_conv1d_fwd(dims, xbc, w, cb, act, None, 0, ring_p)
    y_p = torch.empty((Bn, L, H * P), device="cuda", dtype=torch.bfloat16)
    s_p = torch.empty((Bn, H, P, N), device="cuda")
    m2.m2_ssd_scan_fwd(dims, act[:, :, :H * P], act[:, :, H * P:H * P + G * N], act[:, :, H * P + G * N:], dt, dtb, A,
                       D, y_p, None, s_p, workspace=workspace(dims))
    del act
    # decode chain over the same tokens
    dims1 = dims_of(d.replace(seqlen=1))
    ring = torch.zeros((Bn, W, Cd), device="cuda", dtype=torch.bfloat16)
    state = torch.zeros((Bn, H, P, N), device="cuda")
    y_d = torch.empty((L, Bn, H * P), device="cuda", dtype=torch.bfloat16)
    for t in range(L):
        m2.m2_ssd_step(dims1, xbc[:, t], dt[:, t], w, cb, dtb, A, D, ring, t, state, y_d[t])
    torch.cuda.synchronize()
    es = oracle.max_rel_err(host(state), host(s_p))
    rows = np.arange(0, L, 997)
    ey = oracle.max_rel_err(host(y_d[rows, 0]), host(y_p[0, rows]))
    # the chain's ring (phase L mod W) holds the same tokens as the prefill's ring (phase 0)
    rd, rp = host(ring), host(ring_p)
    for j in range(1, W + 1):
        np.testing.assert_array_equal(rd[:, (L - j) % W], rp[:, W - j])
    _, sr, _, _ = oracle.mixer_prefill(inp.xbc, inp.dt_raw, inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D,
                                       H, P, N, G)
    eo = oracle.max_rel_err(host(state), sr)
    print("32768-step decode chain vs prefill: state %.2e, sampled y %.2e; chain state vs oracle %.2e" % (es, ey, eo))
    assert es <= TOL and ey <= TOL and eo <= TOL


def test_step_bf16_p64_n128():
    """A bf16 decode chain at headdim 64, d_state 128 (the 130m-like shape)."""
    _need_gpu()
    d = workloads.CONFIGS[1].dims.replace(batch=4, seqlen=1)
    steps = 8
    inp = workloads.generate(d, 6500, True, steps)
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    dims = dims_of(d)
    ring, state = dev(inp.ring0, "bf16"), dev32(inp.state0)
    w, cb, dtb, A, D = (dev32(a) for a in (inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D))
    r_ring, r_state = inp.ring0.astype(np.float64), inp.state0.astype(np.float64)
    worst = 0.0
    for t in range(steps):
        y = nan_like((d.batch, H * P), "bf16")
        m2.m2_ssd_step(dims, dev(inp.xbc[t], "bf16"), dev(inp.dt_raw[t], "bf16"), w, cb, dtb, A, D, ring, t, state, y)
        yr, r_ring, r_state = oracle.ssd_step(inp.xbc[t], inp.dt_raw[t], inp.conv_w, inp.conv_b, inp.dt_bias, inp.A,
                                              inp.D, r_ring, t, r_state, H, P, N, G)
        torch.cuda.synchronize()
        worst = max(worst, oracle.max_rel_err(host(y), yr))
    es = oracle.max_rel_err(host(state), r_state)
    print("bf16 step P64 N128: y %.2e state %.2e" % (worst, es))
    assert worst <= TOL and es <= TOL
    np.testing.assert_array_equal(host(ring), r_ring)


@pytest.mark.parametrize("idx", [3, 2])
def test_full_size_conv_every_channel(idx):
    _need_gpu()
    cfg = workloads.CONFIGS[idx]
    d = cfg.dims
    inp = workloads.config_inputs(idx)
    Bn, L, W, Cd = d.batch, d.seqlen, d.d_conv, d.conv_dim
    dims = dims_of(d)
    act = nan_like((Bn, L, Cd), "bf16")
    ring = nan_like((Bn, W, Cd), "bf16")
    m2.m2_conv1d_fwd(dims, dev(inp.xbc, "bf16"), dev32(inp.conv_w), dev32(inp.conv_b), act, dev(inp.ring0, "bf16"), 0,
                     ring)
    torch.cuda.synchronize()
    ref, ref_ring = oracle.conv1d(inp.xbc, inp.conv_w, inp.conv_b, inp.ring0, 0)
    e = oracle.max_rel_err(host(act), ref)
    print("full-size conv %d, all %d channels: %.2e" % (idx, Cd, e))
    assert e <= TOL
    np.testing.assert_array_equal(host(ring), ref_ring)


def _per_token_err(got, ref):
    """Worst token of a [B, L, H, P] output: each token's error floored by that token's own rms."""
    g = got.reshape(got.shape[0], got.shape[1], -1)
    o = ref.reshape(ref.shape[0], ref.shape[1], -1)
    rms = np.sqrt((o ** 2).mean(axis=2, keepdims=True))
    return float((np.abs(g - o) / np.maximum(np.abs(o), rms)).max())


@pytest.mark.parametrize("idx,over,scale", [(3, dict(seqlen=8192), 1e3), (3, dict(seqlen=8192), 1e6),
                                            (1, dict(batch=2, seqlen=4096), 1e4)],
                         ids=["2.7b-x1e3", "2.7b-x1e6", "130m-x1e4"])
def test_large_initial_state_across_segments_per_token(idx, over, scale):
    """An initial state far above the state the inputs drive, on a plan of many segments.  Every later
    segment ran from zero and gets its true initial state's share back from the fix-up for as long as
    that share matters against the segment's own state; the outputs of the later segments must agree
    token by token (each token floored by its own rms).  The first segment starts from the caller's
    state inside the main pass, where a state that dominates the outputs enters as a bf16 operand
    (a per-token error of a few 1e-2 at x1e3, not governed by the fix-up); its tokens are not part of
    this check.  The final state is checked as everywhere."""
    _need_gpu()
    d = workloads.CONFIGS[idx].dims.replace(**over)
    inp = workloads.generate(d, 6700 + idx, True)
    s0 = (inp.state0 * np.float32(scale)).astype(np.float32)
    x, b, c = _split(d, inp)
    dims = dims_of(d)
    assert m2.m2_ssd_scan_workspace(dims) > 0, "expected a plan of several segments"
    y = nan_like((d.batch, d.seqlen, d.d_inner), "bf16")
    s = torch.full((d.batch, d.nheads, d.headdim, d.d_state), float("nan"), device="cuda")
    m2.m2_ssd_scan_fwd(dims, dev(x, "bf16"), dev(b, "bf16"), dev(c, "bf16"), dev(inp.dt_raw, "bf16"),
                       dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y, dev32(s0), s, workspace=workspace(dims))
    torch.cuda.synchronize()
    yr, sr = oracle.ssd_scan(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, s0)
    yg = host(y).reshape(yr.shape)
    # the library's plan: one round of resident blocks, about 512 / (batch x head groups) segments of
    # whole 32-token chunks; the first segment ends before token `first`
    nchunks = (d.seqlen + 31) // 32
    nseg = max(1, min(nchunks, 512 // (d.batch * (d.nheads // (4 if idx == 3 else 2)))))
    first = ((nchunks + nseg - 1) // nseg) * 32
    et = _per_token_err(yg[:, first:], yr[:, first:])
    es = oracle.max_rel_err(host(s), sr)
    print("initial state x%.0e: worst token after the first segment (from token %d) %.2e, state %.2e"
          % (scale, first, et, es))
    assert et <= TOL and es <= TOL


@pytest.mark.parametrize("idx,over", [(0, dict(seqlen=1000)), (3, dict(d_model=128, seqlen=1300))],
                         ids=["tiny-f32-63-segments", "2.7b-4-heads-bf16-41-segments"])
def test_scan_plan_of_more_segments_than_one_load_batch(idx, over):
    """Few heads and a long prompt: the plan cuts the sequence into more segments than the chain kernel
    loads at once (32), down to one chunk per segment, so the chain runs over several load batches and
    nearly every chunk is a segment's first.  Checked against the oracle with a random initial state."""
    _need_gpu()
    d = workloads.CONFIGS[idx].dims.replace(**over)
    inp = workloads.generate(d, 6900 + idx, True)
    x, b, c = _split(d, inp)
    dims = dims_of(d)
    # the workspace holds one fp32 state per (segment, sequence, head): more than 32 segments
    per_seg = d.batch * d.nheads * d.headdim * d.d_state * 4
    assert m2.m2_ssd_scan_workspace(dims) > 33 * per_seg, "expected a plan of more than 32 segments"
    y = nan_like((d.batch, d.seqlen, d.d_inner), d.io)
    s = torch.full((d.batch, d.nheads, d.headdim, d.d_state), float("nan"), device="cuda")
    m2.m2_ssd_scan_fwd(dims, dev(x, d.io), dev(b, d.io), dev(c, d.io), dev(inp.dt_raw, d.io), dev32(inp.dt_bias),
                       dev32(inp.A), dev32(inp.D), y, dev32(inp.state0), s, workspace=workspace(dims))
    torch.cuda.synchronize()
    yr, sr = oracle.ssd_scan(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0)
    ey = oracle.max_rel_err(host(y).reshape(yr.shape), yr)
    es = oracle.max_rel_err(host(s), sr)
    tol = 1e-4 if d.io == "f32" else TOL
    print("plan of many segments (%s): y %.2e state %.2e (bar %.0e)" % (d.io, ey, es, tol))
    assert ey <= tol and es <= tol
