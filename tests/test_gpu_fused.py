"""GPU parity of the one-pass prompt path (m2_mixer_prefill_fwd: conv1d + SiLU and the scan without
writing the conv output) against the fp64 oracle's conv -> scan, and against the two entry points.

Floating outputs within the floored max-relative-error bar of bf16 activations with fp32 state (2e-2);
the conv ring is a copy of inputs and must be bit-identical."""
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


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")


def _fused(d, inp, ring_in=None, phase=0, state_in=None, bias=True, lens=None):
    Bn, L, H, P, N, W, Cd = d.batch, d.seqlen, d.nheads, d.headdim, d.d_state, d.d_conv, d.conv_dim
    dims = dims_of(d)
    y = nan_like((Bn, L, H * P), "bf16")
    s_out = torch.full((Bn, H, P, N), float("nan"), device="cuda")
    ring_out = nan_like((Bn, W, Cd), "bf16")
    n = m2.m2_mixer_prefill_workspace(dims)
    ws = torch.empty(max(n, 1), device="cuda", dtype=torch.uint8)
    lens_d = None if lens is None else torch.as_tensor(np.asarray(lens, np.int32), device="cuda")
    m2.m2_mixer_prefill_fwd(dims, dev(inp.xbc, "bf16"), dev32(inp.conv_w), dev32(inp.conv_b) if bias else None,
                            dev(inp.dt_raw, "bf16"), dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y,
                            dev(ring_in, "bf16"), phase, ring_out, dev32(state_in), s_out, workspace=ws,
                            seq_lens=lens_d)
    torch.cuda.synchronize()
    return host(y).reshape(Bn, L, H, P), host(s_out), host(ring_out)


def _two_kernels(d, inp, ring_in=None, phase=0, state_in=None, bias=True):
    Bn, L, H, P, N, G, W, Cd = d.batch, d.seqlen, d.nheads, d.headdim, d.d_state, d.n_groups, d.d_conv, d.conv_dim
    dims = dims_of(d)
    act = torch.empty((Bn, L, Cd), device="cuda", dtype=torch.bfloat16)
    ring_out = torch.empty((Bn, W, Cd), device="cuda", dtype=torch.bfloat16)
    m2.m2_conv1d_fwd(dims, dev(inp.xbc, "bf16"), dev32(inp.conv_w), dev32(inp.conv_b) if bias else None, act,
                     dev(ring_in, "bf16"), phase, ring_out)
    y = torch.empty((Bn, L, H * P), device="cuda", dtype=torch.bfloat16)
    s_out = torch.empty((Bn, H, P, N), device="cuda")
    m2.m2_ssd_scan_fwd(dims, act[:, :, :H * P], act[:, :, H * P:H * P + G * N], act[:, :, H * P + G * N:],
                       dev(inp.dt_raw, "bf16"), dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y, dev32(state_in),
                       s_out, workspace=workspace(dims))
    torch.cuda.synchronize()
    return host(y).reshape(Bn, L, H, P), host(s_out), host(ring_out)


FUSED_CASES = [
    # (dims overrides of the 2.7B prefill workload, cached state and history, ring phase, bias)
    (dict(batch=2, seqlen=300), True, 0, True),
    (dict(batch=1, seqlen=1000), False, 0, True),         # one sequence: a plan of many short segments
    (dict(batch=2, seqlen=300), True, 2, True),            # history at another ring phase
    (dict(batch=3, seqlen=37), True, 1, False),            # one chunk and a ragged one, no conv bias
    (dict(batch=2, seqlen=5), True, 0, True),              # shorter than a chunk
    (dict(batch=2, seqlen=2), True, 3, True),              # shorter than the conv window
    (dict(batch=2, seqlen=130, d_conv=3), True, 1, True),  # conv width 3
    (dict(batch=2, seqlen=130, d_conv=2), True, 0, True),  # conv width 2
    (dict(batch=2, seqlen=200, n_groups=2), True, 0, True),
    (dict(batch=1, seqlen=700, n_groups=4), False, 0, True),
    # four heads and 41 chunks: 41 one-chunk segments, every block a segment start taking its conv
    # window from memory, and a segment chain longer than one load batch
    (dict(batch=1, seqlen=1300, d_model=128), True, 1, True),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "%s-cache%d-ph%d-bias%d" % c)
def test_fused_prefill_parity(case):
    _need_gpu()
    over, cached, phase, bias = case
    d = workloads.CONFIGS[2].dims.replace(**over)
    inp = workloads.generate(d, 5100 + d.seqlen + d.d_conv, cached)
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    ring_in = inp.ring0 if cached else None
    s_in = inp.state0 if cached else None
    y, s, ring = _fused(d, inp, ring_in, phase, s_in, bias)
    yr, sr, ringr, _ = oracle.mixer_prefill(inp.xbc, inp.dt_raw, inp.conv_w, inp.conv_b if bias else None, inp.dt_bias,
                                            inp.A, inp.D, H, P, N, G, ring_in, phase, s_in)
    ey, es = oracle.max_rel_err(y, yr), oracle.max_rel_err(s, sr)
    print("fused %s: y %.2e state %.2e" % (over, ey, es))
    assert ey <= TOL and es <= TOL
    np.testing.assert_array_equal(ring, ringr)


def test_fused_prefill_empty_prompt():
    """seqlen 0: the state passes through and the ring is a copy of the history."""
    _need_gpu()
    d = workloads.CONFIGS[2].dims.replace(batch=2, seqlen=0)
    inp = workloads.generate(d.replace(seqlen=1), 5300, True)
    inp.xbc, inp.dt_raw = inp.xbc[:, :0], inp.dt_raw[:, :0]
    _, s, ring = _fused(d, inp, inp.ring0, 1, inp.state0)
    _, _, ringr, _ = oracle.mixer_prefill(inp.xbc, inp.dt_raw, inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D,
                                          d.nheads, d.headdim, d.d_state, d.n_groups, inp.ring0, 1, inp.state0)
    np.testing.assert_array_equal(s, inp.state0.astype(np.float64))
    np.testing.assert_array_equal(ring, ringr)


def test_fused_prefill_right_padded_batch():
    """Per-sequence lengths: each sequence ends at its own length (state, ring), padding untouched."""
    _need_gpu()
    lens = [300, 0, 17, 129, 301, -3]
    d = workloads.CONFIGS[2].dims.replace(batch=len(lens), seqlen=300)
    inp = workloads.generate(d, 5400, True)
    y, s, ring = _fused(d, inp, inp.ring0, 0, inp.state0, lens=lens)
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    for b, n in enumerate(lens):
        n = max(0, min(n, d.seqlen))
        yr, sr, ringr, _ = oracle.mixer_prefill(inp.xbc[b:b + 1, :n], inp.dt_raw[b:b + 1, :n], inp.conv_w,
                                                inp.conv_b, inp.dt_bias, inp.A, inp.D, H, P, N, G,
                                                inp.ring0[b:b + 1], 0, inp.state0[b:b + 1])
        if n > 0:
            assert oracle.max_rel_err(y[b:b + 1, :n], yr) <= TOL, b
        assert np.isnan(y[b, n:]).all(), b
        assert oracle.max_rel_err(s[b:b + 1], sr) <= TOL, b
        np.testing.assert_array_equal(ring[b:b + 1], ringr)


def test_fused_prefill_then_decode():
    """A decode step continues from the fused prefill's state and ring exactly as from the oracle's."""
    _need_gpu()
    d = workloads.CONFIGS[2].dims.replace(batch=2, seqlen=77)
    inp = workloads.generate(d, 5500, True)
    H, P, N, G, W, Cd = d.nheads, d.headdim, d.d_state, d.n_groups, d.d_conv, d.conv_dim
    _, s, ring = _fused(d, inp, inp.ring0, 0, inp.state0)
    tok = workloads.generate(d.replace(seqlen=1), 5501, False, 3)
    dims = dims_of(d)
    ring_d, state_d = dev(ring, "bf16"), dev32(s)
    yd = torch.empty((d.batch, H * P), device="cuda", dtype=torch.bfloat16)
    _, sr, ringr, _ = oracle.mixer_prefill(inp.xbc, inp.dt_raw, inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D,
                                           H, P, N, G, inp.ring0, 0, inp.state0)
    for t in range(3):
        m2.m2_ssd_step(dims, dev(tok.xbc[t], "bf16"), dev(tok.dt_raw[t], "bf16"), dev32(inp.conv_w),
                       dev32(inp.conv_b), dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), ring_d, t, state_d, yd)
        yr, ringr, sr = oracle.ssd_step(tok.xbc[t], tok.dt_raw[t], inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D,
                                        ringr, t, sr, H, P, N, G)
    torch.cuda.synchronize()
    assert oracle.max_rel_err(host(yd), yr) <= TOL
    assert oracle.max_rel_err(host(state_d), sr) <= TOL
    np.testing.assert_array_equal(host(ring_d), ringr)


def test_fused_equals_two_kernel_path():
    """The one-pass path and conv -> scan agree (they differ only in the x channels' rounding)."""
    _need_gpu()
    d = workloads.CONFIGS[2].dims.replace(batch=2, seqlen=2048)
    inp = workloads.generate(d, 5600, True)
    y1, s1, r1 = _fused(d, inp, inp.ring0, 0, inp.state0)
    y2, s2, r2 = _two_kernels(d, inp, inp.ring0, 0, inp.state0)
    assert oracle.max_rel_err(y1, y2) <= TOL and oracle.max_rel_err(s1, s2) <= TOL
    np.testing.assert_array_equal(r1, r2)


@pytest.mark.parametrize("idx", [3, 2])
def test_full_size_fused_prefill(idx):
    """The 32768-token prompt and the 8 x 4096 batch with cached state and history, at the launch the
    benchmark times, against the fp64 oracle's conv -> scan over every head."""
    _need_gpu()
    cfg = workloads.CONFIGS[idx]
    d = cfg.dims
    inp = workloads.config_inputs(idx)
    y, s, ring = _fused(d, inp, inp.ring0, 0, inp.state0)
    yr, sr, ringr, _ = oracle.mixer_prefill(inp.xbc, inp.dt_raw, inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D,
                                            d.nheads, d.headdim, d.d_state, d.n_groups, inp.ring0, 0, inp.state0)
    ey, es = oracle.max_rel_err(y, yr), oracle.max_rel_err(s, sr)
    print("fused full size %d: y %.2e state %.2e" % (idx, ey, es))
    assert ey <= TOL and es <= TOL
    np.testing.assert_array_equal(ring, ringr)


def _pack(a, lens):
    """[batch, seqlen, ...] -> the first lens[b] tokens of each row, back to back."""
    return np.concatenate([a[b, :n] for b, n in enumerate(lens)], axis=0)


def _fused_packed(d, lens, xbc_p, dt_p, inp, ring_in, phase, state_in):
    H, P, N, W, Cd = d.nheads, d.headdim, d.d_state, d.d_conv, d.conv_dim
    dims = dims_of(d)
    T = int(sum(lens))
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
    y = nan_like((T, H * P), "bf16")
    s_out = torch.full((len(lens), H, P, N), float("nan"), device="cuda")
    ring_out = nan_like((len(lens), W, Cd), "bf16")
    n = m2.m2_mixer_prefill_workspace_packed(dims, T)
    ws = torch.empty(max(n, 1), device="cuda", dtype=torch.uint8)
    m2.m2_mixer_prefill_fwd_packed(dims, cu, dev(xbc_p, "bf16"), dev32(inp.conv_w), dev32(inp.conv_b),
                                   dev(dt_p, "bf16"), dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y,
                                   dev(ring_in, "bf16"), phase, ring_out, dev32(state_in), s_out, workspace=ws)
    torch.cuda.synchronize()
    return host(y).reshape(T, H, P), host(s_out), host(ring_out), cu


def _two_kernels_packed(d, lens, xbc_p, dt_p, inp, ring_in, phase, state_in, cu):
    H, P, N, G, W, Cd = d.nheads, d.headdim, d.d_state, d.n_groups, d.d_conv, d.conv_dim
    dims = dims_of(d)
    T = int(sum(lens))
    act = torch.empty((T, Cd), device="cuda", dtype=torch.bfloat16)
    ring_out = torch.empty((len(lens), W, Cd), device="cuda", dtype=torch.bfloat16)
    m2.m2_conv1d_fwd_packed(dims, cu, dev(xbc_p, "bf16"), dev32(inp.conv_w), dev32(inp.conv_b), act,
                            dev(ring_in, "bf16"), phase, ring_out)
    y = torch.empty((T, H * P), device="cuda", dtype=torch.bfloat16)
    s_out = torch.empty((len(lens), H, P, N), device="cuda")
    m2.m2_ssd_scan_fwd_packed(dims, cu, act[:, :H * P], act[:, H * P:H * P + G * N], act[:, H * P + G * N:],
                              dev(dt_p, "bf16"), dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y, dev32(state_in),
                              s_out, workspace=workspace(dims, T))
    torch.cuda.synchronize()
    return host(y).reshape(T, H, P), host(s_out), host(ring_out)


PACKED_FUSED_CASES = [
    [300, 0, 17, 129, 301, 1],   # an empty and a one-token prompt, ragged ends
    [2, 3, 40],                  # prompts shorter than the conv window take their history from the ring
    [4096, 1500, 0, 2500],       # several segments per prompt, empty segments
]


@pytest.mark.parametrize("lens", PACKED_FUSED_CASES, ids=lambda l: "-".join(map(str, l)))
def test_fused_prefill_packed_parity(lens):
    """Packed prompts through the one-pass path, each from its own conv history (ring phase 2) and
    initial state, against the oracle's conv -> scan of each prompt; and equal to the two-kernel packed
    path within rounding."""
    _need_gpu()
    d = workloads.CONFIGS[2].dims.replace(batch=len(lens), seqlen=max(lens))
    inp = workloads.generate(d, 5700 + len(lens), True)
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    xbc_p, dt_p = _pack(inp.xbc, lens), _pack(inp.dt_raw, lens)
    y, s, ring, cu = _fused_packed(d, lens, xbc_p, dt_p, inp, inp.ring0, 2, inp.state0)
    worst = [0.0, 0.0]
    for b, n in enumerate(lens):
        yr, sr, ringr, _ = oracle.mixer_prefill(inp.xbc[b:b + 1, :n], inp.dt_raw[b:b + 1, :n], inp.conv_w,
                                                inp.conv_b, inp.dt_bias, inp.A, inp.D, H, P, N, G,
                                                inp.ring0[b:b + 1], 2, inp.state0[b:b + 1])
        t0 = int(sum(lens[:b]))
        if n > 0:
            worst[0] = max(worst[0], oracle.max_rel_err(y[t0:t0 + n][None], yr))
        worst[1] = max(worst[1], oracle.max_rel_err(s[b:b + 1], sr))
        np.testing.assert_array_equal(ring[b:b + 1], ringr)
    y2, s2, r2 = _two_kernels_packed(d, lens, xbc_p, dt_p, inp, inp.ring0, 2, inp.state0, cu)
    e2 = max(oracle.max_rel_err(y, y2), oracle.max_rel_err(s, s2))
    print("fused packed %s: y %.2e state %.2e; vs two-kernel packed path %.2e" % (lens, worst[0], worst[1], e2))
    assert worst[0] <= TOL and worst[1] <= TOL and e2 <= TOL
    np.testing.assert_array_equal(ring, r2)


def test_full_size_fused_prefill_packed():
    """The 8 packed prompts of the benchmark (8192 ... 1024 tokens, 32768 in all, zero history and
    state) at the 2.7B shape: every prompt against the two-kernel packed path, and the shortest and a
    middle one against the oracle's conv -> scan over every head."""
    _need_gpu()
    lens = [8192, 6144, 5120, 4096, 3584, 2560, 2048, 1024]
    d1 = workloads.CONFIGS[3].dims
    T = sum(lens)
    inp = workloads.generate(d1.replace(seqlen=T), 1003, False)
    d = d1.replace(batch=len(lens), seqlen=max(lens))
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    xbc_p, dt_p = inp.xbc[0], inp.dt_raw[0]
    y, s, ring, cu = _fused_packed(d, lens, xbc_p, dt_p, inp, None, 0, None)
    y2, s2, r2 = _two_kernels_packed(d, lens, xbc_p, dt_p, inp, None, 0, None, cu)
    e2 = max(oracle.max_rel_err(y, y2), oracle.max_rel_err(s, s2))
    np.testing.assert_array_equal(ring, r2)
    worst = [0.0, 0.0]
    for b in (7, 4):
        t0, n = int(sum(lens[:b])), lens[b]
        yr, sr, ringr, _ = oracle.mixer_prefill(xbc_p[None, t0:t0 + n], dt_p[None, t0:t0 + n], inp.conv_w,
                                                inp.conv_b, inp.dt_bias, inp.A, inp.D, H, P, N, G, None, 0, None)
        worst[0] = max(worst[0], oracle.max_rel_err(y[t0:t0 + n][None], yr))
        worst[1] = max(worst[1], oracle.max_rel_err(s[b:b + 1], sr))
        np.testing.assert_array_equal(ring[b:b + 1], ringr)
    print("fused packed full size: sampled prompts y %.2e state %.2e; all prompts vs two-kernel path %.2e"
          % (worst[0], worst[1], e2))
    assert worst[0] <= TOL and worst[1] <= TOL and e2 <= TOL


def test_fused_prefill_packed_all_empty():
    """Packed prompts that are all empty (zero rows): each state passes through and each ring is a copy
    of its history, as for an empty prompt of the padded entry point."""
    _need_gpu()
    lens = [0, 0, 0]
    d = workloads.CONFIGS[2].dims.replace(batch=len(lens), seqlen=1)
    inp = workloads.generate(d, 5800, True)
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    xbc_p, dt_p = inp.xbc[0, :0], inp.dt_raw[0, :0]
    _, s, ring, _ = _fused_packed(d, lens, xbc_p, dt_p, inp, inp.ring0, 3, inp.state0)
    np.testing.assert_array_equal(s, inp.state0.astype(np.float64))
    for b in range(len(lens)):
        _, _, ringr, _ = oracle.mixer_prefill(inp.xbc[b:b + 1, :0], inp.dt_raw[b:b + 1, :0], inp.conv_w, inp.conv_b,
                                              inp.dt_bias, inp.A, inp.D, H, P, N, G, inp.ring0[b:b + 1], 3,
                                              inp.state0[b:b + 1])
        np.testing.assert_array_equal(ring[b:b + 1], ringr)
