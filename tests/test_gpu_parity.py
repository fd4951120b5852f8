"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Every case feeds both sides the same seeded inputs (workloads/, values exactly
representable in the storage type).  Floating outputs must agree within the
floored max-relative-error bound: 2e-2 for bf16 activations with fp32 state,
1e-4 for fp32 activations.  Conv ring contents are copies of inputs and must be
bit-identical.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads
from workloads import Dims

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import selective_state_space_mixer_amd as m2
    from gpu_util import dev, dev32, dims_of, host, nan_like, tol_for, workspace


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")


# ----------------------------------------------------------------------------- conv1d

CONV_CASES = [
    # (config index, dims overrides, use ring history, ring phase)
    (0, {}, False, 0),
    (1, dict(batch=2, seqlen=300), False, 0),
    (2, dict(batch=2, seqlen=130), True, 0),
    (2, dict(batch=2, seqlen=130), True, 3),
    (2, dict(batch=2, seqlen=2), True, 1),
    (2, dict(batch=3, seqlen=0), True, 2),
    (0, dict(seqlen=65, d_conv=3), False, 0),
    (0, dict(seqlen=40, d_conv=2), False, 0),
]


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: "cfg%d-%s-ring%d-ph%d" % (c[0], c[1], c[2], c[3]))
def test_conv1d_parity(case):
    _need_gpu()
    idx, over, use_ring, phase = case
    cfg = workloads.CONFIGS[idx]
    d = cfg.dims.replace(**over)
    inp = workloads.generate(d, 1000 + idx, use_ring)
    io = d.io
    Bn, L, Cd, W = d.batch, d.seqlen, d.conv_dim, d.d_conv
    ring_in = inp.ring0 if use_ring else None
    ref, ref_ring = oracle.conv1d(inp.xbc, inp.conv_w, inp.conv_b, ring_in, phase)
    dims = dims_of(d)
    out = nan_like((Bn, L, Cd), io)
    ring_out = nan_like((Bn, W, Cd), io)
    m2.m2_conv1d_fwd(dims, dev(inp.xbc, io), dev32(inp.conv_w), dev32(inp.conv_b), out,
                     dev(ring_in, io), phase, ring_out)
    torch.cuda.synchronize()
    if L > 0:
        assert oracle.max_rel_err(host(out), ref) <= tol_for(io)
    np.testing.assert_array_equal(host(ring_out), ref_ring)


def test_conv1d_strided_unaligned_views_and_no_bias():
    """Token stride not a multiple of the vector width -> scalar path; bias NULL."""
    _need_gpu()
    d = Dims(2, 77, 16, 2, 16, 16, 1, 4, 0, "bf16")
    inp = workloads.generate(d, 7, True)
    Cd = d.conv_dim
    big = np.zeros((2, 77, Cd + 3), np.float32)
    big[:, :, 1:Cd + 1] = inp.xbc
    xbig = dev(big, "bf16")
    x_view = xbig[:, :, 1:Cd + 1]
    out_big = nan_like((2, 77, Cd + 5), "bf16")
    out_view = out_big[:, :, 2:Cd + 2]
    ref, ref_ring = oracle.conv1d(inp.xbc, inp.conv_w, None, inp.ring0, 1)
    ring_out = nan_like((2, 4, Cd), "bf16")
    m2.m2_conv1d_fwd(dims_of(d), x_view, dev32(inp.conv_w), None, out_view, dev(inp.ring0, "bf16"), 1, ring_out)
    torch.cuda.synchronize()
    assert oracle.max_rel_err(host(out_view), ref) <= 2e-2
    np.testing.assert_array_equal(host(ring_out), ref_ring)
    # the padding around the view is untouched
    assert torch.isnan(out_big[:, :, :2]).all() and torch.isnan(out_big[:, :, Cd + 2:]).all()


# ----------------------------------------------------------------------------- scan

def _scan_inputs(d, seed, cached):
    inp = workloads.generate(d, seed, cached)
    x, b, c = inp.split()
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    lead = (d.batch, d.seqlen)
    return (inp, x.reshape(lead + (H, P)), b.reshape(lead + (G, N)), c.reshape(lead + (G, N)))


def _run_scan(d, inp, x, b, c, state_in, strided=False, seq_lens=None):
    io = d.io
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    Bn, L = d.batch, d.seqlen
    dims = dims_of(d)
    if strided:
        # x, B, C as views into one conv-output-like buffer; dt as a view into a wider buffer
        buf = np.concatenate([x.reshape(Bn, L, H * P), b.reshape(Bn, L, G * N), c.reshape(Bn, L, G * N)], -1)
        tb = dev(buf, io)
        xg = tb[:, :, :H * P].unflatten(-1, (H, P))
        bg = tb[:, :, H * P:H * P + G * N].unflatten(-1, (G, N))
        cg = tb[:, :, H * P + G * N:].unflatten(-1, (G, N))
        dtb = dev(np.concatenate([np.zeros((Bn, L, 3), np.float32), inp.dt_raw, np.zeros((Bn, L, 5), np.float32)],
                                 -1), io)
        dtg = dtb[:, :, 3:3 + H]
    else:
        xg, bg, cg, dtg = dev(x, io), dev(b, io), dev(c, io), dev(inp.dt_raw, io)
    y = nan_like((Bn, L, H * P), io)
    s_out = torch.full((Bn, H, P, N), float("nan"), device="cuda")
    m2.m2_ssd_scan_fwd(dims, xg, bg, cg, dtg, dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y,
                       dev32(state_in), s_out, workspace=workspace(dims), seq_lens=_lens_dev(seq_lens))
    torch.cuda.synchronize()
    return host(y).reshape(Bn, L, H, P), host(s_out)


def _lens_dev(lens):
    return None if lens is None else torch.as_tensor(np.asarray(lens, np.int32), device="cuda")


SCAN_CASES = [
    # (config index, dims overrides, cached initial state, strided views)
    (0, {}, False, False),
    (0, dict(seqlen=100), True, True),          # ragged: 100 = 6*16 + 4
    (1, dict(batch=2, seqlen=200), False, False),
    (2, dict(batch=2, seqlen=300), True, True),
    (2, dict(batch=1, seqlen=1), True, False),
    (2, dict(batch=2, seqlen=0), True, False),
    (2, dict(batch=1, seqlen=130, chunk_size=32), True, False),
    (2, dict(batch=1, seqlen=130, chunk_size=16), True, False),
    (0, dict(d_model=64, headdim=32, d_state=16, n_groups=2, seqlen=70, io="bf16"), True, False),
    (0, dict(d_model=64, headdim=16, d_state=32, n_groups=4, seqlen=50), True, False),
]


@pytest.mark.parametrize("case", SCAN_CASES, ids=lambda c: "cfg%d-%s-init%d-str%d" % c)
def test_ssd_scan_parity(case):
    _need_gpu()
    idx, over, cached, strided = case
    d = workloads.CONFIGS[idx].dims.replace(**over)
    inp, x, b, c = _scan_inputs(d, 2000 + idx, cached)
    y, s = _run_scan(d, inp, x, b, c, inp.state0, strided)
    yr, sr = oracle.ssd_scan(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0)
    tol = tol_for(d.io)
    if d.seqlen > 0:
        assert oracle.max_rel_err(y, yr) <= tol
    assert oracle.max_rel_err(s, sr) <= tol


_PN = [(16, 16), (16, 32), (16, 64), (32, 16), (32, 32), (32, 64), (64, 16), (64, 32), (64, 64), (64, 128)]
SHAPE_CASES = ([("bf16", p, n, q) for p, n in _PN + [(128, 64), (128, 128)] for q in (16, 32, 64)] +
               [("f32", p, n, q) for p, n in _PN for q in (16, 32)])


@pytest.mark.parametrize("case", SHAPE_CASES, ids=lambda c: "%s-P%d-N%d-Q%d" % c)
def test_ssd_scan_every_built_shape(case):
    """Every (headdim, d_state, chunk, dtype) the library builds, on a short ragged prompt with a cached
    state, two groups and a plan of several segments (so the chain and the fix-up run too)."""
    _need_gpu()
    io, P, N, Q = case
    d = workloads.Dims(2, 3 * Q + 5, 2 * P, 2, P, N, 2, 4, Q, io)   # 4 heads in 2 groups
    inp, x, b, c = _scan_inputs(d, 2400 + P + N + Q, True)
    y, s = _run_scan(d, inp, x, b, c, inp.state0)
    yr, sr = oracle.ssd_scan(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0)
    tol = tol_for(io)
    assert oracle.max_rel_err(y, yr) <= tol
    assert oracle.max_rel_err(s, sr) <= tol


def test_ssd_scan_buffer_windows_move():
    """A token stride so wide that a 2^31-byte buffer window holds only a few chunks: the kernel must
    move its windows along the sequence (here after every chunk) and still match the oracle."""
    _need_gpu()
    Q = 64
    d = workloads.CONFIGS[2].dims.replace(batch=4, seqlen=3 * Q, chunk_size=Q)
    dims = dims_of(d)
    assert m2.m2_ssd_scan_workspace(dims) == 0, "expected one segment per sequence (the whole walk in one block)"
    Bn, L, H, P, N, G = d.batch, d.seqlen, d.nheads, d.headdim, d.d_state, d.n_groups
    xs = 3_600_000                                   # elements: 7.2 MB per token row of x
    win = (2 ** 31 - 1) // (Q * xs * 2) - 3          # chunks per window, as the library sizes them
    assert 1 <= win < L // Q, "the stride must force at least one window move"
    inp, x, b, c = _scan_inputs(d, 2300, True)
    xbig = torch.empty((Bn, L, xs), device="cuda", dtype=torch.bfloat16)   # 5.5 GB, only the head filled
    xv = xbig[:, :, :H * P]
    xv.copy_(dev(x.reshape(Bn, L, H * P), "bf16"))
    y = nan_like((Bn, L, H * P), "bf16")
    s_out = torch.full((Bn, H, P, N), float("nan"), device="cuda")
    m2.m2_ssd_scan_fwd(dims, xv, dev(b, "bf16"), dev(c, "bf16"), dev(inp.dt_raw, "bf16"), dev32(inp.dt_bias),
                       dev32(inp.A), dev32(inp.D), y, dev32(inp.state0), s_out, workspace=None)
    torch.cuda.synchronize()
    del xbig, xv
    yr, sr = oracle.ssd_scan(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0)
    assert oracle.max_rel_err(host(y).reshape(Bn, L, H, P), yr) <= 2e-2
    assert oracle.max_rel_err(host(s_out), sr) <= 2e-2


def test_ssd_scan_chunk_size_invariance():
    """Results do not depend on the chunk length (up to rounding)."""
    _need_gpu()
    d = workloads.CONFIGS[2].dims.replace(batch=1, seqlen=333)
    inp, x, b, c = _scan_inputs(d, 31, True)
    outs = [_run_scan(d.replace(chunk_size=q), inp, x, b, c, inp.state0) for q in (16, 32, 64)]
    for y, s in outs[1:]:
        assert oracle.max_rel_err(y, outs[0][0]) <= 2e-2
        assert oracle.max_rel_err(s, outs[0][1]) <= 2e-2


def test_ssd_scan_split_prefill_invariance():
    """Chunked prefill (two calls, state handed over) == one call (Zamba2 article §七)."""
    _need_gpu()
    d = workloads.CONFIGS[2].dims.replace(batch=2, seqlen=200)
    inp, x, b, c = _scan_inputs(d, 32, True)
    y, s = _run_scan(d, inp, x, b, c, inp.state0)
    k = 77
    d1, d2 = d.replace(seqlen=k), d.replace(seqlen=d.seqlen - k)

    class Part:
        pass

    p1, p2 = Part(), Part()
    for p, sl in ((p1, slice(0, k)), (p2, slice(k, None))):
        p.dt_raw, p.dt_bias, p.A, p.D = inp.dt_raw[:, sl], inp.dt_bias, inp.A, inp.D
    y1, s1 = _run_scan(d1, p1, x[:, :k], b[:, :k], c[:, :k], inp.state0)
    y2, s2 = _run_scan(d2, p2, x[:, k:], b[:, k:], c[:, k:], s1.astype(np.float32))
    assert oracle.max_rel_err(np.concatenate([y1, y2], 1), y) <= 2e-2
    assert oracle.max_rel_err(s2, s) <= 2e-2


def test_ssd_scan_deterministic():
    _need_gpu()
    d = workloads.CONFIGS[2].dims.replace(batch=2, seqlen=257)
    inp, x, b, c = _scan_inputs(d, 33, True)
    y1, s1 = _run_scan(d, inp, x, b, c, inp.state0)
    y2, s2 = _run_scan(d, inp, x, b, c, inp.state0)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(s1, s2)


# ----------------------------------------------------------------------------- right-padded batches
# Sequence b of a batch holds its first seq_lens[b] tokens; the rest is padding.  Lengths outside
# [0, seqlen] are clamped by the library, so the oracle gets the clamped values.

PAD_CONV_CASES = [
    # (config index, dims overrides, lengths, ring history, ring phase)
    (2, dict(batch=6, seqlen=200), [200, 0, 1, 64, 131, 3], True, 2),
    (0, dict(batch=3, seqlen=70), [70, 5, 0], False, 0),
    (2, dict(batch=2, seqlen=96), [-3, 1000], True, 1),
]


@pytest.mark.parametrize("case", PAD_CONV_CASES, ids=lambda c: "cfg%d-%s-%s" % (c[0], c[1], c[2]))
def test_conv1d_padded_batch_parity(case):
    _need_gpu()
    idx, over, lens, use_ring, phase = case
    d = workloads.CONFIGS[idx].dims.replace(**over)
    inp = workloads.generate(d, 1100 + idx, use_ring)
    io = d.io
    Bn, L, Cd, W = d.batch, d.seqlen, d.conv_dim, d.d_conv
    eff = np.clip(lens, 0, L)
    ring_in = inp.ring0 if use_ring else None
    ref, ref_ring = oracle.conv1d(inp.xbc, inp.conv_w, inp.conv_b, ring_in, phase, seq_lens=eff)
    out = nan_like((Bn, L, Cd), io)
    ring_out = nan_like((Bn, W, Cd), io)
    m2.m2_conv1d_fwd(dims_of(d), dev(inp.xbc, io), dev32(inp.conv_w), dev32(inp.conv_b), out,
                     dev(ring_in, io), phase, ring_out, seq_lens=_lens_dev(lens))
    torch.cuda.synchronize()
    got = host(out)
    for b, n in enumerate(eff):
        if n:
            assert oracle.max_rel_err(got[b, :n], ref[b, :n]) <= tol_for(io), b
        assert np.isnan(got[b, n:]).all(), "padding of sequence %d written" % b
    np.testing.assert_array_equal(host(ring_out), ref_ring)


PAD_SCAN_CASES = [
    # (config index, dims overrides, lengths, cached initial state)
    (2, dict(batch=4, seqlen=300), [300, 0, 37, 129], True),
    (0, dict(batch=3, seqlen=100), [100, 17, 0], True),
    (2, dict(batch=2, seqlen=96), [-3, 1000], False),
    (2, dict(batch=1, seqlen=130, chunk_size=16), [113], True),
]


@pytest.mark.parametrize("case", PAD_SCAN_CASES, ids=lambda c: "cfg%d-%s-%s" % (c[0], c[1], c[2]))
def test_ssd_scan_padded_batch_parity(case):
    _need_gpu()
    idx, over, lens, cached = case
    d = workloads.CONFIGS[idx].dims.replace(**over)
    inp, x, b, c = _scan_inputs(d, 2100 + idx, cached)
    eff = np.clip(lens, 0, d.seqlen)
    y, s = _run_scan(d, inp, x, b, c, inp.state0, seq_lens=lens)
    yr, sr = oracle.ssd_scan(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0, seq_lens=eff)
    tol = tol_for(d.io)
    for bb, n in enumerate(eff):
        if n:
            assert oracle.max_rel_err(y[bb, :n], yr[bb, :n]) <= tol, bb
        assert np.isnan(y[bb, n:]).all(), "padding of sequence %d written" % bb
    assert oracle.max_rel_err(s, sr) <= tol


def test_ssd_scan_padded_batch_several_segments():
    """Long sequences run as several segments per sequence (chain of end states, fix-up of the later
    segments' outputs); a sequence that ends early leaves whole segments empty."""
    _need_gpu()
    d = workloads.CONFIGS[2].dims.replace(batch=3, seqlen=4096)
    assert m2.m2_ssd_scan_workspace(dims_of(d)) > 0, "expected a multi-segment plan at this size"
    lens = [4096, 1500, 0]
    inp, x, b, c = _scan_inputs(d, 2150, True)
    y, s = _run_scan(d, inp, x, b, c, inp.state0, seq_lens=lens)
    yr, sr = oracle.ssd_scan(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0, seq_lens=lens)
    for bb, n in enumerate(lens):
        if n:
            assert oracle.max_rel_err(y[bb, :n], yr[bb, :n]) <= 2e-2, bb
        assert np.isnan(y[bb, n:]).all(), "padding of sequence %d written" % bb
    assert oracle.max_rel_err(s, sr) <= 2e-2


def test_padded_prefill_then_decode():
    """A right-padded prefill hands each sequence's own ring and state to the decode step."""
    _need_gpu()
    L, steps = 150, 4
    lens = [150, 40, 2]
    d = workloads.CONFIGS[2].dims.replace(batch=3, seqlen=L)
    inp = workloads.generate(d, 43, True)
    tok = workloads.generate(d.replace(seqlen=1), 44, False, steps)
    io = d.io
    Bn, H, P, N, G, W, Cd = d.batch, d.nheads, d.headdim, d.d_state, d.n_groups, d.d_conv, d.conv_dim
    dims = dims_of(d)
    lg = _lens_dev(lens)
    act = nan_like((Bn, L, Cd), io)
    ring = nan_like((Bn, W, Cd), io)
    m2.m2_conv1d_fwd(dims, dev(inp.xbc, io), dev32(inp.conv_w), dev32(inp.conv_b), act, dev(inp.ring0, io), 0,
                     ring, seq_lens=lg)
    y = nan_like((Bn, L, H * P), io)
    state = torch.empty((Bn, H, P, N), device="cuda")
    m2.m2_ssd_scan_fwd(dims, act[:, :, :H * P], act[:, :, H * P:H * P + G * N], act[:, :, H * P + G * N:],
                       dev(inp.dt_raw, io), dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y, dev32(inp.state0),
                       state, workspace=workspace(dims), seq_lens=lg)
    ys = []
    xt, dtt = dev(tok.xbc, io), dev(tok.dt_raw, io)
    w, cb, dtb, A, D = (dev32(a) for a in (inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D))
    for t in range(steps):
        yt = nan_like((Bn, H * P), io)
        m2.m2_ssd_step(dims, xt[t], dtt[t], w, cb, dtb, A, D, ring, t, state, yt)
        ys.append(host(yt))
    torch.cuda.synchronize()
    # oracle: the same padded prefill, then the same steps
    ref_act, r_ring = oracle.conv1d(inp.xbc, inp.conv_w, inp.conv_b, inp.ring0, 0, seq_lens=lens)
    rx, rb, rc = oracle.split_act(np.nan_to_num(ref_act), H, P, N, G)
    _, r_state = oracle.ssd_scan(rx, rb, rc, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0, seq_lens=lens)
    for t in range(steps):
        yr, r_ring, r_state = oracle.ssd_step(tok.xbc[t], tok.dt_raw[t], inp.conv_w, inp.conv_b, inp.dt_bias,
                                              inp.A, inp.D, r_ring, t, r_state, H, P, N, G)
        assert oracle.max_rel_err(ys[t], yr) <= 2e-2, "step %d" % t
    assert oracle.max_rel_err(host(state), r_state) <= 2e-2
    np.testing.assert_array_equal(host(ring), r_ring)


# ----------------------------------------------------------------------------- packed batches
# Sequences back to back in one token-major array, row offsets cu_seqlens (int32 [batch + 1]);
# dims.batch is the number of sequences and dims.seqlen the longest one.

def _pack(a, lens):
    return np.concatenate([a[b, :n] for b, n in enumerate(lens)], 0)


def _cu_dev(lens):
    return torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")


PACK_CASES = [
    # (config index, lengths, cached initial state / ring history)
    (2, [200, 0, 1, 64, 131, 3], True),
    (0, [64, 5, 0, 33], True),
    (1, [300, 17], False),
]


@pytest.mark.parametrize("case", PACK_CASES, ids=lambda c: "cfg%d-%s" % (c[0], c[1]))
def test_conv1d_packed_parity(case):
    _need_gpu()
    idx, lens, use_ring = case
    d = workloads.CONFIGS[idx].dims.replace(batch=len(lens), seqlen=max(lens))
    inp = workloads.generate(d, 1200 + idx, use_ring)
    io = d.io
    Cd, W = d.conv_dim, d.d_conv
    xp = _pack(inp.xbc, lens)
    ring_in = inp.ring0 if use_ring else None
    ref, ref_ring = oracle.conv1d_packed(xp, np.concatenate([[0], np.cumsum(lens)]), inp.conv_w, inp.conv_b,
                                         ring_in, 3)
    out = nan_like((len(xp), Cd), io)
    ring_out = nan_like((len(lens), W, Cd), io)
    m2.m2_conv1d_fwd_packed(dims_of(d), _cu_dev(lens), dev(xp, io), dev32(inp.conv_w), dev32(inp.conv_b), out,
                            dev(ring_in, io), 3, ring_out)
    torch.cuda.synchronize()
    assert oracle.max_rel_err(host(out), ref) <= tol_for(io)
    np.testing.assert_array_equal(host(ring_out), ref_ring)


PACK_SCAN_CASES = PACK_CASES + [
    (2, [4096, 1500, 0, 2500], True),   # several segments per sequence; empty segments; an empty sequence
    (0, [50, 13, 0, 64], True, dict(d_model=64, headdim=16, d_state=32, n_groups=4)),
    (0, [70, 1, 33], True, dict(d_model=64, headdim=32, d_state=16, n_groups=2, io="bf16", chunk_size=32)),
]


@pytest.mark.parametrize("case", PACK_SCAN_CASES, ids=lambda c: "cfg%d-%s%s" % (c[0], c[1], c[3] if len(c) > 3 else ""))
def test_ssd_scan_packed_parity(case):
    _need_gpu()
    idx, lens, cached = case[:3]
    over = case[3] if len(case) > 3 else {}
    d = workloads.CONFIGS[idx].dims.replace(batch=len(lens), seqlen=max(lens), **over)
    inp, x, b, c = _scan_inputs(d, 2200 + idx, cached)
    io = d.io
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    xp, bp, cp, dtp = _pack(x, lens), _pack(b, lens), _pack(c, lens), _pack(inp.dt_raw, lens)
    T = len(xp)
    yr, sr = oracle.ssd_scan_packed(xp, bp, cp, dtp, np.concatenate([[0], np.cumsum(lens)]), inp.dt_bias, inp.A,
                                    inp.D, inp.state0)
    dims = dims_of(d)
    y = nan_like((T, H * P), io)
    s_out = torch.full((len(lens), H, P, N), float("nan"), device="cuda")
    m2.m2_ssd_scan_fwd_packed(dims, _cu_dev(lens), dev(xp, io), dev(bp, io), dev(cp, io), dev(dtp, io),
                              dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y, dev32(inp.state0), s_out,
                              workspace=workspace(dims, T))
    torch.cuda.synchronize()
    tol = tol_for(io)
    assert oracle.max_rel_err(host(y).reshape(T, H, P), yr) <= tol
    assert oracle.max_rel_err(host(s_out), sr) <= tol


def test_packed_prefill_then_decode():
    """A packed prefill (conv -> scan through the conv output's strided views) hands each sequence its
    own ring and state; decode steps continue every sequence from there."""
    _need_gpu()
    lens, steps = [150, 40, 2, 77], 3
    d = workloads.CONFIGS[2].dims.replace(batch=len(lens), seqlen=max(lens))
    inp = workloads.generate(d, 45, True)
    tok = workloads.generate(d.replace(seqlen=1), 46, False, steps)
    io = d.io
    Bn, H, P, N, G, W, Cd = d.batch, d.nheads, d.headdim, d.d_state, d.n_groups, d.d_conv, d.conv_dim
    dims = dims_of(d)
    cu = _cu_dev(lens)
    xp, dtp = _pack(inp.xbc, lens), _pack(inp.dt_raw, lens)
    T = len(xp)
    act = nan_like((T, Cd), io)
    ring = nan_like((Bn, W, Cd), io)
    m2.m2_conv1d_fwd_packed(dims, cu, dev(xp, io), dev32(inp.conv_w), dev32(inp.conv_b), act, dev(inp.ring0, io),
                            0, ring)
    y = nan_like((T, H * P), io)
    state = torch.empty((Bn, H, P, N), device="cuda")
    m2.m2_ssd_scan_fwd_packed(dims, cu, act[:, :H * P], act[:, H * P:H * P + G * N], act[:, H * P + G * N:],
                              dev(dtp, io), dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y, dev32(inp.state0),
                              state, workspace=workspace(dims, T))
    ys = []
    xt, dtt = dev(tok.xbc, io), dev(tok.dt_raw, io)
    w, cb, dtb, A, D = (dev32(a) for a in (inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D))
    for t in range(steps):
        yt = nan_like((Bn, H * P), io)
        m2.m2_ssd_step(dims, xt[t], dtt[t], w, cb, dtb, A, D, ring, t, state, yt)
        ys.append(host(yt))
    torch.cuda.synchronize()
    cu_np = np.concatenate([[0], np.cumsum(lens)])
    ref_act, r_ring = oracle.conv1d_packed(xp, cu_np, inp.conv_w, inp.conv_b, inp.ring0, 0)
    assert oracle.max_rel_err(host(act), ref_act) <= 2e-2
    rx, rb, rc = oracle.split_act(ref_act, H, P, N, G)
    ry, r_state = oracle.ssd_scan_packed(rx, rb, rc, dtp, cu_np, inp.dt_bias, inp.A, inp.D, inp.state0)
    assert oracle.max_rel_err(host(y).reshape(T, H, P), ry) <= 2e-2
    for t in range(steps):
        yr, r_ring, r_state = oracle.ssd_step(tok.xbc[t], tok.dt_raw[t], inp.conv_w, inp.conv_b, inp.dt_bias,
                                              inp.A, inp.D, r_ring, t, r_state, H, P, N, G)
        assert oracle.max_rel_err(ys[t], yr) <= 2e-2, "step %d" % t
    assert oracle.max_rel_err(host(state), r_state) <= 2e-2
    np.testing.assert_array_equal(host(ring), r_ring)


# ----------------------------------------------------------------------------- decode step

def _gpu_chain(d, inp, steps, ring0, state0, first_step=0):
    io = d.io
    Bn, H, P, N, W, Cd = d.batch, d.nheads, d.headdim, d.d_state, d.d_conv, d.conv_dim
    dims = dims_of(d)
    ring = dev(ring0, io) if ring0 is not None else torch.zeros((Bn, W, Cd), device="cuda", dtype=torch.bfloat16
                                                                if io == "bf16" else torch.float32)
    state = dev32(state0) if state0 is not None else torch.zeros((Bn, H, P, N), device="cuda")
    xt = dev(inp.xbc, io)
    dtt = dev(inp.dt_raw, io)
    w, cb, dtb, A, D = (dev32(a) for a in (inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D))
    ys = []
    for t in range(steps):
        y = nan_like((Bn, H * P), io)
        m2.m2_ssd_step(dims, xt[t], dtt[t], w, cb, dtb, A, D, ring, first_step + t, state, y)
        ys.append(y)
    torch.cuda.synchronize()
    return np.stack([host(y) for y in ys]), host(ring), host(state)


@pytest.mark.parametrize("over,steps", [(dict(batch=3), 6), (dict(batch=2, d_conv=3), 5),
                                        (dict(batch=1, d_model=64, headdim=16, d_state=32, n_groups=2), 7)])
def test_ssd_step_chain_parity(over, steps):
    _need_gpu()
    d = workloads.CONFIGS[4].dims.replace(**over)
    inp = workloads.generate(d, 1004, True, steps)
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    ys, ring, state = _gpu_chain(d, inp, steps, inp.ring0, inp.state0)
    r_ring, r_state = inp.ring0.astype(np.float64), inp.state0.astype(np.float64)
    for t in range(steps):
        yr, r_ring, r_state = oracle.ssd_step(inp.xbc[t], inp.dt_raw[t], inp.conv_w, inp.conv_b, inp.dt_bias,
                                              inp.A, inp.D, r_ring, t, r_state, H, P, N, G)
        assert oracle.max_rel_err(ys[t], yr) <= 2e-2, "step %d" % t
    assert oracle.max_rel_err(state, r_state) <= 2e-2
    np.testing.assert_array_equal(ring, r_ring)


STEP_SHAPES = [("bf16", 16, 16, 4), ("f32", 24, 32, 3), ("bf16", 64, 64, 2), ("f32", 64, 128, 4),
               ("bf16", 128, 64, 4), ("bf16", 32, 256, 3), ("f32", 80, 64, 4), ("bf16", 256, 32, 4)]


@pytest.mark.parametrize("case", STEP_SHAPES, ids=lambda c: "%s-P%d-N%d-W%d" % c)
def test_ssd_step_every_kind_of_shape(case):
    """Decode steps over head sizes that use every per-thread state share the kernel has (1, 2, 4, 8
    float4 per thread), odd head sizes, each d_state it builds, each conv width, both dtypes."""
    _need_gpu()
    io, P, N, W = case
    d = workloads.Dims(3, 1, 2 * P, 2, P, N, 2, W, 0, io)   # 4 heads in 2 groups
    steps = 3
    inp = workloads.generate(d, 1500 + P + N, True, steps)
    H, G = d.nheads, d.n_groups
    ys, ring, state = _gpu_chain(d, inp, steps, inp.ring0, inp.state0, first_step=2)
    r_ring, r_state = inp.ring0.astype(np.float64), inp.state0.astype(np.float64)
    tol = tol_for(io)
    for t in range(steps):
        yr, r_ring, r_state = oracle.ssd_step(inp.xbc[t], inp.dt_raw[t], inp.conv_w, inp.conv_b, inp.dt_bias,
                                              inp.A, inp.D, r_ring, 2 + t, r_state, H, P, N, G)
        assert oracle.max_rel_err(ys[t], yr) <= tol, "step %d" % t
    assert oracle.max_rel_err(state, r_state) <= tol
    np.testing.assert_array_equal(ring, r_ring)


def test_ssd_step_fp32_chain_parity():
    _need_gpu()
    d = workloads.CONFIGS[0].dims.replace(batch=2, seqlen=1)
    steps = 64
    inp = workloads.generate(d, 1000, True, steps)
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    ys, ring, state = _gpu_chain(d, inp, steps, inp.ring0, inp.state0, first_step=5)
    r_ring, r_state = inp.ring0.astype(np.float64), inp.state0.astype(np.float64)
    yref = []
    for t in range(steps):
        yr, r_ring, r_state = oracle.ssd_step(inp.xbc[t], inp.dt_raw[t], inp.conv_w, inp.conv_b, inp.dt_bias,
                                              inp.A, inp.D, r_ring, 5 + t, r_state, H, P, N, G)
        yref.append(yr)
    assert oracle.max_rel_err(ys, np.stack(yref)) <= 1e-4
    assert oracle.max_rel_err(state, r_state) <= 1e-4
    np.testing.assert_array_equal(ring, r_ring)


def test_decode_chain_equals_prefill():
    """Token-by-token decode path == chunked prefill path (Zamba2 article §七), both on the GPU."""
    _need_gpu()
    L = 45
    d = workloads.CONFIGS[2].dims.replace(batch=2, seqlen=L)
    inp = workloads.generate(d, 41, True)
    io = d.io
    Bn, H, P, N, G, W, Cd = d.batch, d.nheads, d.headdim, d.d_state, d.n_groups, d.d_conv, d.conv_dim
    dims = dims_of(d)
    # prefill: conv (ring history at phase 0) -> scan, both through the ABI
    act = nan_like((Bn, L, Cd), io)
    ring_out = nan_like((Bn, W, Cd), io)
    m2.m2_conv1d_fwd(dims, dev(inp.xbc, io), dev32(inp.conv_w), dev32(inp.conv_b), act, dev(inp.ring0, io), 0,
                     ring_out)
    y = nan_like((Bn, L, H * P), io)
    s_out = torch.empty((Bn, H, P, N), device="cuda")
    dt = dev(inp.dt_raw, io)
    m2.m2_ssd_scan_fwd(dims, act[:, :, :H * P], act[:, :, H * P:H * P + G * N], act[:, :, H * P + G * N:], dt,
                       dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y, dev32(inp.state0), s_out,
                       workspace=workspace(dims))
    torch.cuda.synchronize()

    class Tok:
        pass

    tok = Tok()
    tok.xbc = np.ascontiguousarray(inp.xbc.transpose(1, 0, 2))
    tok.dt_raw = np.ascontiguousarray(inp.dt_raw.transpose(1, 0, 2))
    tok.conv_w, tok.conv_b, tok.dt_bias, tok.A, tok.D = inp.conv_w, inp.conv_b, inp.dt_bias, inp.A, inp.D
    ys, ring, state = _gpu_chain(d, tok, L, inp.ring0, inp.state0)
    assert oracle.max_rel_err(state, host(s_out)) <= 2e-2
    assert oracle.max_rel_err(ys.transpose(1, 0, 2), host(y)) <= 2e-2
    ro = host(ring_out)
    for j in range(1, W + 1):
        np.testing.assert_array_equal(ring[:, (L - j) % W], ro[:, W - j])


# ----------------------------------------------------------------------------- full-size workloads

def _sampled_scan_check(idx, heads, batches):
    cfg = workloads.CONFIGS[idx]
    d = cfg.dims
    inp = workloads.config_inputs(idx)
    io = d.io
    Bn, L, H, P, N, G, W, Cd = d.batch, d.seqlen, d.nheads, d.headdim, d.d_state, d.n_groups, d.d_conv, d.conv_dim
    dims = dims_of(d)
    act = torch.empty((Bn, L, Cd), device="cuda", dtype=torch.bfloat16)
    ring_out = torch.empty((Bn, W, Cd), device="cuda", dtype=torch.bfloat16)
    xbc = dev(inp.xbc, io)
    m2.m2_conv1d_fwd(dims, xbc, dev32(inp.conv_w), dev32(inp.conv_b), act, dev(inp.ring0, io), 0, ring_out)
    y = torch.empty((Bn, L, H * P), device="cuda", dtype=torch.bfloat16)
    s_out = torch.empty((Bn, H, P, N), device="cuda")
    m2.m2_ssd_scan_fwd(dims, act[:, :, :H * P], act[:, :, H * P:H * P + G * N], act[:, :, H * P + G * N:],
                       dev(inp.dt_raw, io), dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y,
                       dev32(inp.state0), s_out, workspace=workspace(dims))
    torch.cuda.synchronize()
    del xbc
    # conv: sampled channels against the oracle (x, B and C channels)
    chans = np.array([0, 1, H * P - 1, H * P, H * P + N - 1, Cd - 1])
    for b in batches:
        ring_b = None if inp.ring0 is None else inp.ring0[b:b + 1][:, :, chans]
        ref, ref_ring = oracle.conv1d(inp.xbc[b:b + 1][:, :, chans], inp.conv_w[chans], inp.conv_b[chans], ring_b, 0)
        got = host(act[b:b + 1][:, :, torch.as_tensor(chans, device="cuda")])
        assert oracle.max_rel_err(got, ref) <= 2e-2
        np.testing.assert_array_equal(host(ring_out[b:b + 1][:, :, torch.as_tensor(chans, device="cuda")]),
                                      ref_ring)
    # scan: whole sequences of sampled (b, h), fed the GPU's own conv output (per-kernel parity)
    for b in batches:
        a_b = host(act[b])
        for h in heads:
            g = h // (H // G)
            xs = a_b[:, h * P:(h + 1) * P].reshape(1, L, 1, P)
            bs = a_b[:, H * P + g * N:H * P + (g + 1) * N].reshape(1, L, 1, N)
            cs = a_b[:, H * P + G * N + g * N:H * P + G * N + (g + 1) * N].reshape(1, L, 1, N)
            s0 = None if inp.state0 is None else inp.state0[b:b + 1, h:h + 1]
            yr, sr = oracle.ssd_scan(xs, bs, cs, inp.dt_raw[b:b + 1, :, h:h + 1], inp.dt_bias[h:h + 1],
                                     inp.A[h:h + 1], inp.D[h:h + 1], s0)
            got_y = host(y[b, :, h * P:(h + 1) * P]).reshape(1, L, 1, P)
            assert oracle.max_rel_err(got_y, yr) <= 2e-2, (b, h)
            assert oracle.max_rel_err(host(s_out[b:b + 1, h:h + 1]), sr) <= 2e-2, (b, h)


def test_full_size_prefill_b8_l4096_sampled():
    _need_gpu()
    _sampled_scan_check(2, heads=[0, 37, 79], batches=[0, 7])


def test_full_size_prefill_b1_l32768_sampled():
    _need_gpu()
    _sampled_scan_check(3, heads=[0, 52, 79], batches=[0])


def test_full_size_prefill_130m_sampled():
    _need_gpu()
    _sampled_scan_check(1, heads=[0, 23], batches=[0, 3])


def test_full_size_packed_prompts_sampled():
    """Eight prompts of 8192 .. 1024 tokens (32768 in all) packed back to back at the Zamba2-2.7B shape,
    as the benchmark runs them: sampled prompts and heads of the scan, fed the GPU's own conv output."""
    _need_gpu()
    lens = [8192, 6144, 5120, 4096, 3584, 2560, 2048, 1024]
    d1 = workloads.CONFIGS[3].dims
    T = sum(lens)
    inp = workloads.generate(d1.replace(seqlen=T), 1003, False)
    H, P, N, G, W, Cd = d1.nheads, d1.headdim, d1.d_state, d1.n_groups, d1.d_conv, d1.conv_dim
    d = d1.replace(batch=len(lens), seqlen=max(lens))
    dims = dims_of(d)
    cu = _cu_dev(lens)
    cu_np = np.concatenate([[0], np.cumsum(lens)])
    act = torch.empty((T, Cd), device="cuda", dtype=torch.bfloat16)
    ring_out = torch.empty((len(lens), W, Cd), device="cuda", dtype=torch.bfloat16)
    m2.m2_conv1d_fwd_packed(dims, cu, dev(inp.xbc[0], "bf16"), dev32(inp.conv_w), dev32(inp.conv_b), act, None, 0,
                            ring_out)
    y = torch.empty((T, H * P), device="cuda", dtype=torch.bfloat16)
    s_out = torch.empty((len(lens), H, P, N), device="cuda")
    m2.m2_ssd_scan_fwd_packed(dims, cu, act[:, :H * P], act[:, H * P:H * P + G * N], act[:, H * P + G * N:],
                              dev(inp.dt_raw[0], "bf16"), dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y, None,
                              s_out, workspace=workspace(dims, T))
    torch.cuda.synchronize()
    a_all = host(act)
    for b in (0, 3, 7):
        r0, r1 = cu_np[b], cu_np[b + 1]
        n = r1 - r0
        # conv of sampled channels of this prompt, and its ring
        chans = np.array([0, H * P - 1, H * P, Cd - 1])
        ref, ref_ring = oracle.conv1d(inp.xbc[0][None, r0:r1][:, :, chans], inp.conv_w[chans], inp.conv_b[chans])
        assert oracle.max_rel_err(a_all[None, r0:r1][:, :, chans], ref) <= 2e-2, b
        np.testing.assert_array_equal(host(ring_out[b])[:, chans], ref_ring[0])
        for h in (0, 41, 79):
            g = h // (H // G)
            xs = a_all[r0:r1, h * P:(h + 1) * P].reshape(1, n, 1, P)
            bs = a_all[r0:r1, H * P + g * N:H * P + (g + 1) * N].reshape(1, n, 1, N)
            cs = a_all[r0:r1, H * P + G * N + g * N:H * P + G * N + (g + 1) * N].reshape(1, n, 1, N)
            yr, sr = oracle.ssd_scan(xs, bs, cs, inp.dt_raw[0][None, r0:r1, h:h + 1], inp.dt_bias[h:h + 1],
                                     inp.A[h:h + 1], inp.D[h:h + 1])
            got = host(y[r0:r1, h * P:(h + 1) * P]).reshape(1, n, 1, P)
            assert oracle.max_rel_err(got, yr) <= 2e-2, (b, h)
            assert oracle.max_rel_err(host(s_out[b:b + 1, h:h + 1]), sr) <= 2e-2, (b, h)


def test_full_size_decode_b256_sampled():
    """256 sequences, a few chained steps; sampled sequences against the oracle chain."""
    _need_gpu()
    cfg = workloads.CONFIGS[4]
    d = cfg.dims
    steps = 3
    inp = workloads.generate(d, 1004, True, steps)
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    ys, ring, state = _gpu_chain(d, inp, steps, inp.ring0, inp.state0)
    for b in (0, 131, 255):
        r_ring = inp.ring0[b:b + 1].astype(np.float64)
        r_state = inp.state0[b:b + 1].astype(np.float64)
        for t in range(steps):
            yr, r_ring, r_state = oracle.ssd_step(inp.xbc[t, b:b + 1], inp.dt_raw[t, b:b + 1], inp.conv_w,
                                                  inp.conv_b, inp.dt_bias, inp.A, inp.D, r_ring, t, r_state,
                                                  H, P, N, G)
            assert oracle.max_rel_err(ys[t, b:b + 1], yr) <= 2e-2
        assert oracle.max_rel_err(state[b:b + 1], r_state) <= 2e-2
        np.testing.assert_array_equal(ring[b:b + 1], r_ring)


# ----------------------------------------------------------------------------- gated group RMSNorm

NORM_CASES = [
    # (io, rows, d_inner, group_size, norm_before_gate, mode)
    ("bf16", 64, 5120, 5120, False, "plain"),     # Zamba2-2.7B: one group over d_inner
    ("bf16", 64, 5120, 5120, True, "plain"),
    ("bf16", 37, 1536, 1536, False, "strided"),   # 130m-like d_inner, rows inside a wider buffer
    ("bf16", 9, 5120, 1280, True, "in_place"),    # four groups, out written over y
    ("f32", 33, 256, 64, False, "plain"),         # groups smaller than a wave's row
    ("f32", 5, 96, 24, True, "strided"),          # six pieces per group
    ("bf16", 0, 5120, 5120, False, "plain"),      # no rows
]


@pytest.mark.parametrize("case", NORM_CASES, ids=lambda c: "%s-%dx%d-g%d-nbg%d-%s" % c)
def test_gated_rmsnorm_parity(case):
    _need_gpu()
    io, T, D, gs, nbg, mode = case
    y, z, w = workloads.norm_inputs(T, D, 3000 + D + T, io)
    if mode == "strided":
        # y and z as column slices of one [T, 2D + 16] buffer (the gate and the scan output side by side)
        buf = dev(np.concatenate([z, y, np.zeros((T, 16), np.float32)], 1), io)
        zg, yg = buf[:, :D], buf[:, D:2 * D]
    else:
        yg, zg = dev(y, io), dev(z, io)
    out = yg if mode == "in_place" else nan_like((T, D), io)
    m2.m2_gated_rmsnorm(yg, zg, dev32(w), out, gs, eps=1e-5, norm_before_gate=nbg)
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(y, z, w, gs, 1e-5, nbg)
    if T > 0:
        assert oracle.max_rel_err(host(out), ref) <= tol_for(io)


@pytest.mark.parametrize("nbg", [False, True], ids=["gate-first", "norm-first"])
def test_full_size_gated_rmsnorm_32k_sampled(nbg):
    """The whole 32k-token prefill output at the 2.7B shape, both gate orders (each its own kernel);
    sampled rows against the oracle."""
    _need_gpu()
    T, D = 32768, 5120
    y, z, w = workloads.norm_inputs(T, D, 3100, "bf16")
    out = nan_like((T, D), "bf16")
    m2.m2_gated_rmsnorm(dev(y, "bf16"), dev(z, "bf16"), dev32(w), out, D, norm_before_gate=nbg)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 4095, 17000, 32767])
    got = host(out[torch.from_numpy(rows).cuda()])
    ref = oracle.gated_rmsnorm(y[rows], z[rows], w, D, 1e-5, nbg)
    e = oracle.max_rel_err(got, ref)
    print("full-size gated norm (norm first: %s), sampled rows: %.2e" % (nbg, e))
    assert e <= 2e-2
    assert not torch.isnan(out.float()).any().item()
