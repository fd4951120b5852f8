"""GPU parity of the scan's backward (m2_ssd_scan_bwd) against the fp64 oracle's adjoint recurrence.

The backward returns the gradients of sum(dy * y) + <dstate_out, state_out> for the scan of the
Zamba2 mixer (article "Transformers 中 Zamba2 混合架构模型解析", §三, its training path).  Every case
compares dx, dB, dC, d(raw dt), dt_bias, dA, dD and dstate_in with oracle.ssd_scan_bwd on the same
seeded bf16 inputs, floored max-relative error <= 2e-2, and prints the errors it reaches:
  - small shapes: a ragged last chunk, one whole chunk, one token, grouped heads, no D, no initial
    state and no final adjoint, a dt clamp that binds at both bounds, and an empty prompt;
  - the 2.7B mixer shape at 2 x 2048 tokens, every head; with four B/C groups at 2 x 4096 tokens;
  - the 32768-token prompt in the launch configuration of the benchmark, on four sampled heads (a
    second call with dy and dstate_out zero outside them gives dB and dC over those heads alone);
  - right-padded batches (per-sequence lengths, padded positions left untouched), small and at the
    2.7B shape;
  - packed batches (sequences back to back at cu_seqlens offsets, each from its own state) against
    oracle.ssd_scan_bwd_packed, small (an empty, a one-token, a mid-chunk and a chunk-aligned
    sequence) and at the 2.7B shape; rows after the last sequence left untouched.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import selective_state_space_mixer_amd as m2
    from gpu_util import dev, dev32, dims_of, host, nan_like

TOL = 2e-2
KEYS = ("dx", "dB", "dC", "ddt_raw", "ddt_bias", "dA", "dD", "dstate_in")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")


def _split(d, inp):
    x, b, c = inp.split()
    lead = (d.batch, d.seqlen)
    return (x.reshape(lead + (d.nheads, d.headdim)), b.reshape(lead + (d.n_groups, d.d_state)),
            c.reshape(lead + (d.n_groups, d.d_state)))


def run_bwd(d, x, b, c, dt_raw, dt_bias, A, D, state_in, dy, ds, dt_min=0.0, dt_max=float("inf"), seq_lens=None):
    """The library's backward through the C ABI; every output starts as NaN so unwritten values show."""
    dims = dims_of(d)
    B, L, H, P, N, G = d.batch, d.seqlen, d.nheads, d.headdim, d.d_state, d.n_groups
    out = {"dx": nan_like((B, L, H * P), "bf16"), "dB": nan_like((B, L, G * N), "bf16"),
           "dC": nan_like((B, L, G * N), "bf16"), "ddt_raw": nan_like((B, L, H), "bf16")}
    for k in ("ddt_bias", "dA", "dD"):
        out[k] = torch.full((H,), float("nan"), device="cuda")
    out["dstate_in"] = torch.full((B, H, P, N), float("nan"), device="cuda")
    nws = m2.m2_ssd_scan_bwd_workspace(dims)
    assert nws > 0
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    m2.m2_ssd_scan_bwd(dims, dev(x, "bf16"), dev(b, "bf16"), dev(c, "bf16"), dev(dt_raw, "bf16"), dev32(dt_bias),
                       dev32(A), dev32(D), dev(dy, "bf16"), out["dx"], out["dB"], out["dC"], out["ddt_raw"],
                       out["ddt_bias"], out["dA"], out["dD"], state_in=dev32(state_in), dstate_out=dev32(ds),
                       dstate_in=out["dstate_in"], dt_min=dt_min, dt_max=dt_max, workspace=ws,
                       seq_lens=None if seq_lens is None else torch.as_tensor(np.asarray(seq_lens, np.int32), device="cuda"))
    torch.cuda.synchronize()
    res = {k: host(v) for k, v in out.items()}
    res["dx"] = res["dx"].reshape(B, L, H, P)
    res["dB"] = res["dB"].reshape(B, L, G, N)
    res["dC"] = res["dC"].reshape(B, L, G, N)
    return res


def errors(got, ref, keys=KEYS):
    return {k: oracle.max_rel_err(got[k], ref[k]) for k in keys}


def report(tag, err):
    print("%s: %s" % (tag, " ".join("%s %.2e" % kv for kv in err.items())))
    assert max(err.values()) <= TOL, err


SMALL = workloads.CONFIGS[2].dims.replace(d_model=256)   # 8 heads of 64 x 64, bf16
CASES = [
    ("ragged", dict(batch=2, seqlen=200), True, True, True, False),
    ("one-chunk-no-state", dict(batch=1, seqlen=64), False, False, True, False),
    ("one-token", dict(batch=2, seqlen=1), True, True, True, False),
    ("groups2", dict(batch=2, seqlen=130, n_groups=2), True, True, True, False),
    ("groups8", dict(batch=1, seqlen=100, n_groups=8), True, True, True, False),
    ("no-D", dict(batch=1, seqlen=300), True, True, False, False),
    ("clamp", dict(batch=2, seqlen=150), True, True, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_scan_backward_small(case):
    _need_gpu()
    tag, over, cached, with_ds, with_D, clamp = case
    d = SMALL.replace(**over)
    inp = workloads.generate(d, 7100 + len(tag), cached)
    x, b, c = _split(d, inp)
    dy, ds = workloads.grad_inputs(d, 7200 + len(tag), with_ds)
    D = inp.D if with_D else None
    lo, hi = (0.03, 0.12) if clamp else (0.0, float("inf"))
    if clamp:
        sp = np.logaddexp(0.0, inp.dt_raw.astype(np.float64) + inp.dt_bias)
        assert (sp < lo).sum() > 0 and (sp > hi).sum() > 0, "both clamp bounds must bind"
    got = run_bwd(d, x, b, c, inp.dt_raw, inp.dt_bias, inp.A, D, inp.state0, dy, ds, lo, hi)
    ref = oracle.ssd_scan_bwd(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, D, inp.state0, dy, ds, lo, hi)
    report("backward %s %s" % (tag, over), errors(got, ref))


def test_scan_backward_empty_prompt():
    """seqlen 0: the final state's gradient passes to dstate_in unchanged; the parameter sums are zero."""
    _need_gpu()
    d = SMALL.replace(batch=2, seqlen=0)
    rng = np.random.default_rng(3)
    H, P, N = d.nheads, d.headdim, d.d_state
    ds = rng.standard_normal((2, H, P, N)).astype(np.float32)
    z = np.zeros((2, 0, H, P), np.float32)
    zb = np.zeros((2, 0, 1, N), np.float32)
    got = run_bwd(d, z, zb, zb, np.zeros((2, 0, H), np.float32), np.full(H, -3.0, np.float32),
                  -np.ones(H, np.float32), np.ones(H, np.float32), None, z, ds)
    assert np.array_equal(got["dstate_in"], ds.astype(np.float64))
    for k in ("ddt_bias", "dA", "dD"):
        assert np.array_equal(got[k], np.zeros(H)), k


def test_scan_backward_2p7b_shape_every_head():
    _need_gpu()
    d = workloads.CONFIGS[2].dims.replace(batch=2, seqlen=2048)
    inp = workloads.generate(d, 7301, True)
    x, b, c = _split(d, inp)
    dy, ds = workloads.grad_inputs(d, 7302)
    got = run_bwd(d, x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0, dy, ds)
    ref = oracle.ssd_scan_bwd(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0, dy, ds)
    report("backward 2.7b 2x2048", errors(got, ref))


def test_scan_backward_full_size_32k_sampled_heads():
    """The 32768-token prompt (all 80 heads on the GPU, as the benchmark runs it); the oracle takes four
    heads.  Per-head gradients are compared from the full call; dB and dC, sums over the heads, from a
    second call whose dy and dstate_out are zero outside the sampled heads."""
    _need_gpu()
    d = workloads.CONFIGS[3].dims
    inp = workloads.config_inputs(3)
    x, b, c = _split(d, inp)
    dy, ds = workloads.grad_inputs(d, 7401)
    heads = [0, 27, 53, 79]
    got = run_bwd(d, x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, None, dy, ds)
    dy_m = np.zeros_like(dy)
    dy_m[:, :, heads] = dy[:, :, heads]
    ds_m = np.zeros_like(ds)
    ds_m[:, heads] = ds[:, heads]
    got_m = run_bwd(d, x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, None, dy_m, ds_m)
    ref = oracle.ssd_scan_bwd(x[:, :, heads], b, c, inp.dt_raw[:, :, heads], inp.dt_bias[heads], inp.A[heads],
                              inp.D[heads], None, dy[:, :, heads], ds[:, heads])
    sel = {"dx": got["dx"][:, :, heads], "ddt_raw": got["ddt_raw"][:, :, heads], "ddt_bias": got["ddt_bias"][heads],
           "dA": got["dA"][heads], "dD": got["dD"][heads], "dstate_in": got["dstate_in"][:, heads],
           "dB": got_m["dB"], "dC": got_m["dC"]}
    report("backward 32k, heads %s" % heads, errors(sel, ref))


def test_scan_backward_groups4_2x4096_every_head():
    """Four B/C groups of 20 heads at the 2.7B head shape, 2 x 4096 tokens (several segments per
    sequence, so the segment chains run), initial state and final adjoint given, every head and every
    gradient against the oracle."""
    _need_gpu()
    d = workloads.CONFIGS[2].dims.replace(batch=2, seqlen=4096, n_groups=4)
    inp = workloads.generate(d, 7501, True)
    x, b, c = _split(d, inp)
    dy, ds = workloads.grad_inputs(d, 7502)
    got = run_bwd(d, x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0, dy, ds)
    ref = oracle.ssd_scan_bwd(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0, dy, ds)
    report("backward 4 groups 2x4096", errors(got, ref))


def _padded_errors(got, ref, lens):
    """Errors over each sequence's real tokens; the per-token gradients past a length must be untouched."""
    err = {}
    for k in ("dx", "dB", "dC", "ddt_raw"):
        e = 0.0
        for bi, n in enumerate(lens):
            if n:
                e = max(e, oracle.max_rel_err(got[k][bi, :n], ref[k][bi, :n]))
            assert np.isnan(got[k][bi, n:]).all(), "%s written past the length of sequence %d" % (k, bi)
        err[k] = e
    for k in ("ddt_bias", "dA", "dD", "dstate_in"):
        err[k] = oracle.max_rel_err(got[k], ref[k])
    return err


@pytest.mark.parametrize("shape", ["small", "2.7b"])
def test_scan_backward_right_padded(shape):
    """Right-padded batches (per-sequence lengths): a full sequence, an empty one (its dstate_in is
    dstate_out, bit for bit), one ending inside a chunk and one on a chunk boundary; and the 2.7B shape
    at 2 x 2048 tokens with a 1000-token sequence, on a plan of several segments.  Every gradient
    against the oracle with the same lengths; padded positions untouched."""
    _need_gpu()
    if shape == "small":
        d, lens, seed = SMALL.replace(batch=4, seqlen=300), [300, 0, 131, 64], 7601
    else:
        d, lens, seed = workloads.CONFIGS[2].dims.replace(batch=2, seqlen=2048), [2048, 1000], 7611
    inp = workloads.generate(d, seed, True)
    x, b, c = _split(d, inp)
    dy, ds = workloads.grad_inputs(d, seed + 1)
    got = run_bwd(d, x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0, dy, ds, seq_lens=lens)
    ref = oracle.ssd_scan_bwd(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0, dy, ds, seq_lens=lens)
    for bi, n in enumerate(lens):
        if n == 0:
            assert np.array_equal(got["dstate_in"][bi], ds[bi].astype(np.float64)), "empty sequence %d" % bi
    report("backward right-padded %s %s" % (shape, lens), _padded_errors(got, ref, lens))


@pytest.mark.parametrize("shape", ["small", "2.7b"])
def test_scan_backward_packed(shape):
    """Packed batches through m2_ssd_scan_bwd_packed: each sequence's gradients on its own rows, from its
    own state_in and dstate_out; an empty sequence's dstate_in is its dstate_out, bit for bit.  The
    packed arrays carry 5 spare rows past the last sequence, which must stay untouched."""
    _need_gpu()
    if shape == "small":
        lens, base, seed = [130, 0, 1, 64, 77], SMALL, 7701
    else:
        lens, base, seed = [1500, 64, 2048, 333], workloads.CONFIGS[2].dims, 7711
    d = base.replace(batch=len(lens), seqlen=max(lens))
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    inp = workloads.generate(d, seed, True)
    x, b, c = _split(d, inp)
    dy, ds = workloads.grad_inputs(d, seed + 1)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pack = lambda a: np.concatenate([a[i, :n] for i, n in enumerate(lens)], 0)
    xp, bp, cp, dtp, dyp = pack(x), pack(b), pack(c), pack(inp.dt_raw), pack(dy)
    T, spare = int(cu[-1]), 5
    dims = dims_of(d)
    out = {"dx": nan_like((T + spare, H * P), "bf16"), "dB": nan_like((T + spare, G * N), "bf16"),
           "dC": nan_like((T + spare, G * N), "bf16"), "ddt_raw": nan_like((T + spare, H), "bf16")}
    for k in ("ddt_bias", "dA", "dD"):
        out[k] = torch.full((H,), float("nan"), device="cuda")
    out["dstate_in"] = torch.full((d.batch, H, P, N), float("nan"), device="cuda")
    ws = torch.empty(m2.m2_ssd_scan_bwd_workspace(dims), dtype=torch.uint8, device="cuda")
    m2.m2_ssd_scan_bwd_packed(dims, torch.as_tensor(cu, device="cuda"), dev(xp, "bf16"), dev(bp, "bf16"),
                              dev(cp, "bf16"), dev(dtp, "bf16"), dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D),
                              dev(dyp, "bf16"), out["dx"][:T], out["dB"][:T], out["dC"][:T], out["ddt_raw"][:T],
                              out["ddt_bias"], out["dA"], out["dD"], state_in=dev32(inp.state0),
                              dstate_out=dev32(ds), dstate_in=out["dstate_in"], workspace=ws)
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in out.items()}
    for k in ("dx", "dB", "dC", "ddt_raw"):
        assert np.isnan(got[k][T:]).all(), "%s written past the last sequence" % k
        got[k] = got[k][:T]
    got["dx"] = got["dx"].reshape(T, H, P)
    got["dB"] = got["dB"].reshape(T, G, N)
    got["dC"] = got["dC"].reshape(T, G, N)
    ref = oracle.ssd_scan_bwd_packed(xp, bp, cp, dtp, cu, inp.dt_bias, inp.A, inp.D, inp.state0, dyp, ds)
    for i, n in enumerate(lens):
        if n == 0:
            assert np.array_equal(got["dstate_in"][i], ds[i].astype(np.float64)), "empty sequence %d" % i
    report("backward packed %s %s" % (shape, lens), errors(got, ref))
