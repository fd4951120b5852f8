"""Seeded random cases against the fp64 oracle, across the option space that the hand-picked tests cover
one corner at a time: 1-5 prompts of lengths 0 ... 3000 tokens (on and off chunk and window boundaries),
1, 2 or 4 B/C groups, 4-32 heads, conv widths 2-4, with or without conv history at ring phases 0-5 and
an initial state.

- the one-pass prompt path, right-padded (seq_lens) and packed (cu_seqlens), each prompt against the
  oracle's conv -> scan (y, final state; rings bit-exact; padding untouched);
- the scan backward, right-padded and packed, every gradient against the oracle's adjoint recurrence;
- the scan on its own, right-padded and packed, over every built (headdim, d_state, chunk, dtype), 1-12
  heads in 1, 2 or 4 groups, against the oracle per sequence (2e-2 for bf16, 1e-4 for fp32);
- chains of decode steps over head sizes 8-256, d_state 16-256, conv widths 2-4, both dtypes, from any
  ring phase, each step's output and the final state and ring against the oracle's step chain.

The case list is drawn from a fixed seed when the tests are collected, so a failure names its case."""
import random

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import selective_state_space_mixer_amd as m2
    from gpu_util import dev, dev32, dims_of, host, nan_like
    import test_gpu_bwd as tb
    import test_gpu_parity as tp
    from gpu_util import tol_for, workspace

TOL = 2e-2


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")


def _fwd_cases(seed=7, n=40):
    rng, out = random.Random(seed), []
    while len(out) < n:
        nb = rng.randint(1, 5)
        lens = [rng.choice([0, 1, 2, 3, 5, 31, 32, 33, 64, 100, 257, 700, 1500, 3000]) for _ in range(nb)]
        groups, d_model, d_conv = rng.choice([1, 2, 4]), rng.choice([128, 256, 512]), rng.choice([2, 3, 4])
        cached, phase = rng.random() < 0.7, rng.randint(0, 5)
        if (2 * d_model // 64 // groups) % 4:   # the one-pass path takes heads per group in fours
            continue
        out.append((lens, groups, d_model, d_conv, cached, phase, 9000 + len(out)))
    return out


def _bwd_cases(seed=11, n=16):
    rng, out = random.Random(seed), []
    while len(out) < n:
        nb = rng.randint(1, 4)
        lens = [rng.choice([0, 1, 2, 63, 64, 65, 100, 300, 1000, 2100]) for _ in range(nb)]
        groups, d_model = rng.choice([1, 2, 4]), rng.choice([128, 256, 512])
        if (2 * d_model // 64) % groups:
            continue
        out.append((lens, groups, d_model, 9500 + len(out)))
    return out


def _scan_cases(seed=5, n=30):
    from test_gpu_parity import SHAPE_CASES
    rng, out = random.Random(seed), []
    for _ in range(n):
        io, P, N, Q = rng.choice(SHAPE_CASES)
        nb = rng.randint(1, 4)
        lens = [rng.choice([0, 1, Q - 1, Q, Q + 1, 3 * Q + 5, 200, 700, 1600]) for _ in range(nb)]
        G = rng.choice([1, 2, 4])
        out.append((io, P, N, Q, G, G * rng.choice([1, 2, 3]), lens, rng.random() < 0.7, 9900 + len(out)))
    return out


@pytest.mark.parametrize("case", _fwd_cases(), ids=lambda c: "L%s-G%d-dm%d-W%d-h%d-ph%d" % (
    "_".join(map(str, c[0])), c[1], c[2], c[3], c[4], c[5]))
def test_random_one_pass_prefill(case):
    _need_gpu()
    lens, groups, d_model, d_conv, cached, phase, seed = case
    nb = len(lens)
    d = workloads.CONFIGS[2].dims.replace(batch=nb, seqlen=max(1, max(lens)), n_groups=groups, d_model=d_model,
                                          d_conv=d_conv)
    inp = workloads.generate(d, seed, cached)
    ring_in = inp.ring0 if cached else None
    s_in = inp.state0 if cached else None
    H, P, N, G, W, Cd = d.nheads, d.headdim, d.d_state, d.n_groups, d.d_conv, d.conv_dim
    dims = dims_of(d)
    # packed
    T = sum(lens)
    xbc_p = np.concatenate([inp.xbc[b, :n] for b, n in enumerate(lens)], axis=0)
    dt_p = np.concatenate([inp.dt_raw[b, :n] for b, n in enumerate(lens)], axis=0)
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
    y = nan_like((T, H * P), "bf16")
    s = torch.full((nb, H, P, N), float("nan"), device="cuda")
    ring = nan_like((nb, W, Cd), "bf16")
    ws = torch.empty(max(m2.m2_mixer_prefill_workspace_packed(dims, T), 1), device="cuda", dtype=torch.uint8)
    m2.m2_mixer_prefill_fwd_packed(dims, cu, dev(xbc_p, "bf16"), dev32(inp.conv_w), dev32(inp.conv_b),
                                   dev(dt_p, "bf16"), dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y,
                                   dev(ring_in, "bf16"), phase, ring, dev32(s_in), s, workspace=ws)
    # right-padded
    yq = nan_like((nb, d.seqlen, H * P), "bf16")
    sq = torch.full((nb, H, P, N), float("nan"), device="cuda")
    ringq = nan_like((nb, W, Cd), "bf16")
    wsq = torch.empty(max(m2.m2_mixer_prefill_workspace(dims), 1), device="cuda", dtype=torch.uint8)
    m2.m2_mixer_prefill_fwd(dims, dev(inp.xbc, "bf16"), dev32(inp.conv_w), dev32(inp.conv_b), dev(inp.dt_raw, "bf16"),
                            dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), yq, dev(ring_in, "bf16"), phase, ringq,
                            dev32(s_in), sq, workspace=wsq,
                            seq_lens=torch.as_tensor(np.asarray(lens, np.int32), device="cuda"))
    torch.cuda.synchronize()
    yh, sh, rh = host(y).reshape(T, H, P), host(s), host(ring)
    yqh, sqh, rqh = host(yq).reshape(nb, d.seqlen, H, P), host(sq), host(ringq)
    worst = 0.0
    for b, n in enumerate(lens):
        yr, sr, rr, _ = oracle.mixer_prefill(inp.xbc[b:b + 1, :n], inp.dt_raw[b:b + 1, :n], inp.conv_w, inp.conv_b,
                                             inp.dt_bias, inp.A, inp.D, H, P, N, G,
                                             None if ring_in is None else ring_in[b:b + 1], phase,
                                             None if s_in is None else s_in[b:b + 1])
        t0 = sum(lens[:b])
        errs = [oracle.max_rel_err(sh[b:b + 1], sr), oracle.max_rel_err(sqh[b:b + 1], sr)]
        if n > 0:
            errs += [oracle.max_rel_err(yh[t0:t0 + n][None], yr), oracle.max_rel_err(yqh[b:b + 1, :n], yr)]
        worst = max([worst] + errs)
        assert max(errs) <= TOL, (b, errs)
        np.testing.assert_array_equal(rh[b:b + 1], rr)
        np.testing.assert_array_equal(rqh[b:b + 1], rr)
        assert np.isnan(yqh[b, n:]).all(), "padding of sequence %d written" % b
    print("random one-pass %s: worst %.2e" % (lens, worst))


@pytest.mark.parametrize("case", _bwd_cases(), ids=lambda c: "L%s-G%d-dm%d" % ("_".join(map(str, c[0])), c[1], c[2]))
def test_random_scan_backward(case):
    _need_gpu()
    lens, groups, d_model, seed = case
    d = workloads.CONFIGS[2].dims.replace(batch=len(lens), seqlen=max(1, max(lens)), n_groups=groups, d_model=d_model)
    inp = workloads.generate(d, seed, True)
    x, b, c = tb._split(d, inp)
    dy, ds = workloads.grad_inputs(d, seed + 100)
    H, P, N, G = d.nheads, d.headdim, d.d_state, d.n_groups
    got = tb.run_bwd(d, x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0, dy, ds, seq_lens=lens)
    ref = oracle.ssd_scan_bwd(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0, dy, ds, seq_lens=lens)
    e1 = tb._padded_errors(got, ref, lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pack = lambda a: np.concatenate([a[i, :n] for i, n in enumerate(lens)], 0)
    xp, bp, cp, dtp, dyp = pack(x), pack(b), pack(c), pack(inp.dt_raw), pack(dy)
    T, dims = int(cu[-1]), dims_of(d)
    out = {"dx": nan_like((T, H * P), "bf16"), "dB": nan_like((T, G * N), "bf16"),
           "dC": nan_like((T, G * N), "bf16"), "ddt_raw": nan_like((T, H), "bf16")}
    for k in ("ddt_bias", "dA", "dD"):
        out[k] = torch.full((H,), float("nan"), device="cuda")
    out["dstate_in"] = torch.full((d.batch, H, P, N), float("nan"), device="cuda")
    ws = torch.empty(m2.m2_ssd_scan_bwd_workspace(dims), dtype=torch.uint8, device="cuda")
    m2.m2_ssd_scan_bwd_packed(dims, torch.as_tensor(cu, device="cuda"), dev(xp, "bf16"), dev(bp, "bf16"),
                              dev(cp, "bf16"), dev(dtp, "bf16"), dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D),
                              dev(dyp, "bf16"), out["dx"], out["dB"], out["dC"], out["ddt_raw"], out["ddt_bias"],
                              out["dA"], out["dD"], state_in=dev32(inp.state0), dstate_out=dev32(ds),
                              dstate_in=out["dstate_in"], workspace=ws)
    torch.cuda.synchronize()
    g2 = {k: host(v) for k, v in out.items()}
    g2["dx"], g2["dB"], g2["dC"] = g2["dx"].reshape(T, H, P), g2["dB"].reshape(T, G, N), g2["dC"].reshape(T, G, N)
    r2 = oracle.ssd_scan_bwd_packed(xp, bp, cp, dtp, cu, inp.dt_bias, inp.A, inp.D, inp.state0, dyp, ds)
    e2 = tb.errors(g2, r2)
    print("random backward %s G%d: padded %.2e packed %.2e" % (lens, groups, max(e1.values()), max(e2.values())))
    assert max(e1.values()) <= TOL, e1
    assert max(e2.values()) <= TOL, e2


@pytest.mark.parametrize("case", _scan_cases(), ids=lambda c: "%s-P%d-N%d-Q%d-G%d-H%d-L%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "_".join(map(str, c[6]))))
def test_random_scan(case):
    _need_gpu()
    io, P, N, Q, G, H, lens, cached, seed = case
    nb = len(lens)
    d = workloads.Dims(nb, max(1, max(lens)), H * P // 2, 2, P, N, G, 4, Q, io)
    inp, x, b, c = tp._scan_inputs(d, seed, cached)
    s0 = inp.state0
    dims, tol = dims_of(d), tol_for(io)
    yq, sq = tp._run_scan(d, inp, x, b, c, s0, seq_lens=lens)
    pack = lambda a: np.concatenate([a[i, :n] for i, n in enumerate(lens)], 0)
    xp, bp, cp, dtp = pack(x), pack(b), pack(c), pack(inp.dt_raw)
    T = len(xp)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    y = nan_like((T, H * P), io)
    s = torch.full((nb, H, P, N), float("nan"), device="cuda")
    m2.m2_ssd_scan_fwd_packed(dims, torch.as_tensor(cu, device="cuda"), dev(xp, io), dev(bp, io), dev(cp, io),
                              dev(dtp, io), dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y, dev32(s0), s,
                              workspace=workspace(dims, T))
    torch.cuda.synchronize()
    errs = []
    for bi, n in enumerate(lens):
        yr, sr = oracle.ssd_scan(x[bi:bi + 1, :n], b[bi:bi + 1, :n], c[bi:bi + 1, :n], inp.dt_raw[bi:bi + 1, :n],
                                 inp.dt_bias, inp.A, inp.D, None if s0 is None else s0[bi:bi + 1])
        errs.append(oracle.max_rel_err(sq[bi:bi + 1], sr))
        if n:
            errs.append(oracle.max_rel_err(yq[bi:bi + 1, :n], yr))
    yr2, sr2 = oracle.ssd_scan_packed(xp, bp, cp, dtp, cu, inp.dt_bias, inp.A, inp.D, s0)
    errs.append(oracle.max_rel_err(host(s), sr2))
    if T:
        errs.append(oracle.max_rel_err(host(y).reshape(T, H, P), yr2))
    print("random scan %s P%d N%d Q%d G%d H%d %s: worst %.2e (bar %.0e)" % (io, P, N, Q, G, H, lens, max(errs), tol))
    assert max(errs) <= tol, errs


def _step_cases(seed=13, n=24):
    rng, out = random.Random(seed), []
    while len(out) < n:
        io = rng.choice(["bf16", "f32"])
        P, N = rng.choice([8, 16, 24, 32, 48, 64, 80, 96, 128, 256]), rng.choice([16, 32, 64, 128, 256])
        if P * (N // 4) > 8 * 256 or P + 2 * N > 1024:   # the shapes the decode kernel builds
            continue
        G = rng.choice([1, 2, 4])
        out.append((io, P, N, G, G * rng.choice([1, 2]), rng.choice([2, 3, 4]), rng.randint(1, 4),
                    rng.randint(2, 6), rng.randint(0, 5), rng.random() < 0.8, 9700 + len(out)))
    return out


@pytest.mark.parametrize("case", _step_cases(), ids=lambda c: "%s-P%d-N%d-G%d-H%d-W%d-B%d-S%d-from%d" % c[:9])
def test_random_decode_chain(case):
    _need_gpu()
    io, P, N, G, H, W, Bn, steps, first, cached, seed = case
    d = workloads.Dims(Bn, 1, H * P // 2, 2, P, N, G, W, 0, io)
    inp = workloads.generate(d, seed, cached, steps)
    ys, ring, state = tp._gpu_chain(d, inp, steps, inp.ring0, inp.state0, first_step=first)
    Cd = d.conv_dim
    r_ring = inp.ring0.astype(np.float64) if inp.ring0 is not None else np.zeros((Bn, W, Cd))
    r_state = inp.state0.astype(np.float64) if inp.state0 is not None else np.zeros((Bn, H, P, N))
    tol = tol_for(io)
    worst = 0.0
    for t in range(steps):
        yr, r_ring, r_state = oracle.ssd_step(inp.xbc[t], inp.dt_raw[t], inp.conv_w, inp.conv_b, inp.dt_bias, inp.A,
                                              inp.D, r_ring, first + t, r_state, H, P, N, G)
        e = oracle.max_rel_err(ys[t], yr)
        worst = max(worst, e)
        assert e <= tol, "step %d: %.2e" % (t, e)
    es = oracle.max_rel_err(state, r_state)
    print("random decode chain %s P%d N%d G%d H%d W%d: y %.2e state %.2e" % (io, P, N, G, H, W, worst, es))
    assert es <= tol
    np.testing.assert_array_equal(ring, r_ring)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_packed_scan_many_sequences(io):
    """260 packed prompts, two of 640 tokens among short and empty ones, at a small shape: more
    sequences than one block of the plan kernel covers, and a chunks-per-segment pick that splits
    the long prompts into many short segments; every output and final state against the oracle."""
    _need_gpu()
    rng = random.Random(17)
    nb, P, N, Q, G, H = 260, 16, 16, 16, 1, 4
    lens = [rng.choice([0, 1, 5, 15, 16, 17, 40]) for _ in range(nb)]
    lens[3] = lens[200] = 640
    d = workloads.Dims(nb, max(lens), H * P // 2, 2, P, N, G, 4, Q, io)
    inp, x, b, c = tp._scan_inputs(d, 9990 + (io == "bf16"), True)
    s0 = inp.state0
    dims, tol = dims_of(d), tol_for(io)
    pack = lambda a: np.concatenate([a[i, :n] for i, n in enumerate(lens)], 0)
    xp, bp, cp, dtp = pack(x), pack(b), pack(c), pack(inp.dt_raw)
    T = len(xp)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    y = nan_like((T, H * P), io)
    s = torch.full((nb, H, P, N), float("nan"), device="cuda")
    m2.m2_ssd_scan_fwd_packed(dims, torch.as_tensor(cu, device="cuda"), dev(xp, io), dev(bp, io), dev(cp, io),
                              dev(dtp, io), dev32(inp.dt_bias), dev32(inp.A), dev32(inp.D), y, dev32(s0), s,
                              workspace=workspace(dims, T))
    torch.cuda.synchronize()
    yr, sr = oracle.ssd_scan_packed(xp, bp, cp, dtp, cu, inp.dt_bias, inp.A, inp.D, s0)
    errs = [oracle.max_rel_err(host(s), sr), oracle.max_rel_err(host(y).reshape(T, H, P), yr)]
    print("packed scan, %d prompts (%d tokens) %s: state %.2e y %.2e (bar %.0e)" % (nb, T, io, errs[0], errs[1], tol))
    assert max(errs) <= tol, errs


def _many_prompt_cases(seed=47, n=3):
    """12-40 prompts at 16-32 heads: enough chunks against the resident blocks that the packed scan
    picks its segment length on the device (padded and packed, through the one-pass test's body)."""
    rng, out = random.Random(seed), []
    for i in range(n):
        nb = rng.randint(12, 40)
        maxlen = rng.choice([600, 1000, 1500])
        lens = [rng.choice([0, 1, 3, 31, 33, 100, 257, maxlen // 2, maxlen]) for _ in range(nb)]
        d_model = rng.choice([512, 1024]) if nb <= 24 else 512
        groups = rng.choice([1, 2])
        out.append((lens, groups, d_model, rng.choice([2, 3, 4]), rng.random() < 0.7, rng.randint(0, 5), 30000 + i))
    return out


@pytest.mark.parametrize("case", _many_prompt_cases(), ids=lambda c: "n%d-G%d-dm%d" % (len(c[0]), c[1], c[2]))
def test_one_pass_prefill_many_prompts(case):
    test_random_one_pass_prefill(case)
