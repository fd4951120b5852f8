"""Pins for the fp64 oracle's scan backward (oracle.ssd_scan_bwd), independent of its own code.

The backward of the Zamba2 mixer's scan (article "Transformers 中 Zamba2 混合架构模型解析", §三:
the stateful mixer's training path) returns the gradients of
    L = sum_t dy_t . y_t + <dS, S_final>
for the recurrence S_t = exp(dt_t A) S_{t-1} + dt_t x_t (outer) B_t, y_t = S_t C_t + D x_t,
dt = clamp(softplus(dt_raw + dt_bias)).  The pins:
  - L is affine in x, B, C, D and the initial state, so L(v + e) - L(v) = <dv, e> holds exactly
    (up to rounding) for any direction e: checked with the forward oracle, which its own pins fix;
  - dt_raw, dt_bias and A enter nonlinearly: central finite differences of L, element by element
    on samples, including tokens the dt clamp holds (whose gradient must be zero);
  - A = 0 reduces the scan to causal linear attention; its gradients are written here as numpy
    matrix products from that closed form;
  - the backward of a prompt split in two calls, with the adjoint of the first call's final state
    taken from the second call's dstate_in, equals the backward of the whole prompt;
  - every gradient equals PyTorch's reverse-mode autograd (fp64, CPU) through the token recurrence
    written out with torch ops, with and without a clamp.
"""
import numpy as np
import pytest

import oracle


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def case(seed, Bn=2, L=23, H=4, P=5, N=3, G=2, state=True):
    r = np.random.default_rng(seed)
    c = dict(x=r.normal(size=(Bn, L, H, P)), Bm=r.normal(size=(Bn, L, G, N)) / np.sqrt(N),
             Cm=r.normal(size=(Bn, L, G, N)) / np.sqrt(N), dt_raw=r.normal(size=(Bn, L, H)),
             dt_bias=r.uniform(-3, -1, H), A=-np.exp(r.uniform(0, np.log(16), H)), D=r.normal(size=H),
             state_in=r.normal(size=(Bn, H, P, N)) * 0.5 if state else None)
    dy = r.normal(size=(Bn, L, H, P))
    dS = r.normal(size=(Bn, H, P, N))
    return c, dy, dS, r


def loss(c, dy, dS, **over):
    a = dict(c)
    a.update(over)
    y, s = oracle.ssd_scan(**a)
    return float((y * dy).sum() + (s * dS).sum())


@pytest.mark.parametrize("name,grad", [("x", "dx"), ("Bm", "dB"), ("Cm", "dC"), ("D", "dD"),
                                       ("state_in", "dstate_in")])
def test_affine_inputs_exact_directional_derivative(name, grad):
    c, dy, dS, r = case(1)
    g = oracle.ssd_scan_bwd(**c, dy=dy, dstate_out=dS)
    for k in range(3):
        e = r.normal(size=np.shape(c[name]))
        lhs = loss(c, dy, dS, **{name: c[name] + e}) - loss(c, dy, dS)
        rhs = float((g[grad] * e).sum())
        assert lhs == pytest.approx(rhs, rel=1e-9, abs=1e-9), (name, k, lhs, rhs)


def _central(f, v, idx, h):
    e = np.zeros_like(v)
    e[idx] = h
    return (f(v + e) - f(v - e)) / (2 * h)


def test_dt_raw_by_central_differences():
    c, dy, dS, r = case(2)
    g = oracle.ssd_scan_bwd(**c, dy=dy, dstate_out=dS)
    f = lambda v: loss(c, dy, dS, dt_raw=v)
    idxs = [tuple(r.integers(0, s) for s in c["dt_raw"].shape) for _ in range(24)] + [(0, 0, 0), (1, 22, 3)]
    scale = np.abs(g["ddt_raw"]).max()
    for idx in idxs:
        fd = _central(f, c["dt_raw"], idx, 1e-5)
        assert abs(fd - g["ddt_raw"][idx]) <= 1e-7 * scale, (idx, fd, g["ddt_raw"][idx])


def test_dt_bias_and_A_by_central_differences():
    c, dy, dS, _ = case(3)
    g = oracle.ssd_scan_bwd(**c, dy=dy, dstate_out=dS)
    for name, grad in (("dt_bias", "ddt_bias"), ("A", "dA")):
        f = lambda v: loss(c, dy, dS, **{name: v})
        for h in range(c[name].shape[0]):
            fd = _central(f, c[name], (h,), 1e-6)
            assert fd == pytest.approx(g[grad][h], rel=1e-6, abs=1e-8 * np.abs(g[grad]).max()), (name, h)


def test_clamped_tokens_have_zero_dt_gradient_and_the_rest_match_differences():
    c, dy, dS, r = case(4)
    sp = np.logaddexp(0.0, c["dt_raw"] + c["dt_bias"])
    lo, hi = np.quantile(sp, 0.25), np.quantile(sp, 0.75)
    g = oracle.ssd_scan_bwd(**c, dy=dy, dstate_out=dS, dt_min=lo, dt_max=hi)
    clamped = (sp < lo) | (sp > hi)
    assert clamped.sum() > 10 and np.all(g["ddt_raw"][clamped] == 0.0)
    f = lambda v: loss(dict(c, dt_min=lo, dt_max=hi), dy, dS, dt_raw=v)
    free = np.argwhere(~clamped & (np.abs(sp - lo) > 1e-3) & (np.abs(sp - hi) > 1e-3))
    scale = np.abs(g["ddt_raw"]).max()
    for idx in map(tuple, free[r.choice(len(free), 16, replace=False)]):
        fd = _central(f, c["dt_raw"], idx, 1e-6)
        assert abs(fd - g["ddt_raw"][idx]) <= 1e-6 * scale, idx


def test_zero_decay_is_causal_linear_attention():
    """A = 0: S_t = S_0 + sum_{s<=t} dt_s x_s B_s^T, so per (sequence, head) with K[t,s] = dt_s C_t.B_s
    (s <= t):  y = K X + C S_0^T + D X  and  S_final = S_0 + X^T diag(dt) B.  Then, with
    M[t,s] = dt_s dY_t.X_s (s <= t):
        dX = K^T dY + D dY + diag(dt) B dS^T          dC = dY S_0 + M B
        dB = M^T C + diag(dt) X dS                    dS_0 = dY^T C + dS
        d(dt)_s = sum_{t>=s} (C_t.B_s)(dY_t.X_s) + X_s . dS B_s   (no decay term at A = 0)"""
    c, dy, dS, _ = case(5, Bn=2, L=17, H=4, P=3, N=5, G=2)
    c["A"] = np.zeros_like(c["A"])
    g = oracle.ssd_scan_bwd(**c, dy=dy, dstate_out=dS)
    Bn, L, H, P = c["x"].shape
    G, N = c["Bm"].shape[2:]
    dt = np.logaddexp(0.0, c["dt_raw"] + c["dt_bias"])
    mask = np.tril(np.ones((L, L)))
    dB = np.zeros_like(c["Bm"])
    dC = np.zeros_like(c["Cm"])
    for b in range(Bn):
        for h in range(H):
            gi = h // (H // G)
            X, dY, Bg, Cg, d = c["x"][b, :, h], dy[b, :, h], c["Bm"][b, :, gi], c["Cm"][b, :, gi], dt[b, :, h]
            S0, dSh = c["state_in"][b, h], dS[b, h]
            K = (Cg @ Bg.T) * d[None, :] * mask
            dX = K.T @ dY + c["D"][h] * dY + d[:, None] * (Bg @ dSh.T)
            assert rel(g["dx"][b, :, h], dX) < 1e-12
            Mx = (dY @ X.T) * d[None, :] * mask
            dC[b, :, gi] += dY @ S0 + Mx @ Bg
            dB[b, :, gi] += Mx.T @ Cg + d[:, None] * (X @ dSh)
            assert rel(g["dstate_in"][b, h], dY.T @ Cg + dSh) < 1e-12
            # d(dt_s) at A = 0: only the factor dt_s of token s's input; the decay has no dt term
            ddt = ((Cg @ Bg.T) * (dY @ X.T) * mask).sum(axis=0) + np.einsum("sp,pn,sn->s", X, dSh, Bg)
            sig = 1.0 / (1.0 + np.exp(-(c["dt_raw"][b, :, h] + c["dt_bias"][h])))
            assert rel(g["ddt_raw"][b, :, h], ddt * sig) < 1e-12
    assert rel(g["dB"], dB) < 1e-12 and rel(g["dC"], dC) < 1e-12
    assert rel(g["dD"], np.einsum("blhp,blhp->h", dy, c["x"])) < 1e-12


def test_split_prompt_backward_equals_whole():
    c, dy, dS, _ = case(6, L=29)
    whole = oracle.ssd_scan_bwd(**c, dy=dy, dstate_out=dS)
    L1 = 11
    first = {k: (v[:, :L1] if k in ("x", "Bm", "Cm", "dt_raw") else v) for k, v in c.items()}
    _, mid = oracle.ssd_scan(**first)
    second = {k: (v[:, L1:] if k in ("x", "Bm", "Cm", "dt_raw") else v) for k, v in c.items()}
    second["state_in"] = mid
    g2 = oracle.ssd_scan_bwd(**second, dy=dy[:, L1:], dstate_out=dS)
    g1 = oracle.ssd_scan_bwd(**first, dy=dy[:, :L1], dstate_out=g2["dstate_in"])
    for k in ("dx", "dB", "dC", "ddt_raw"):
        assert rel(np.concatenate([g1[k], g2[k]], axis=1), whole[k]) < 1e-11, k
    for k in ("ddt_bias", "dA", "dD"):
        assert rel(g1[k] + g2[k], whole[k]) < 1e-11, k
    assert rel(g1["dstate_in"], whole["dstate_in"]) < 1e-11


def test_no_initial_state_and_no_final_adjoint():
    c, dy, dS, _ = case(7, state=False)
    g = oracle.ssd_scan_bwd(**c, dy=dy)
    zero = dict(c, state_in=np.zeros((2, 4, 5, 3)))
    g0 = oracle.ssd_scan_bwd(**zero, dy=dy, dstate_out=np.zeros_like(dS))
    for k in g:
        assert np.array_equal(g[k], g0[k]), k


@pytest.mark.parametrize("clamp", [False, True], ids=["no-clamp", "clamp"])
def test_matches_autograd_of_the_token_recurrence(clamp):
    """Every gradient, the nonlinear ones (dt_raw, dt_bias, A) included, against PyTorch's reverse-mode
    autograd in fp64 on the CPU, run through the token recurrence written out here with torch ops
    (S_t = e^(dt_t A) S_{t-1} + dt_t x_t B_t^T, y_t = S_t C_t + D x_t, dt = clamp(softplus(dt_raw +
    dt_bias))): an independent differentiation, exact up to rounding.  With the clamp, its bounds are
    set between token values so that no token sits on one (where the derivative is a convention)."""
    torch = pytest.importorskip("torch")
    c, dy, dS, _ = case(8, Bn=2, L=19, H=4, P=3, N=5, G=2)
    lo, hi = 0.0, float("inf")
    if clamp:
        sp = np.sort(np.logaddexp(0.0, c["dt_raw"] + c["dt_bias"]).ravel())
        lo, hi = (sp[30] + sp[31]) / 2, (sp[-31] + sp[-30]) / 2
    g = oracle.ssd_scan_bwd(**c, dy=dy, dstate_out=dS, dt_min=lo, dt_max=hi)
    T = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in c.items() if v is not None}
    Bn, L, H, P = c["x"].shape
    G = c["Bm"].shape[2]
    dt = torch.nn.functional.softplus(T["dt_raw"] + T["dt_bias"], beta=1.0, threshold=1e30)
    if clamp:
        dt = torch.clamp(dt, lo, hi)
    S = T["state_in"]
    loss = torch.zeros((), dtype=torch.float64)
    hg = torch.arange(H) // (H // G)
    for t in range(L):
        a = torch.exp(dt[:, t] * T["A"])                                   # [Bn, H]
        Bt, Ct = T["Bm"][:, t][:, hg], T["Cm"][:, t][:, hg]                # [Bn, H, N]
        S = a[..., None, None] * S + (dt[:, t][..., None] * T["x"][:, t])[..., None] * Bt[:, :, None, :]
        y = (S * Ct[:, :, None, :]).sum(-1) + T["D"][None, :, None] * T["x"][:, t]
        loss = loss + (y * torch.tensor(dy[:, t])).sum()
    loss = loss + (S * torch.tensor(dS)).sum()
    loss.backward()
    pairs = {"dx": "x", "dB": "Bm", "dC": "Cm", "ddt_raw": "dt_raw", "ddt_bias": "dt_bias", "dA": "A",
             "dD": "D", "dstate_in": "state_in"}
    for gk, ck in pairs.items():
        assert rel(g[gk], T[ck].grad.numpy()) < 1e-12, (gk, rel(g[gk], T[ck].grad.numpy()))


def test_right_padded_batch_equals_each_sequence_alone():
    """Right padding (a per-sequence length, the reading the forward oracle follows): the backward of a
    padded batch, with dstate_out the adjoint of the state after each sequence's last real token, equals
    the backward of each sequence's real tokens alone (the case every pin above fixes), including an
    empty sequence (dstate_in = dstate_out) and a full one; the per-token gradients past a length are
    left unwritten, and junk in the padded positions changes nothing."""
    c, dy, dS, r = case(9, Bn=4, L=21, H=4, P=3, N=5, G=2)
    lens = np.array([21, 13, 0, 1])
    junk = dict(c)
    dyj = dy.copy()
    for b, n in enumerate(lens):
        for k in ("x", "Bm", "Cm", "dt_raw"):
            junk[k] = junk[k].copy()
            junk[k][b, n:] = r.normal(size=junk[k][b, n:].shape) * 7.0
        dyj[b, n:] = r.normal(size=dyj[b, n:].shape) * 7.0
    g = oracle.ssd_scan_bwd(**junk, dy=dyj, dstate_out=dS, seq_lens=lens)
    sums = {k: np.zeros_like(g[k]) for k in ("ddt_bias", "dA", "dD")}
    for b, n in enumerate(lens):
        one = {k: (v[b:b + 1, :n] if k in ("x", "Bm", "Cm", "dt_raw") else v) for k, v in c.items()}
        one["state_in"] = c["state_in"][b:b + 1]
        gb = oracle.ssd_scan_bwd(**one, dy=dy[b:b + 1, :n], dstate_out=dS[b:b + 1])
        for k in ("dx", "dB", "dC", "ddt_raw"):
            assert rel(g[k][b, :n], gb[k][0]) < 1e-12 if n else True, (k, b)
            assert np.isnan(g[k][b, n:]).all(), (k, b)
        assert rel(g["dstate_in"][b], gb["dstate_in"][0]) < 1e-12, b
        for k in sums:
            sums[k] += gb[k]
    assert np.array_equal(g["dstate_in"][2], dS[2]), "an empty sequence passes dstate_out through"
    for k in sums:
        assert rel(g[k], sums[k]) < 1e-12, k


def test_packed_batch_matches_derivatives_of_the_packed_forward():
    """Packed batches (sequences back to back, each scanned on its own from its own state): the
    gradients of L = sum dy . y + <dS, state_out> over the packed forward oracle, with an empty
    sequence, a one-token one and two longer ones.  L is affine in x, B, C and the initial states, so
    one step along a random direction gives the exact directional derivative; d(raw dt) and
    dt_bias by central differences, sampled at each sequence's first and last tokens (a gradient that
    leaked across a sequence boundary would show there)."""
    r = np.random.default_rng(12)
    lens = [7, 0, 1, 11]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, P, N, G = int(cu[-1]), 4, 3, 5, 2
    c = dict(x=r.normal(size=(T, H, P)), Bm=r.normal(size=(T, G, N)) / np.sqrt(N),
             Cm=r.normal(size=(T, G, N)) / np.sqrt(N), dt_raw=r.normal(size=(T, H)),
             dt_bias=r.uniform(-3, -1, H), A=-np.exp(r.uniform(0, np.log(16), H)), D=r.normal(size=H),
             state_in=r.normal(size=(len(lens), H, P, N)) * 0.5)
    dy = r.normal(size=(T, H, P))
    dS = r.normal(size=(len(lens), H, P, N))

    def L(**over):
        a = dict(c)
        a.update(over)
        y, s = oracle.ssd_scan_packed(cu_seqlens=cu, **a)
        return float((y * dy).sum() + (s * dS).sum())

    g = oracle.ssd_scan_bwd_packed(cu_seqlens=cu, **c, dy=dy, dstate_out=dS)
    assert np.array_equal(g["dstate_in"][1], dS[1]), "an empty sequence passes dstate_out through"
    for name, grad in (("x", "dx"), ("Bm", "dB"), ("Cm", "dC"), ("state_in", "dstate_in"), ("D", "dD")):
        e = r.normal(size=np.shape(c[name]))
        lhs = L(**{name: c[name] + e}) - L()
        assert lhs == pytest.approx(float((g[grad] * e).sum()), rel=1e-9, abs=1e-9), name
    for t in (0, 6, 7, 8, 18):
        for h in (0, 3):
            num = _central(lambda v: L(dt_raw=v), c["dt_raw"], (t, h), 1e-5)
            assert num == pytest.approx(g["ddt_raw"][t, h], rel=1e-5, abs=1e-7), (t, h)
    for h in range(H):
        num = _central(lambda v: L(dt_bias=v), c["dt_bias"], (h,), 1e-5)
        assert num == pytest.approx(g["ddt_bias"][h], rel=1e-5, abs=1e-7), h
