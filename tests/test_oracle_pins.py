"""Pins for the fp64 oracle, independent of the oracle's own code.

Each test checks the oracle against something other than itself: a library
routine (numpy.logaddexp, numpy.convolve, scipy.signal.lfilter,
scipy.special.expit), a closed form, a brute-force unrolled sum written
here from the mathematics, or an invariant the recurrence must satisfy.
The steps being pinned are those of the Zamba2 mixer (article "Transformers 中
Zamba2 混合架构模型解析", §三: conv1d of width mamba_d_conv + SiLU, then the
chunked scan or the single-token state update), with the selective
state-space recurrence S_t = exp(dt_t A) S_{t-1} + dt_t x_t (outer) B_t,
y_t = S_t C_t + D x_t and dt = softplus(dt_raw + dt_bias).
"""
import numpy as np
import pytest
import scipy.signal
import scipy.special

import oracle

RTOL = 1e-12


def silu(v):
    return v * scipy.special.expit(v)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ----------------------------------------------------------------- softplus / dt

def test_softplus_matches_logaddexp():
    for v in np.concatenate([np.linspace(-50, 50, 1001), [-700.0, -30.0, 30.0, 29.9, 30.1, 700.0]]):
        assert oracle.softplus(v) == pytest.approx(np.logaddexp(0.0, v), rel=1e-14, abs=1e-300)


def test_scan_applies_softplus_to_raw_plus_bias():
    # one token, P = N = 1, x = B = C = 1, D = 0: y_0 = dt_0 = softplus(raw + bias)
    raws = np.array([-3.0, 0.0, 0.7, 5.0])
    for raw in raws:
        for bias in (-4.0, -2.5, 1.0):
            y, s = oracle.ssd_scan(np.ones((1, 1, 1, 1)), np.ones((1, 1, 1, 1)), np.ones((1, 1, 1, 1)),
                                   np.full((1, 1, 1), raw), np.array([bias]), np.array([-1.0]))
            want = np.logaddexp(0.0, raw + bias)
            assert y[0, 0, 0, 0] == pytest.approx(want, rel=1e-14)
            assert s[0, 0, 0, 0] == pytest.approx(want, rel=1e-14)


def test_dt_clamp():
    # softplus(-10) ~ 4.5e-5 is raised to dt_min; softplus(3) ~ 3.05 is cut to dt_max
    one = np.ones((1, 1, 1, 1))
    y, _ = oracle.ssd_scan(one, one, one, np.full((1, 1, 1), -10.0), np.array([0.0]), np.array([-1.0]),
                           dt_min=1e-4)
    assert y[0, 0, 0, 0] == pytest.approx(1e-4, rel=1e-14)
    y, _ = oracle.ssd_scan(one, one, one, np.full((1, 1, 1), 3.0), np.array([0.0]), np.array([-1.0]),
                           dt_max=0.5)
    assert y[0, 0, 0, 0] == pytest.approx(0.5, rel=1e-14)


# ----------------------------------------------------------------- conv1d + SiLU

@pytest.mark.parametrize("W", [2, 3, 4])
def test_conv_impulse_reproduces_taps_in_order(W):
    # impulse at t0: the pre-activation at t0 + d is tap W-1-d (the last tap sees the current token)
    L, Cd, t0 = 12, 3, 5
    rng = np.random.default_rng(1)
    w = rng.uniform(-1, 1, (Cd, W))
    x = np.zeros((1, L, Cd))
    x[0, t0, :] = 1.0
    out, _ = oracle.conv1d(x, w, np.zeros(Cd))
    want_pre = np.zeros((L, Cd))
    for d in range(W):
        want_pre[t0 + d] = w[:, W - 1 - d]
    np.testing.assert_allclose(out[0], silu(want_pre), rtol=1e-14, atol=1e-300)


def test_conv_matches_numpy_convolve_and_lfilter():
    rng = np.random.default_rng(2)
    Bn, L, Cd, W = 2, 37, 5, 4
    x = rng.standard_normal((Bn, L, Cd))
    w = rng.uniform(-0.5, 0.5, (Cd, W))
    bias = rng.uniform(-0.5, 0.5, Cd)
    out, ring = oracle.conv1d(x, w, bias)
    for b in range(Bn):
        for c in range(Cd):
            pre = np.convolve(x[b, :, c], w[c, ::-1])[:L] + bias[c]
            np.testing.assert_allclose(out[b, :, c], silu(pre), rtol=1e-13, atol=1e-15)
            pre2 = scipy.signal.lfilter(w[c, ::-1], [1.0], x[b, :, c]) + bias[c]
            np.testing.assert_allclose(out[b, :, c], silu(pre2), rtol=1e-13, atol=1e-15)
    # ring at phase 0: slot j holds token L-W+j
    np.testing.assert_array_equal(ring, x[:, L - W:, :])


@pytest.mark.parametrize("phase", [0, 1, 2, 3, 6])
def test_conv_history_from_ring(phase):
    # conv with history == conv of [history tokens, x] with the history part dropped
    rng = np.random.default_rng(3)
    Bn, L, Cd, W = 2, 9, 4, 4
    hist = rng.standard_normal((Bn, W - 1, Cd))     # tokens -3, -2, -1
    x = rng.standard_normal((Bn, L, Cd))
    w = rng.uniform(-0.5, 0.5, (Cd, W))
    bias = rng.uniform(-0.5, 0.5, Cd)
    ring = rng.standard_normal((Bn, W, Cd))        # dead slot keeps junk
    for j in range(1, W):                          # token -j lives in slot (phase - j) mod W
        ring[:, (phase - j) % W, :] = hist[:, W - 1 - j, :]
    out, ring_out = oracle.conv1d(x, w, bias, ring, phase)
    full = np.concatenate([hist, x], axis=1)
    ref, _ = oracle.conv1d(full, w, bias)
    np.testing.assert_allclose(out, ref[:, W - 1:], rtol=1e-14, atol=1e-300)
    np.testing.assert_array_equal(ring_out, full[:, -W:, :])


def test_conv_short_prompt_ring_takes_history():
    rng = np.random.default_rng(4)
    Bn, Cd, W = 1, 3, 4
    hist = rng.standard_normal((Bn, W, Cd))        # phase 0 ring: slot j = token j - W
    x = rng.standard_normal((Bn, 2, Cd))
    w = rng.uniform(-0.5, 0.5, (Cd, W))
    _, ring_out = oracle.conv1d(x, w, None, hist, 0)
    seq = np.concatenate([hist[:, 1:], x], axis=1)  # tokens -3..1
    np.testing.assert_array_equal(ring_out, seq[:, -W:])


def test_conv_split_invariance():
    rng = np.random.default_rng(5)
    Bn, L, Cd, W = 2, 40, 6, 4
    x = rng.standard_normal((Bn, L, Cd))
    w = rng.uniform(-0.5, 0.5, (Cd, W))
    bias = rng.uniform(-0.5, 0.5, Cd)
    whole, ring_whole = oracle.conv1d(x, w, bias)
    for k in (1, 3, 4, 17):
        a, ring_a = oracle.conv1d(x[:, :k], w, bias)
        b, ring_b = oracle.conv1d(x[:, k:], w, bias, ring_a, 0)
        np.testing.assert_allclose(np.concatenate([a, b], 1), whole, rtol=1e-14, atol=1e-300)
        np.testing.assert_array_equal(ring_b, ring_whole)


# ----------------------------------------------------------------- scan recurrence

def _rand_scan(rng, Bn, L, H, P, N, G, with_state=True):
    x = rng.standard_normal((Bn, L, H, P))
    Bm = rng.standard_normal((Bn, L, G, N)) / np.sqrt(N)
    Cm = rng.standard_normal((Bn, L, G, N)) / np.sqrt(N)
    dt_raw = rng.standard_normal((Bn, L, H))
    dt_bias = rng.uniform(-4, -2, H) + 2.0    # larger dt so that decay matters at small L
    A = -np.exp(rng.uniform(0, np.log(16), H))
    D = rng.standard_normal(H)
    S0 = 0.3 * rng.standard_normal((Bn, H, P, N)) if with_state else None
    return x, Bm, Cm, dt_raw, dt_bias, A, D, S0


def _bruteforce(x, Bm, Cm, dt_raw, dt_bias, A, D, S0):
    """Quadratic (dual) form: every output as an explicit sum over earlier tokens.

    y_t = exp(A sum_{r<=t} dt_r) (S0 C_t) + sum_{s<=t} exp(A sum_{s<r<=t} dt_r) dt_s (C_t.B_s) x_s + D x_t
    S_L = exp(A sum_r dt_r) S0 + sum_s exp(A sum_{r>s} dt_r) dt_s x_s (outer) B_s
    """
    Bn, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    y = np.zeros_like(x)
    S = np.zeros((Bn, H, P, N))
    for b in range(Bn):
        for h in range(H):
            g = h // (H // G)
            dt = np.logaddexp(0.0, dt_raw[b, :, h] + dt_bias[h])
            for t in range(L):
                acc = np.exp(A[h] * dt[: t + 1].sum()) * (S0[b, h] @ Cm[b, t, g]) if S0 is not None else 0.0
                for s in range(t + 1):
                    acc = acc + np.exp(A[h] * dt[s + 1: t + 1].sum()) * dt[s] * (Cm[b, t, g] @ Bm[b, s, g]) * x[b, s, h]
                y[b, t, h] = acc + D[h] * x[b, t, h]
            St = np.exp(A[h] * dt.sum()) * S0[b, h] if S0 is not None else np.zeros((P, N))
            for s in range(L):
                St = St + np.exp(A[h] * dt[s + 1:].sum()) * dt[s] * np.outer(x[b, s, h], Bm[b, s, g])
            S[b, h] = St
    return y, S


@pytest.mark.parametrize("shape", [(2, 24, 4, 3, 5, 2), (1, 17, 2, 4, 4, 1), (1, 1, 3, 2, 3, 3)])
def test_scan_matches_bruteforce(shape):
    rng = np.random.default_rng(10)
    args = _rand_scan(rng, *shape)
    y, s = oracle.ssd_scan(*args[:7], state_in=args[7])
    yb, sb = _bruteforce(*args)
    assert rel(y, yb) < RTOL
    assert rel(s, sb) < RTOL


def test_scan_matches_bruteforce_zero_state_no_D():
    rng = np.random.default_rng(11)
    x, Bm, Cm, dt_raw, dt_bias, A, D, _ = _rand_scan(rng, 1, 20, 2, 3, 4, 1, with_state=False)
    y, s = oracle.ssd_scan(x, Bm, Cm, dt_raw, dt_bias, A, None, None)
    yb, sb = _bruteforce(x, Bm, Cm, dt_raw, dt_bias, A, np.zeros_like(D), None)
    assert rel(y, yb) < RTOL and rel(s, sb) < RTOL


def test_scan_constant_dt_matches_lfilter():
    # constant dt, A: each state entry is a first-order IIR driven by u_t = dt x_t[p] B_t[n]
    rng = np.random.default_rng(12)
    L, P, N = 50, 3, 4
    x = rng.standard_normal((1, L, 1, P))
    Bm = rng.standard_normal((1, L, 1, N))
    Cm = rng.standard_normal((1, L, 1, N))
    raw, bias, A, D = 0.3, -1.0, -2.5, 0.7
    S0 = rng.standard_normal((1, 1, P, N))
    y, s = oracle.ssd_scan(x, Bm, Cm, np.full((1, L, 1), raw), np.array([bias]), np.array([A]),
                           np.array([D]), S0)
    dt = np.logaddexp(0.0, raw + bias)
    lam = np.exp(dt * A)
    S = np.zeros((L, P, N))
    for p in range(P):
        for n in range(N):
            u = x[0, :, 0, p] * Bm[0, :, 0, n]
            S[:, p, n] = scipy.signal.lfilter([dt], [1.0, -lam], u) + lam ** np.arange(1, L + 1) * S0[0, 0, p, n]
    yref = np.einsum("tpn,tn->tp", S, Cm[0, :, 0]) + D * x[0, :, 0]
    assert rel(y[0, :, 0], yref) < 1e-12
    assert rel(s[0, 0], S[-1]) < 1e-12


def test_scan_constant_inputs_closed_form():
    # constant dt, x, B: S_t = lam^(t+1) S0 + dt x B^T (1 - lam^(t+1)) / (1 - lam), lam = exp(dt A)
    L, P, N = 300, 2, 3
    xv = np.array([0.5, -1.5])
    bv = np.array([1.0, 2.0, -0.5])
    cv = np.array([0.3, -0.2, 0.9])
    raw, bias, A, D = 0.0, 0.0, -0.75, 0.25
    S0 = np.arange(P * N, dtype=np.float64).reshape(1, 1, P, N) / 7.0
    x = np.broadcast_to(xv, (1, L, 1, P)).copy()
    Bm = np.broadcast_to(bv, (1, L, 1, N)).copy()
    Cm = np.broadcast_to(cv, (1, L, 1, N)).copy()
    y, s = oracle.ssd_scan(x, Bm, Cm, np.full((1, L, 1), raw), np.array([bias]), np.array([A]),
                           np.array([D]), S0)
    dt = np.log(2.0)
    lam = np.exp(dt * A)
    for t in (0, 1, 7, L - 1):
        St = lam ** (t + 1) * S0[0, 0] + dt * np.outer(xv, bv) * (1 - lam ** (t + 1)) / (1 - lam)
        np.testing.assert_allclose(y[0, t, 0], St @ cv + D * xv, rtol=1e-12, atol=1e-14)
    steady = dt * np.outer(xv, bv) / (1 - lam)
    np.testing.assert_allclose(s[0, 0], steady, rtol=1e-12)


def test_scan_A_zero_is_causal_linear_attention():
    # A = 0: no decay, y = tril(C B^T) (dt * X) + D X
    rng = np.random.default_rng(13)
    L, P, N = 33, 4, 6
    x, Bm, Cm, dt_raw, dt_bias, _, D, _ = _rand_scan(rng, 1, L, 1, P, N, 1, with_state=False)
    y, _ = oracle.ssd_scan(x, Bm, Cm, dt_raw, dt_bias, np.zeros(1), D)
    dt = np.logaddexp(0.0, dt_raw[0, :, 0] + dt_bias[0])
    M = np.tril(Cm[0, :, 0] @ Bm[0, :, 0].T)
    yref = M @ (dt[:, None] * x[0, :, 0]) + D[0] * x[0, :, 0]
    assert rel(y[0, :, 0], yref) < 1e-12


def test_scan_strong_decay_is_memoryless():
    rng = np.random.default_rng(14)
    L, P, N = 16, 3, 4
    x, Bm, Cm, dt_raw, dt_bias, _, D, S0 = _rand_scan(rng, 1, L, 1, P, N, 1)
    y, s = oracle.ssd_scan(x, Bm, Cm, dt_raw, np.array([3.0]), np.array([-1e5]), D, S0)
    dt = np.logaddexp(0.0, dt_raw[0, :, 0] + 3.0)
    yref = dt[:, None] * np.einsum("tn,tn->t", Cm[0, :, 0], Bm[0, :, 0])[:, None] * x[0, :, 0] + D[0] * x[0, :, 0]
    np.testing.assert_allclose(y[0, :, 0], yref, rtol=1e-12, atol=1e-14)


def test_scan_scalar_by_hand():
    # P = N = 1, three tokens, written out by hand
    x = np.array([1.0, 2.0, -1.0]).reshape(1, 3, 1, 1)
    Bm = np.array([0.5, 1.0, 2.0]).reshape(1, 3, 1, 1)
    Cm = np.array([1.0, -1.0, 0.5]).reshape(1, 3, 1, 1)
    raw = np.array([0.0, 1.0, -1.0]).reshape(1, 3, 1)
    A, D, s0 = -0.5, 2.0, 0.25
    y, s = oracle.ssd_scan(x, Bm, Cm, raw, np.array([0.0]), np.array([A]), np.array([D]),
                           np.array([[[[s0]]]]))
    S = s0
    want = []
    for t in range(3):
        dt = np.log1p(np.exp(raw[0, t, 0]))
        S = np.exp(dt * A) * S + dt * x[0, t, 0, 0] * Bm[0, t, 0, 0]
        want.append(S * Cm[0, t, 0, 0] + D * x[0, t, 0, 0])
    np.testing.assert_allclose(y[0, :, 0, 0], want, rtol=1e-14)
    assert s[0, 0, 0, 0] == pytest.approx(S, rel=1e-14)


# ----------------------------------------------------------------- invariants

def test_scan_causality():
    rng = np.random.default_rng(20)
    args = list(_rand_scan(rng, 1, 30, 2, 3, 4, 1))
    y0, _ = oracle.ssd_scan(*args[:7], state_in=args[7])
    for t in (0, 11, 29):
        pert = [a.copy() for a in args]
        pert[0][0, t] += 1.0       # x
        pert[1][0, t] += 1.0       # B
        pert[2][0, t] += 1.0       # C
        pert[3][0, t] += 1.0       # dt_raw
        y1, _ = oracle.ssd_scan(*pert[:7], state_in=pert[7])
        np.testing.assert_array_equal(y1[0, :t], y0[0, :t])
        assert np.all(y1[0, t] != y0[0, t])


def test_scan_linearity_and_superposition():
    rng = np.random.default_rng(21)
    x, Bm, Cm, dt_raw, dt_bias, A, D, S0 = _rand_scan(rng, 2, 25, 2, 3, 4, 1)
    x2 = rng.standard_normal(x.shape)
    ya, sa = oracle.ssd_scan(x, Bm, Cm, dt_raw, dt_bias, A, D, None)
    yb, sb = oracle.ssd_scan(x2, Bm, Cm, dt_raw, dt_bias, A, D, None)
    yc, sc = oracle.ssd_scan(2.0 * x - 3.0 * x2, Bm, Cm, dt_raw, dt_bias, A, D, None)
    assert rel(yc, 2 * ya - 3 * yb) < 1e-12 and rel(sc, 2 * sa - 3 * sb) < 1e-12
    # initial-state part and input part add up
    y0, s0 = oracle.ssd_scan(np.zeros_like(x), Bm, Cm, dt_raw, dt_bias, A, D, S0)
    yf, sf = oracle.ssd_scan(x, Bm, Cm, dt_raw, dt_bias, A, D, S0)
    assert rel(yf, ya + y0) < 1e-12 and rel(sf, sa + s0) < 1e-12


def test_scan_head_and_batch_permutation():
    rng = np.random.default_rng(22)
    x, Bm, Cm, dt_raw, dt_bias, A, D, S0 = _rand_scan(rng, 3, 12, 4, 2, 3, 2)
    y, s = oracle.ssd_scan(x, Bm, Cm, dt_raw, dt_bias, A, D, S0)
    hp = np.array([1, 0, 3, 2])   # swap heads within each group (2 heads per group)
    bp = np.array([2, 0, 1])
    y2, s2 = oracle.ssd_scan(x[bp][:, :, hp], Bm[bp], Cm[bp], dt_raw[bp][:, :, hp], dt_bias[hp], A[hp], D[hp],
                             S0[bp][:, hp])
    np.testing.assert_allclose(y2, y[bp][:, :, hp], rtol=1e-15, atol=0)
    np.testing.assert_allclose(s2, s[bp][:, hp], rtol=1e-15, atol=0)


def test_scan_split_prefill_invariance():
    # chunked prefill == whole prefill (the test the Zamba2 article lists in §七)
    rng = np.random.default_rng(23)
    x, Bm, Cm, dt_raw, dt_bias, A, D, S0 = _rand_scan(rng, 2, 40, 2, 3, 4, 1)
    y, s = oracle.ssd_scan(x, Bm, Cm, dt_raw, dt_bias, A, D, S0)
    for k in (1, 13, 39):
        ya, sa = oracle.ssd_scan(x[:, :k], Bm[:, :k], Cm[:, :k], dt_raw[:, :k], dt_bias, A, D, S0)
        yb, sb = oracle.ssd_scan(x[:, k:], Bm[:, k:], Cm[:, k:], dt_raw[:, k:], dt_bias, A, D, sa)
        assert rel(np.concatenate([ya, yb], 1), y) < 1e-13
        assert rel(sb, s) < 1e-13


# ----------------------------------------------------------------- decode step

def _rand_step(rng, Bn, H, P, N, G, W, L):
    Cd = H * P + 2 * G * N
    xbc = rng.standard_normal((Bn, L, Cd))
    dt_raw = rng.standard_normal((Bn, L, H))
    w = rng.uniform(-0.5, 0.5, (Cd, W))
    bias = rng.uniform(-0.5, 0.5, Cd)
    dt_bias = rng.uniform(-4, -2, H)
    A = -np.exp(rng.uniform(0, np.log(16), H))
    D = rng.standard_normal(H)
    ring0 = 0.1 * rng.standard_normal((Bn, W, Cd))
    S0 = 0.1 * rng.standard_normal((Bn, H, P, N))
    return xbc, dt_raw, w, bias, dt_bias, A, D, ring0, S0


@pytest.mark.parametrize("dims", [(2, 4, 3, 5, 2, 4), (1, 2, 2, 2, 1, 3), (3, 1, 1, 1, 1, 2)])
def test_step_chain_equals_prefill(dims):
    # the token-by-token path must equal the chunked prompt path (article §七)
    Bn, H, P, N, G, W = dims
    L = 11
    rng = np.random.default_rng(30)
    xbc, dt_raw, w, bias, dt_bias, A, D, ring0, S0 = _rand_step(rng, Bn, H, P, N, G, W, L)
    y_pre, s_pre, ring_pre, _ = oracle.mixer_prefill(xbc, dt_raw, w, bias, dt_bias, A, D, H, P, N, G,
                                                     ring0, 0, S0)
    ring, S = ring0, S0
    ys = []
    for t in range(L):
        y, ring, S = oracle.ssd_step(xbc[:, t], dt_raw[:, t], w, bias, dt_bias, A, D, ring, t, S, H, P, N, G)
        ys.append(y)
    ys = np.stack(ys, 1).reshape(Bn, L, H, P)
    assert rel(ys, y_pre) < 1e-13
    assert rel(S, s_pre) < 1e-13
    # the chain's ring is at phase L; the prefill's at phase 0: token -j in slot (L-j)%W vs W-j
    for j in range(1, W + 1):
        np.testing.assert_array_equal(ring[:, (L - j) % W], ring_pre[:, W - j])


def test_step_scalar_by_hand():
    # H = P = N = 1, G = 1, W = 2: channels (x, B, C)
    w = np.array([[0.5, 1.0], [1.0, -1.0], [2.0, 0.25]])
    bias = np.array([0.1, 0.0, -0.2])
    # phase 1: token -1 sits in slot (1-1) % 2 = 0; slot 1 is dead and receives the new token
    ring = np.array([[[0.2, -0.4, 0.6], [9.0, 9.0, 9.0]]])
    tok = np.array([[1.0, 2.0, -1.0]])
    A, D, raw, dtb, s0 = -1.0, 0.5, 0.3, -0.3, 0.75
    y, ring2, S = oracle.ssd_step(tok, np.array([[raw]]), w, bias, np.array([dtb]), np.array([A]), np.array([D]),
                                  ring, 1, np.array([[[[s0]]]]), 1, 1, 1, 1)
    act = silu(bias + w[:, 0] * ring[0, 0] + w[:, 1] * tok[0])
    dt = np.log(2.0)
    Snew = np.exp(dt * A) * s0 + dt * act[0] * act[1]
    assert S[0, 0, 0, 0] == pytest.approx(Snew, rel=1e-14)
    assert y[0, 0] == pytest.approx(Snew * act[2] + D * act[0], rel=1e-14)
    np.testing.assert_array_equal(ring2[0, 1], tok[0])
    np.testing.assert_array_equal(ring2[0, 0], ring[0, 0])


def test_max_rel_err_metric():
    ref = np.array([1.0, -2.0, 0.0, 1e-9])
    rms = np.sqrt(np.mean(ref ** 2))
    got = ref + np.array([0.01, 0.0, 0.02, 0.0])
    assert oracle.max_rel_err(got, ref) == pytest.approx(max(0.01 / 1.0, 0.02 / rms))


# ----------------------------------------------------------------------------- gated group RMSNorm
# Zamba2 article §三 (group RMSNorm times SiLU of the gate after the scan), §五 (rms_norm_eps 1e-5).

def test_gated_rmsnorm_by_hand():
    # two groups of two; z = ln 3 gives sigmoid(z) = 3/4, so SiLU(z) = 0.75 ln 3 exactly
    y = np.array([[3.0, 4.0, 1.0, -2.0]])
    z = np.full((1, 4), np.log(3.0))
    w = np.array([1.0, 2.0, -1.0, 0.5])
    s = 0.75 * np.log(3.0)
    nb = oracle.gated_rmsnorm(y, z, w, 2, eps=0.0, norm_before_gate=True)
    want = np.array([3 / np.sqrt(12.5), 2 * 4 / np.sqrt(12.5), -1 / np.sqrt(2.5), 0.5 * -2 / np.sqrt(2.5)]) * s
    np.testing.assert_allclose(nb[0], want, rtol=1e-14)
    # gate first with a common gate: SiLU(z) cancels inside each group's normalisation
    gf = oracle.gated_rmsnorm(y, z, w, 2, eps=0.0, norm_before_gate=False)
    np.testing.assert_allclose(gf[0], want / s, rtol=1e-14)


def test_gated_rmsnorm_eps_placement():
    # y = (1, 1), gate first with SiLU = 1 is impossible exactly, so take norm first with z -> large:
    # out = y / sqrt(mean(y^2) + eps) * SiLU(z); mean(y^2) = 1, eps = 1 -> 1/sqrt(2) * SiLU(z)
    y = np.ones((1, 2))
    z = np.full((1, 2), 40.0)
    out = oracle.gated_rmsnorm(y, z, np.ones(2), 2, eps=1.0, norm_before_gate=True)
    np.testing.assert_allclose(out[0], 40.0 / (1.0 + np.exp(-40.0)) / np.sqrt(2.0), rtol=1e-14)


def test_gated_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(7)
    y, z = rng.standard_normal((5, 48)), rng.standard_normal((5, 48))
    out = oracle.gated_rmsnorm(y, z, np.ones(48), 16, eps=0.0)
    # every group of the gate-first output has unit mean square
    np.testing.assert_allclose((out.reshape(5, 3, 16) ** 2).mean(-1), 1.0, rtol=1e-12)
    # and the output does not change when y is scaled by a positive factor
    np.testing.assert_allclose(oracle.gated_rmsnorm(3.5 * y, z, np.ones(48), 16, eps=0.0), out, rtol=1e-12)
    # norm first: scaling y leaves it unchanged too, and the gate multiplies elementwise
    nb = oracle.gated_rmsnorm(y, z, np.ones(48), 16, eps=0.0, norm_before_gate=True)
    np.testing.assert_allclose(oracle.gated_rmsnorm(0.25 * y, z, np.ones(48), 16, eps=0.0, norm_before_gate=True),
                               nb, rtol=1e-12)


def test_gated_rmsnorm_groups_are_independent_and_zero_gate():
    rng = np.random.default_rng(8)
    y, z, w = rng.standard_normal((2, 32)), rng.standard_normal((2, 32)), rng.standard_normal(32)
    a = oracle.gated_rmsnorm(y, z, w, 8)
    y2 = y.copy()
    y2[:, 8:16] *= 100.0
    b = oracle.gated_rmsnorm(y2, z, w, 8)
    np.testing.assert_array_equal(np.delete(a, np.s_[8:16], 1), np.delete(b, np.s_[8:16], 1))
    # SiLU(0) = 0: a zero gate zeroes the output in both orders (eps keeps it finite)
    zero = np.zeros_like(z)
    assert not np.any(oracle.gated_rmsnorm(y, zero, w, 8))
    assert not np.any(oracle.gated_rmsnorm(y, zero, w, 8, norm_before_gate=True))


# ----------------------------------------------------------------- right-padded batches

def test_conv_padded_batch_equals_each_sequence_alone():
    # sequence b of a right-padded batch: outputs and ring equal those of its first lens[b] tokens run
    # on their own; positions past lens[b] stay unwritten (NaN); the ring holds the last W real tokens
    rng = np.random.default_rng(40)
    Bn, L, Cd, W = 5, 13, 4, 4
    x = rng.standard_normal((Bn, L, Cd))
    w = rng.uniform(-0.5, 0.5, (Cd, W))
    bias = rng.uniform(-0.5, 0.5, Cd)
    ring = rng.standard_normal((Bn, W, Cd))
    lens = np.array([13, 0, 2, 7, 4])
    for phase in (0, 3):
        out, ring_out = oracle.conv1d(x, w, bias, ring, phase, seq_lens=lens)
        for b, n in enumerate(lens):
            ob, rb = oracle.conv1d(x[b:b + 1, :n], w, bias, ring[b:b + 1], phase)
            np.testing.assert_allclose(out[b, :n], ob[0], rtol=1e-14, atol=1e-300)
            assert np.isnan(out[b, n:]).all()
            np.testing.assert_array_equal(ring_out[b], rb[0])
            hist = np.stack([ring[b, (phase - j) % W] for j in range(W, 0, -1)])   # tokens -W..-1
            np.testing.assert_array_equal(ring_out[b], np.concatenate([hist, x[b, :n]])[-W:])


def test_scan_padded_batch_equals_each_sequence_alone():
    rng = np.random.default_rng(41)
    Bn, L, H, P, N, G = 4, 19, 4, 3, 5, 2
    x, Bm, Cm, dt_raw, dt_bias, A, D, S0 = _rand_scan(rng, Bn, L, H, P, N, G)
    lens = np.array([19, 0, 1, 11])
    y, s = oracle.ssd_scan(x, Bm, Cm, dt_raw, dt_bias, A, D, S0, seq_lens=lens)
    for b, n in enumerate(lens):
        sl = slice(b, b + 1)
        yb, sb = _bruteforce(x[sl, :n], Bm[sl, :n], Cm[sl, :n], dt_raw[sl, :n], dt_bias, A, D, S0[sl])
        assert rel(y[b, :n], yb[0]) < RTOL if n else True
        assert np.isnan(y[b, n:]).all()
        assert rel(s[b], sb[0]) < RTOL
    np.testing.assert_array_equal(s[1], S0[1])     # an empty sequence hands its state back unchanged


def test_scan_padding_content_is_ignored():
    # whatever sits in the padded positions must not reach any output
    rng = np.random.default_rng(42)
    x, Bm, Cm, dt_raw, dt_bias, A, D, S0 = _rand_scan(rng, 3, 16, 2, 3, 4, 1)
    lens = np.array([16, 5, 9])
    y, s = oracle.ssd_scan(x, Bm, Cm, dt_raw, dt_bias, A, D, S0, seq_lens=lens)
    junk = [a.copy() for a in (x, Bm, Cm, dt_raw)]
    for a in junk:
        for b, n in enumerate(lens):
            a[b, n:] = 1e3 * rng.standard_normal(a[b, n:].shape)
    y2, s2 = oracle.ssd_scan(*junk, dt_bias, A, D, S0, seq_lens=lens)
    np.testing.assert_array_equal(np.nan_to_num(y, nan=7.0), np.nan_to_num(y2, nan=7.0))
    np.testing.assert_array_equal(s, s2)


# ----------------------------------------------------------------- packed batches

def test_packed_equals_padded_batch():
    # the packed form (sequences back to back, sliced apart) against the right-padded form (one
    # row per sequence, lengths given to the C oracle): two different routes to the same sums
    rng = np.random.default_rng(50)
    lens = np.array([7, 0, 19, 1, 12])
    Bn, L, H, P, N, G, W = len(lens), int(lens.max()), 4, 3, 5, 2, 4
    Cd = H * P + 2 * G * N
    x, Bm, Cm, dt_raw, dt_bias, A, D, S0 = _rand_scan(rng, Bn, L, H, P, N, G)
    xbc = rng.standard_normal((Bn, L, Cd))
    w = rng.uniform(-0.5, 0.5, (Cd, W))
    ring = rng.standard_normal((Bn, W, Cd))
    cu = np.concatenate([[0], np.cumsum(lens)])
    pack = lambda a: np.concatenate([a[b, :n] for b, n in enumerate(lens)], 0)
    yp, sp = oracle.ssd_scan_packed(pack(x), pack(Bm), pack(Cm), pack(dt_raw), cu, dt_bias, A, D, S0)
    yq, sq = oracle.ssd_scan(x, Bm, Cm, dt_raw, dt_bias, A, D, S0, seq_lens=lens)
    np.testing.assert_allclose(yp, pack(yq), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(sp, sq, rtol=1e-13, atol=1e-300)
    op, rp = oracle.conv1d_packed(pack(xbc), cu, w, None, ring, 2)
    oq, rq = oracle.conv1d(xbc, w, None, ring, 2, seq_lens=lens)
    np.testing.assert_allclose(op, pack(oq), rtol=1e-14, atol=1e-300)
    np.testing.assert_array_equal(rp, rq)


def test_packed_sequences_do_not_interact():
    # changing one sequence's tokens changes no other sequence's outputs or state
    rng = np.random.default_rng(51)
    lens = [9, 14, 5]
    T, H, P, N, G = sum(lens), 2, 3, 4, 1
    x, Bm, Cm, dt_raw, dt_bias, A, D, _ = _rand_scan(rng, 1, T, H, P, N, G)
    x, Bm, Cm, dt_raw = x[0], Bm[0], Cm[0], dt_raw[0]
    cu = np.concatenate([[0], np.cumsum(lens)])
    y1, s1 = oracle.ssd_scan_packed(x, Bm, Cm, dt_raw, cu, dt_bias, A, D)
    x2 = x.copy()
    x2[cu[1]:cu[2]] += 1.0
    y2, s2 = oracle.ssd_scan_packed(x2, Bm, Cm, dt_raw, cu, dt_bias, A, D)
    for b in (0, 2):
        np.testing.assert_array_equal(y1[cu[b]:cu[b + 1]], y2[cu[b]:cu[b + 1]])
        np.testing.assert_array_equal(s1[b], s2[b])
    assert not np.allclose(y1[cu[1]:cu[2]], y2[cu[1]:cu[2]])
