"""fp64 CPU oracle of the Mamba-2 mixer hot path (ctypes wrapper of m2_oracle.c).

TEST INFRASTRUCTURE ONLY: the parity tests, the smoke check and the
benchmark's CPU-baseline leg may use this package; the product path never
does.  It neither imports nor loads the HIP library, and the HIP library
shares no code with it.

All arrays are numpy float64, C-contiguous, in the layouts documented in
m2_oracle.c.  Functions return new arrays and never modify their inputs
(the step copies ``ring`` and ``state`` before updating them).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m2_oracle.c")
_LIB = os.path.join(_HERE, "libm2oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C99, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fopenmp",
                               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.c_void_p
        i64 = ctypes.c_int64
        f64 = ctypes.c_double
        lib.oracle_conv1d.argtypes = [i64, i64, i64, i64, dp, dp, dp, dp, i64, dp, dp, dp]
        lib.oracle_conv1d.restype = None
        lib.oracle_ssd_scan.argtypes = [i64] * 6 + [dp] * 7 + [f64, f64, dp, dp, dp, dp]
        lib.oracle_ssd_scan.restype = None
        lib.oracle_ssd_step.argtypes = [i64] * 6 + [dp] * 7 + [f64, f64, dp, i64, dp, dp]
        lib.oracle_ssd_step.restype = None
        lib.oracle_softplus.argtypes = [f64]
        lib.oracle_softplus.restype = f64
        lib.oracle_gated_rmsnorm.argtypes = [i64, i64, i64, dp, dp, dp, f64, i64, dp]
        lib.oracle_ssd_scan_bwd.argtypes = [i64] * 6 + [dp] * 7 + [f64, f64] + [dp] * 3 + [dp] * 8 + [dp]
        lib.oracle_ssd_scan_bwd.restype = None
        lib.oracle_gated_rmsnorm.restype = None
        _lib = lib
    return _lib


def _f64(a, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("oracle: expected shape %s, got %s" % (tuple(shape), a.shape))
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def softplus(v: float) -> float:
    return _load().oracle_softplus(float(v))


def gated_rmsnorm(y, z, w, group_size: int, eps: float = 1e-5, norm_before_gate: bool = False):
    """Gated group RMSNorm (m2_oracle.c, "norm").  y, z [..., D], w [D] -> out [..., D]."""
    y = _f64(y)
    lead, D = y.shape[:-1], y.shape[-1]
    if D % group_size:
        raise ValueError("oracle: D %d is not a multiple of group_size %d" % (D, group_size))
    z = _f64(z, y.shape)
    w = _f64(w, (D,))
    T = int(np.prod(lead)) if lead else 1
    out = np.empty_like(y)
    _load().oracle_gated_rmsnorm(T, D, group_size, _p(y), _p(z), _p(w), float(eps), int(bool(norm_before_gate)),
                                 _p(out))
    return out


def _lens(seq_lens, Bn, L):
    if seq_lens is None:
        return None
    a = np.ascontiguousarray(seq_lens, dtype=np.int64)
    if a.shape != (Bn,) or a.min(initial=0) < 0 or a.max(initial=0) > L:
        raise ValueError("oracle: seq_lens must be [batch] values in [0, seqlen]")
    return a


def conv1d(x, w, bias=None, ring_in=None, ring_in_step: int = 0, want_ring: bool = True, seq_lens=None):
    """Causal depthwise conv1d + SiLU.  x [B,L,Cd], w [Cd,W] -> (out [B,L,Cd], ring_out [B,W,Cd]).

    seq_lens [B] (optional): sequence b holds only its first seq_lens[b] tokens; outputs past them
    are NaN here, and ring_out holds the W tokens before seq_lens[b]."""
    x = _f64(x)
    Bn, L, Cd = x.shape
    w = _f64(w)
    W = w.shape[1]
    w = _f64(w, (Cd, W))
    bias = _f64(bias, (Cd,))
    ring_in = _f64(ring_in, (Bn, W, Cd))
    lens = _lens(seq_lens, Bn, L)
    out = np.full_like(x, np.nan)
    ring_out = np.empty((Bn, W, Cd)) if want_ring else None
    _load().oracle_conv1d(Bn, L, Cd, W, _p(x), _p(w), _p(bias), _p(ring_in), int(ring_in_step),
                          _p(ring_out), _p(out), _p(lens))
    return out, ring_out


def ssd_scan(x, Bm, Cm, dt_raw, dt_bias, A, D=None, state_in=None,
             dt_min: float = 0.0, dt_max: float = float("inf"), seq_lens=None):
    """Sequential selective-SSM recurrence.

    x [B,L,H,P], Bm/Cm [B,L,G,N], dt_raw [B,L,H] -> (y [B,L,H,P], state_out [B,H,P,N]).
    seq_lens [B] (optional): sequence b consumes only its first seq_lens[b] tokens; y past them is
    NaN here, and state_out is the state after its last token."""
    x = _f64(x)
    Bn, L, H, P = x.shape
    Bm = _f64(Bm)
    G, N = Bm.shape[2], Bm.shape[3]
    Bm = _f64(Bm, (Bn, L, G, N))
    Cm = _f64(Cm, (Bn, L, G, N))
    dt_raw = _f64(dt_raw, (Bn, L, H))
    dt_bias = _f64(dt_bias, (H,))
    A = _f64(A, (H,))
    D = _f64(D, (H,))
    state_in = _f64(state_in, (Bn, H, P, N))
    if H % G:
        raise ValueError("oracle: nheads must be a multiple of n_groups")
    lens = _lens(seq_lens, Bn, L)
    y = np.full_like(x, np.nan)
    state_out = np.empty((Bn, H, P, N))
    _load().oracle_ssd_scan(Bn, L, H, P, N, G, _p(x), _p(Bm), _p(Cm), _p(dt_raw), _p(dt_bias), _p(A),
                            _p(D), float(dt_min), float(dt_max), _p(state_in), _p(y), _p(state_out), _p(lens))
    return y, state_out


def ssd_scan_bwd(x, Bm, Cm, dt_raw, dt_bias, A, D=None, state_in=None, dy=None, dstate_out=None,
                 dt_min: float = 0.0, dt_max: float = float("inf"), seq_lens=None):
    """Gradients of L = sum(dy * y) + sum(dstate_out * state_out) for ssd_scan's outputs.

    Same inputs as ssd_scan, plus dy [B,L,H,P] and dstate_out [B,H,P,N] (None: zero).  Returns a dict
    with dx [B,L,H,P], dB and dC [B,L,G,N], ddt_raw [B,L,H], ddt_bias, dA, dD [H] and dstate_in
    [B,H,P,N].  seq_lens [B] (optional): as for ssd_scan (state_out is the state after sequence b's
    last real token); dx, dB, dC and ddt_raw past a sequence's length are NaN here."""
    x = _f64(x)
    Bn, L, H, P = x.shape
    Bm = _f64(Bm)
    G, N = Bm.shape[2], Bm.shape[3]
    Bm = _f64(Bm, (Bn, L, G, N))
    Cm = _f64(Cm, (Bn, L, G, N))
    dt_raw = _f64(dt_raw, (Bn, L, H))
    dt_bias = _f64(dt_bias, (H,))
    A = _f64(A, (H,))
    D = _f64(D, (H,))
    state_in = _f64(state_in, (Bn, H, P, N))
    dy = _f64(dy, (Bn, L, H, P)) if dy is not None else np.zeros((Bn, L, H, P))
    dstate_out = _f64(dstate_out, (Bn, H, P, N))
    if H % G:
        raise ValueError("oracle: nheads must be a multiple of n_groups")
    lens = _lens(seq_lens, Bn, L)
    out = {"dx": np.full_like(x, np.nan), "dB": np.full((Bn, L, G, N), np.nan), "dC": np.full((Bn, L, G, N), np.nan),
           "ddt_raw": np.full((Bn, L, H), np.nan), "ddt_bias": np.empty(H), "dA": np.empty(H), "dD": np.empty(H),
           "dstate_in": np.empty((Bn, H, P, N))}
    _load().oracle_ssd_scan_bwd(Bn, L, H, P, N, G, _p(x), _p(Bm), _p(Cm), _p(dt_raw), _p(dt_bias), _p(A),
                                _p(D), float(dt_min), float(dt_max), _p(state_in), _p(dy), _p(dstate_out),
                                _p(out["dx"]), _p(out["dB"]), _p(out["dC"]), _p(out["ddt_raw"]),
                                _p(out["ddt_bias"]), _p(out["dA"]), _p(out["dD"]), _p(out["dstate_in"]), _p(lens))
    return out


def _cu(cu_seqlens, T):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("oracle: cu_seqlens must rise from 0 to the token count")
    return cu


def conv1d_packed(x, cu_seqlens, w, bias=None, ring_in=None, ring_in_step: int = 0):
    """Packed batch: x [T, Cd] holds sequence b at rows cu_seqlens[b] .. cu_seqlens[b+1]-1.

    Each sequence is convolved on its own (its history from ring_in[b], or zero), exactly as conv1d
    does for one sequence.  Returns (out [T, Cd], ring_out [nseq, W, Cd])."""
    x = _f64(x)
    T, Cd = x.shape
    cu = _cu(cu_seqlens, T)
    W = np.asarray(w).shape[1]
    out = np.empty_like(x)
    rings = []
    for b in range(cu.size - 1):
        r = None if ring_in is None else np.asarray(ring_in)[b:b + 1]
        o, ro = conv1d(x[None, cu[b]:cu[b + 1]], w, bias, r, ring_in_step)
        out[cu[b]:cu[b + 1]] = o[0]
        rings.append(ro[0])
    return out, (np.stack(rings) if rings else np.empty((0, W, Cd)))


def ssd_scan_packed(x, Bm, Cm, dt_raw, cu_seqlens, dt_bias, A, D=None, state_in=None,
                    dt_min: float = 0.0, dt_max: float = float("inf")):
    """Packed batch: x [T, H, P], Bm/Cm [T, G, N], dt_raw [T, H]; sequence b at rows
    cu_seqlens[b] .. cu_seqlens[b+1]-1, starting from state_in[b] (or zero), scanned on its own.
    Returns (y [T, H, P], state_out [nseq, H, P, N])."""
    x = _f64(x)
    T, H, P = x.shape
    N = np.asarray(Bm).shape[2]
    cu = _cu(cu_seqlens, T)
    y = np.empty_like(x)
    states = []
    for b in range(cu.size - 1):
        sl = slice(cu[b], cu[b + 1])
        s0 = None if state_in is None else np.asarray(state_in)[b:b + 1]
        yb, sb = ssd_scan(x[None, sl], np.asarray(Bm)[None, sl], np.asarray(Cm)[None, sl],
                          np.asarray(dt_raw)[None, sl], dt_bias, A, D, s0, dt_min, dt_max)
        y[sl] = yb[0]
        states.append(sb[0])
    return y, (np.stack(states) if states else np.empty((0, H, P, N)))


def ssd_scan_bwd_packed(x, Bm, Cm, dt_raw, cu_seqlens, dt_bias, A, D=None, state_in=None, dy=None,
                        dstate_out=None, dt_min: float = 0.0, dt_max: float = float("inf")):
    """Backward of ssd_scan_packed: each sequence's gradients from ssd_scan_bwd on its own rows (with
    its own state_in[b] and dstate_out[b]); dx, dB, dC, ddt_raw [T, ...] by rows, ddt_bias, dA and dD
    summed over the sequences, dstate_in [nseq, H, P, N]."""
    x = _f64(x)
    T, H, P = x.shape
    G, N = np.asarray(Bm).shape[1], np.asarray(Bm).shape[2]
    cu = _cu(cu_seqlens, T)
    out = {"dx": np.empty_like(x), "dB": np.empty((T, G, N)), "dC": np.empty((T, G, N)), "ddt_raw": np.empty((T, H)),
           "ddt_bias": np.zeros(H), "dA": np.zeros(H), "dD": np.zeros(H)}
    dsi = []
    for b in range(cu.size - 1):
        sl = slice(cu[b], cu[b + 1])
        one = lambda a: None if a is None else np.asarray(a)[b:b + 1]
        gb = ssd_scan_bwd(x[None, sl], np.asarray(Bm)[None, sl], np.asarray(Cm)[None, sl], np.asarray(dt_raw)[None, sl],
                          dt_bias, A, D, one(state_in), None if dy is None else np.asarray(dy)[None, sl],
                          one(dstate_out), dt_min, dt_max)
        for k in ("dx", "dB", "dC", "ddt_raw"):
            out[k][sl] = gb[k][0]
        for k in ("ddt_bias", "dA", "dD"):
            out[k] += gb[k]
        dsi.append(gb["dstate_in"][0])
    out["dstate_in"] = np.stack(dsi) if dsi else np.empty((0, H, P, N))
    return out


def ssd_step(xbc_tok, dt_tok, w, bias, dt_bias, A, D, ring, step: int, state,
             H: int, P: int, N: int, G: int = 1,
             dt_min: float = 0.0, dt_max: float = float("inf")):
    """One decode token: xbc_tok [B,Cd], dt_tok [B,H], ring [B,W,Cd], state [B,H,P,N].

    Returns (y [B,H*P], ring_new, state_new)."""
    xbc_tok = _f64(xbc_tok)
    Bn, Cd = xbc_tok.shape
    if Cd != H * P + 2 * G * N or H % G:
        raise ValueError("oracle: inconsistent step dims")
    w = _f64(w)
    W = w.shape[1]
    w = _f64(w, (Cd, W))
    bias = _f64(bias, (Cd,))
    dt_tok = _f64(dt_tok, (Bn, H))
    dt_bias = _f64(dt_bias, (H,))
    A = _f64(A, (H,))
    D = _f64(D, (H,))
    ring = np.array(_f64(ring, (Bn, W, Cd)), copy=True)
    state = np.array(_f64(state, (Bn, H, P, N)), copy=True)
    y = np.empty((Bn, H * P))
    _load().oracle_ssd_step(Bn, H, P, N, G, W, _p(xbc_tok), _p(dt_tok), _p(w), _p(bias), _p(dt_bias),
                            _p(A), _p(D), float(dt_min), float(dt_max), _p(ring), int(step), _p(state), _p(y))
    return y, ring, state


def split_act(act, H: int, P: int, N: int, G: int = 1):
    """Channel split of a conv output [..., Cd] into x [..., H, P], B and C [..., G, N]."""
    Di = H * P
    x = act[..., :Di].reshape(act.shape[:-1] + (H, P))
    b = act[..., Di:Di + G * N].reshape(act.shape[:-1] + (G, N))
    c = act[..., Di + G * N:Di + 2 * G * N].reshape(act.shape[:-1] + (G, N))
    return x, b, c


def mixer_prefill(xbc, dt_raw, conv_w, conv_b, dt_bias, A, D, H, P, N, G=1,
                  ring_in=None, ring_in_step=0, state_in=None):
    """conv1d + SiLU -> split -> scan, all in fp64.  Returns (y, state_out, ring_out, act)."""
    act, ring_out = conv1d(xbc, conv_w, conv_b, ring_in, ring_in_step)
    x, b, c = split_act(act, H, P, N, G)
    y, s = ssd_scan(x, b, c, dt_raw, dt_bias, A, D, state_in)
    return y, s, ring_out, act


def max_rel_err(got, ref) -> float:
    """max_i |g_i - o_i| / max(|o_i|, rms(o)) over the compared tensor (floored relative error)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError("shape mismatch %s vs %s" % (got.shape, ref.shape))
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    den = np.maximum(np.abs(ref), rms if rms > 0 else 1e-300)
    return float(np.max(np.abs(got - ref) / den))
