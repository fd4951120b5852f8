"""Seeded synthetic inputs for the Mamba-2 mixer hot path.

This module is shared by the parity tests, the benchmark and the oracle
checks.  It draws random tensors and rounds them to the storage type; it
holds none of the mixer's arithmetic (no convolution, no softplus, no
recurrence), so neither the oracle nor the HIP path depends on the other
through it.

Shapes follow the mixer of the Zamba2 article ("Transformers 中 Zamba2 混合架构模型解析",
§三 Mamba2 Mixer and the §五 configuration table): ``d_inner = expand * d_model``,
``conv_dim = d_inner + 2 * n_groups * d_state``, depthwise conv width ``d_conv``.

Recipe (seed ``1000 + config index``, numpy PCG64, draw order fixed):
xBC ~ N(0,1) with the B and C channels scaled by 1/sqrt(d_state); dt_raw ~ N(0,1);
dt_bias ~ U(-4,-2); A = -exp(U(0, ln 16)); D ~ N(0,1); conv w, bias ~ U(-0.5,0.5);
initial state and conv history ~ N(0, 0.1) where the workload starts from a
cached state, else zero.  Floats are drawn in fp32 and rounded to bf16 with
round-to-nearest-even for bf16 workloads.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    out = (rounded >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to(a: np.ndarray, io: str) -> np.ndarray:
    """fp32 array holding values exactly representable in the storage type ``io``."""
    a = np.asarray(a, dtype=np.float32)
    if io == BF16:
        return bf16_to_f32(bf16_bits(a))
    return a


@dataclasses.dataclass(frozen=True)
class Dims:
    batch: int
    seqlen: int
    d_model: int
    expand: int
    headdim: int
    d_state: int
    n_groups: int = 1
    d_conv: int = 4
    chunk_size: int = 0
    io: str = BF16

    @property
    def d_inner(self) -> int:
        return self.expand * self.d_model

    @property
    def nheads(self) -> int:
        return self.d_inner // self.headdim

    @property
    def conv_dim(self) -> int:
        return self.d_inner + 2 * self.n_groups * self.d_state

    def replace(self, **kw) -> "Dims":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Config:
    index: int
    name: str
    dims: Dims
    cached_init: bool      # start from a random cached state / conv history
    decode_steps: int = 0  # > 0: decode workload of this many chained tokens


# The five workloads: a tiny fp32 case, a 130m-like mixer, and three at the
# Zamba2-2.7B mixer shape (hidden 2560, expand 2, d_state 64, headdim 64).
CONFIGS = [
    Config(0, "tiny-fp32", Dims(1, 64, 16, 2, 16, 16, 1, 4, 16, F32), False),
    Config(1, "mamba2-130m-like", Dims(4, 2048, 768, 2, 64, 128, 1, 4, 0, BF16), False),
    Config(2, "zamba2-2.7b-prefill-b8-l4096", Dims(8, 4096, 2560, 2, 64, 64, 1, 4, 0, BF16), True),
    Config(3, "zamba2-2.7b-prefill-b1-l32768", Dims(1, 32768, 2560, 2, 64, 64, 1, 4, 0, BF16), False),
    Config(4, "zamba2-2.7b-decode-b256-x128", Dims(256, 1, 2560, 2, 64, 64, 1, 4, 0, BF16), True, 128),
]


@dataclasses.dataclass
class Inputs:
    """One seeded draw.  Float arrays are fp32 holding io-representable values.

    xbc      [B, L, conv_dim]  conv input (x | B | C channel order); for decode
             workloads [steps, B, conv_dim]
    dt_raw   [B, L, H]         (decode: [steps, B, H])
    dt_bias, A, D [H]          fp32 parameters
    conv_w   [conv_dim, W], conv_b [conv_dim]  fp32 parameters
    state0   [B, H, P, N] fp32 or None
    ring0    [B, W, conv_dim] io-representable or None (slot-major conv history)
    """
    dims: Dims
    xbc: np.ndarray
    dt_raw: np.ndarray
    dt_bias: np.ndarray
    A: np.ndarray
    D: np.ndarray
    conv_w: np.ndarray
    conv_b: np.ndarray
    state0: Optional[np.ndarray]
    ring0: Optional[np.ndarray]

    # views of the conv input as scan inputs (x, B, C), as used by scan-only tests
    def split(self, act: Optional[np.ndarray] = None):
        d = self.dims
        a = self.xbc if act is None else act
        x = a[..., : d.d_inner]
        b = a[..., d.d_inner: d.d_inner + d.n_groups * d.d_state]
        c = a[..., d.d_inner + d.n_groups * d.d_state:]
        return x, b, c


def generate(dims: Dims, seed: int, cached_init: bool, steps: int = 0) -> Inputs:
    """Draw one workload.  ``steps > 0`` draws ``steps`` decode tokens per sequence."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, L, H, P, N, G, W = dims.batch, dims.seqlen, dims.nheads, dims.headdim, dims.d_state, dims.n_groups, dims.d_conv
    cd = dims.conv_dim
    lead = (steps, B) if steps > 0 else (B, L)
    xbc = rng.standard_normal(lead + (cd,), dtype=np.float32)
    xbc[..., dims.d_inner:] *= np.float32(1.0 / math.sqrt(N))
    dt_raw = rng.standard_normal(lead + (H,), dtype=np.float32)
    dt_bias = rng.uniform(-4.0, -2.0, size=H).astype(np.float32)
    A = (-np.exp(rng.uniform(0.0, math.log(16.0), size=H))).astype(np.float32)
    D = rng.standard_normal(H, dtype=np.float32)
    conv_w = rng.uniform(-0.5, 0.5, size=(cd, W)).astype(np.float32)
    conv_b = rng.uniform(-0.5, 0.5, size=cd).astype(np.float32)
    state0 = ring0 = None
    if cached_init:
        state0 = (0.1 * rng.standard_normal((B, H, P, N), dtype=np.float32)).astype(np.float32)
        ring0 = (0.1 * rng.standard_normal((B, W, cd), dtype=np.float32)).astype(np.float32)
    io = dims.io
    return Inputs(
        dims=dims,
        xbc=round_to(xbc, io),
        dt_raw=round_to(dt_raw, io),
        dt_bias=dt_bias, A=A, D=D, conv_w=conv_w, conv_b=conv_b,
        state0=state0,
        ring0=None if ring0 is None else round_to(ring0, io),
    )


def config_inputs(index: int, dims: Optional[Dims] = None) -> Inputs:
    """Inputs of workload ``index`` (optionally at reduced dims with the same recipe)."""
    cfg = CONFIGS[index]
    return generate(dims or cfg.dims, 1000 + index, cfg.cached_init, cfg.decode_steps)


def bf16_storage(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 storage of an array whose values are bf16-representable."""
    return bf16_bits(a)


def norm_inputs(ntok: int, d_inner: int, seed: int, io: str):
    """Inputs of the gated group RMSNorm: y shaped like a scan output, z like the gate half of the
    input projection (both ~N(0,1)), and a weight near one (1 + 0.1 N(0,1), fp32)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    y = rng.standard_normal((ntok, d_inner), dtype=np.float32)
    z = rng.standard_normal((ntok, d_inner), dtype=np.float32)
    w = (1.0 + 0.1 * rng.standard_normal(d_inner, dtype=np.float32)).astype(np.float32)
    return round_to(y, io), round_to(z, io), w


def grad_inputs(dims: Dims, seed: int, with_state: bool = True):
    """Upstream gradients for the scan's backward: dy shaped like the scan output [B, L, H, P] (~N(0,1),
    rounded to the activation type) and, if with_state, the final state's gradient [B, H, P, N]
    (~N(0, 0.1), fp32); else None."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dy = rng.standard_normal((dims.batch, dims.seqlen, dims.nheads, dims.headdim), dtype=np.float32)
    ds = None
    if with_state:
        ds = (0.1 * rng.standard_normal((dims.batch, dims.nheads, dims.headdim, dims.d_state),
                                        dtype=np.float32)).astype(np.float32)
    return round_to(dy, dims.io), ds
