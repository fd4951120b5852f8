"""Helpers for the GPU parity tests: move seeded inputs to the device and results back.

Everything numeric is done by the library under test (on the GPU) or by the
oracle (on the CPU); this module only converts between numpy and torch.
"""
import numpy as np
import torch

import selective_state_space_mixer_amd as m2

BF16_TOL = 2e-2   # bf16 activations, fp32 state
F32_TOL = 1e-4    # fp32 activations


def tol_for(io: str) -> float:
    return BF16_TOL if io == "bf16" else F32_TOL


def torch_io(io: str):
    return torch.bfloat16 if io == "bf16" else torch.float32


def dev(a, io: str = "f32"):
    """numpy (values representable in io) -> GPU tensor of the io dtype (exact)."""
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device="cuda", dtype=torch_io(io))


def dev32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def dims_of(d) -> "m2.M2Dims":
    """workloads.Dims -> the C ABI dims struct."""
    return m2.make_dims(d.batch, d.seqlen, d.d_model, d.expand, d.headdim, d.d_state, d.n_groups, d.d_conv,
                        d.chunk_size, d.io)


def nan_like(shape, io: str):
    return torch.full(shape, float("nan"), device="cuda", dtype=torch_io(io))


def workspace(dims, packed_tokens=None):
    """Scan workspace for dims (a packed batch: pass its token count)."""
    n = m2.m2_ssd_scan_workspace(dims) if packed_tokens is None else m2.m2_ssd_scan_workspace_packed(dims, packed_tokens)
    return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda") if n > 0 else None
