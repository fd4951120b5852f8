"""Python binding of libm2ssd.so, the gfx950 Mamba-2 mixer hot path (include/m2ssd.h).

Argument marshalling only: each function takes torch tensors that already live
on the GPU, checks that their layout is one the C ABI can describe (sizes,
strides, dtype), and passes raw device pointers, element strides and the
current HIP stream to the entry point of the same name.  Every step of the
computation runs in the library's kernels.  There is no CPU fallback: if the
library is missing, importing this package raises.

Names and semantics follow the C ABI:
    m2_conv1d_fwd, m2_conv1d_fwd_packed, m2_ssd_scan_workspace, m2_ssd_scan_fwd,
    m2_ssd_scan_workspace_packed, m2_ssd_scan_fwd_packed, m2_ssd_scan_fwd_noalloc, m2_mixer_prefill_workspace,
    m2_mixer_prefill_fwd, m2_mixer_prefill_workspace_packed, m2_mixer_prefill_fwd_packed, m2_ssd_step, m2_gated_rmsnorm, m2_ssd_scan_bwd_workspace, m2_ssd_scan_bwd,
    m2_ssd_scan_bwd_packed, m2_stream_copy, m2_status_str, m2_abi_version, m2_last_hip_error
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libm2ssd.so")

M2_OK, M2_ERR_NULL, M2_ERR_SHAPE, M2_ERR_DTYPE, M2_ERR_ALIAS, M2_ERR_WORKSPACE, M2_ERR_UNSUPPORTED, \
    M2_ERR_LAUNCH, M2_ERR_TOO_LARGE = range(9)
M2_STATIC_SCRATCH_BYTES = 64 << 20
M2_F32, M2_BF16 = 0, 1
ABI_VERSION = 8

EXPORTS = ("m2_conv1d_fwd", "m2_conv1d_fwd_packed", "m2_ssd_scan_workspace", "m2_ssd_scan_fwd",
           "m2_ssd_scan_workspace_packed", "m2_ssd_scan_fwd_packed", "m2_ssd_scan_fwd_noalloc",
           "m2_mixer_prefill_workspace", "m2_mixer_prefill_fwd", "m2_mixer_prefill_workspace_packed",
           "m2_mixer_prefill_fwd_packed", "m2_ssd_step", "m2_gated_rmsnorm", "m2_stream_copy",
           "m2_ssd_scan_bwd_workspace", "m2_ssd_scan_bwd", "m2_ssd_scan_bwd_packed",
           "m2_status_str", "m2_abi_version", "m2_last_hip_error")


class M2Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("d_model", ctypes.c_int32), ("expand", ctypes.c_int32), ("headdim", ctypes.c_int32),
                ("d_state", ctypes.c_int32), ("n_groups", ctypes.c_int32), ("d_conv", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("io", ctypes.c_int32)]

    @property
    def d_inner(self):
        return self.expand * self.d_model

    @property
    def nheads(self):
        return self.d_inner // self.headdim

    @property
    def conv_dim(self):
        return self.d_inner + 2 * self.n_groups * self.d_state


class M2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = "%s failed: status %d (%s)" % (fn, status, m2_status_str(status))
        if status == M2_ERR_LAUNCH:
            msg += ": " + m2_last_hip_error()
        super().__init__(msg)


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libm2ssd.so is not built (%s); run `python selective_state_space_mixer_amd/build.py`"
                          % LIB_PATH)
    # The kernels must run on the HIP runtime instance that owns torch's device memory and
    # streams.  Importing torch first loads its HIP runtime, and libm2ssd.so then binds to
    # that already-loaded libamdhip64.so.7 instead of loading a second copy.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    dp = ctypes.POINTER(M2Dims)
    lib.m2_conv1d_fwd.argtypes = [dp, vp, i64, vp, vp, vp, i64, vp, vp, i64, vp, vp]
    lib.m2_conv1d_fwd.restype = ctypes.c_int
    lib.m2_conv1d_fwd_packed.argtypes = [dp, i64, vp, vp, i64, vp, vp, vp, i64, vp, vp, i64, vp]
    lib.m2_conv1d_fwd_packed.restype = ctypes.c_int
    lib.m2_ssd_scan_workspace.argtypes = [dp]
    lib.m2_ssd_scan_workspace.restype = sz
    lib.m2_ssd_scan_workspace_packed.argtypes = [dp, i64]
    lib.m2_ssd_scan_workspace_packed.restype = sz
    lib.m2_ssd_scan_fwd.argtypes = [dp, vp, i64, vp, vp, i64, vp, i64, vp, vp, vp, f32, f32, vp, vp, vp, i64,
                                    vp, sz, vp, vp]
    lib.m2_ssd_scan_fwd.restype = ctypes.c_int
    lib.m2_ssd_scan_fwd_packed.argtypes = [dp, i64, vp, vp, i64, vp, vp, i64, vp, i64, vp, vp, vp, f32, f32, vp, vp,
                                           vp, i64, vp, sz, vp]
    lib.m2_ssd_scan_fwd_packed.restype = ctypes.c_int
    lib.m2_ssd_scan_fwd_noalloc.argtypes = [dp, vp, i64, vp, vp, i64, vp, i64, vp, vp, vp, f32, f32, vp, vp, vp, i64,
                                            vp, vp]
    lib.m2_ssd_scan_fwd_noalloc.restype = ctypes.c_int
    lib.m2_mixer_prefill_workspace.argtypes = [dp]
    lib.m2_mixer_prefill_workspace.restype = sz
    lib.m2_mixer_prefill_fwd.argtypes = [dp, vp, i64, vp, vp, vp, i64, vp, vp, i64, vp, vp, vp, f32, f32, vp, vp, vp,
                                         i64, vp, sz, vp, vp]
    lib.m2_mixer_prefill_fwd.restype = ctypes.c_int
    lib.m2_mixer_prefill_workspace_packed.argtypes = [dp, i64]
    lib.m2_mixer_prefill_workspace_packed.restype = sz
    lib.m2_mixer_prefill_fwd_packed.argtypes = [dp, i64, vp, vp, i64, vp, vp, vp, i64, vp, vp, i64, vp, vp, vp, f32,
                                                f32, vp, vp, vp, i64, vp, sz, vp]
    lib.m2_mixer_prefill_fwd_packed.restype = ctypes.c_int
    lib.m2_ssd_step.argtypes = [dp, vp, i64, vp, i64, vp, vp, vp, vp, vp, f32, f32, vp, i64, vp, vp, vp]
    lib.m2_ssd_step.restype = ctypes.c_int
    lib.m2_gated_rmsnorm.argtypes = [i64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, i64, vp, i64, vp, f32,
                                     ctypes.c_int32, vp, i64, vp]
    lib.m2_gated_rmsnorm.restype = ctypes.c_int
    lib.m2_ssd_scan_bwd_workspace.argtypes = [dp]
    lib.m2_ssd_scan_bwd_workspace.restype = sz
    lib.m2_ssd_scan_bwd.argtypes = [dp, vp, i64, vp, vp, i64, vp, i64, vp, vp, vp, f32, f32, vp, vp, i64, vp, vp, i64,
                                    vp, vp, i64, vp, i64, vp, vp, vp, vp, vp, sz, vp, vp]
    lib.m2_ssd_scan_bwd.restype = ctypes.c_int
    lib.m2_ssd_scan_bwd_packed.argtypes = [dp, i64, vp, vp, i64, vp, vp, i64, vp, i64, vp, vp, vp, f32, f32, vp, vp,
                                           i64, vp, vp, i64, vp, vp, i64, vp, i64, vp, vp, vp, vp, vp, sz, vp]
    lib.m2_ssd_scan_bwd_packed.restype = ctypes.c_int
    lib.m2_stream_copy.argtypes = [vp, vp, sz, vp]
    lib.m2_stream_copy.restype = ctypes.c_int
    lib.m2_status_str.argtypes = [ctypes.c_int]
    lib.m2_status_str.restype = ctypes.c_char_p
    lib.m2_abi_version.argtypes = []
    lib.m2_abi_version.restype = ctypes.c_int
    lib.m2_last_hip_error.argtypes = []
    lib.m2_last_hip_error.restype = ctypes.c_char_p
    if lib.m2_abi_version() != ABI_VERSION:
        raise ImportError("libm2ssd.so ABI version %d, binding expects %d" % (lib.m2_abi_version(), ABI_VERSION))
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def make_dims(batch, seqlen, d_model, expand, headdim, d_state, n_groups=1, d_conv=4, chunk_size=0,
              io=M2_BF16) -> M2Dims:
    if isinstance(io, str):
        io = {"bf16": M2_BF16, "f32": M2_F32}[io]
    return M2Dims(batch, seqlen, d_model, expand, headdim, d_state, n_groups, d_conv, chunk_size, io)


def m2_status_str(status: int) -> str:
    return _lib.m2_status_str(int(status)).decode()


def m2_abi_version() -> int:
    return _lib.m2_abi_version()


def m2_last_hip_error() -> str:
    return _lib.m2_last_hip_error().decode()


# ----------------------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def _io_dtype(dims: M2Dims):
    torch = _torch()
    return torch.bfloat16 if dims.io == M2_BF16 else torch.float32


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(t, name, dtype, device_like=None):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)


def _tok_stride(t, name, dims: M2Dims, row: int) -> int:
    """Token stride of a [B, L, ..., row-elements] tensor whose last dims are contiguous.

    The ABI describes such a view by one token stride, with batch stride = L * token stride."""
    if t is None:
        return row
    shape = tuple(t.shape)
    if t.dim() < 3:
        raise ValueError("%s: expected at least 3 dims, got %s" % (name, shape))
    Bn, L = shape[0], shape[1]
    if (Bn, L) != (dims.batch, dims.seqlen):
        raise ValueError("%s: leading dims %s, expected (batch, seqlen) = %s" % (name, (Bn, L),
                                                                               (dims.batch, dims.seqlen)))
    inner = math.prod(shape[2:])
    if inner != row:
        raise ValueError("%s: trailing size %d, expected %d" % (name, inner, row))
    if Bn == 0 or L == 0:
        return row
    # trailing dims must be packed
    exp = 1
    for d in range(t.dim() - 1, 1, -1):
        if shape[d] != 1 and t.stride(d) != exp:
            raise ValueError("%s: trailing dims must be contiguous" % name)
        exp *= shape[d]
    if L > 1:
        ts = t.stride(1)
    else:
        ts = t.stride(0) if Bn > 1 else row
    if Bn > 1 and t.stride(0) != L * ts:
        raise ValueError("%s: batch stride must equal seqlen * token stride" % name)
    return ts


def _lens_ptr(seq_lens, dims: M2Dims):
    """Device pointer of an int32 [batch] lengths tensor (None: no padding)."""
    if seq_lens is None:
        return None
    _check(seq_lens, "seq_lens", _torch().int32)
    if not seq_lens.is_contiguous() or tuple(seq_lens.shape) != (dims.batch,):
        raise ValueError("seq_lens must be a contiguous int32 [batch] tensor")
    return _ptr(seq_lens)


def _call(fn, *args):
    st = getattr(_lib, fn)(*args)
    if st != M2_OK:
        raise M2Error(fn, st)


def m2_conv1d_fwd(dims: M2Dims, xbc, w, bias, out, ring_in=None, ring_in_step: int = 0, ring_out=None,
                  stream=None, seq_lens=None) -> None:
    """out[b,t,c] = SiLU(bias[c] + sum_k w[c,k] x[b,t-(W-1)+k,c]); see include/m2ssd.h.

    xbc, out [B, L, conv_dim] (io dtype, token-strided views allowed); w [conv_dim, W] f32;
    bias [conv_dim] f32 or None; ring_in / ring_out [B, W, conv_dim] io or None;
    seq_lens: int32 [B] GPU tensor of each right-padded sequence's length, or None."""
    torch = _torch()
    io = _io_dtype(dims)
    Cd = dims.conv_dim
    for n, t in (("xbc", xbc), ("out", out), ("ring_in", ring_in), ("ring_out", ring_out)):
        _check(t, n, io)
    for n, t in (("w", w), ("bias", bias)):
        _check(t, n, torch.float32)
    if not w.is_contiguous() or tuple(w.shape) != (Cd, dims.d_conv):
        raise ValueError("w must be contiguous [conv_dim, d_conv]")
    if bias is not None and (not bias.is_contiguous() or bias.numel() != Cd):
        raise ValueError("bias must be contiguous [conv_dim]")
    for n, t in (("ring_in", ring_in), ("ring_out", ring_out)):
        if t is not None and (not t.is_contiguous() or tuple(t.shape) != (dims.batch, dims.d_conv, Cd)):
            raise ValueError("%s must be contiguous [batch, d_conv, conv_dim]" % n)
    xs = _tok_stride(xbc, "xbc", dims, Cd)
    os_ = _tok_stride(out, "out", dims, Cd)
    _call("m2_conv1d_fwd", ctypes.byref(dims), _ptr(xbc), xs, _ptr(w), _ptr(bias), _ptr(ring_in),
          int(ring_in_step), _ptr(ring_out), _ptr(out), os_, _lens_ptr(seq_lens, dims), _stream(stream))


def m2_ssd_scan_workspace(dims: M2Dims) -> int:
    return int(_lib.m2_ssd_scan_workspace(ctypes.byref(dims)))


def m2_ssd_scan_workspace_packed(dims: M2Dims, total_tokens: int) -> int:
    return int(_lib.m2_ssd_scan_workspace_packed(ctypes.byref(dims), int(total_tokens)))


def _scan_args(dims: M2Dims, x, B, C, dt, dt_bias, A, D, y, state_in, state_out):
    """Checked pointers and token strides of a padded-batch scan call (shared by both scan entry points)."""
    torch = _torch()
    io = _io_dtype(dims)
    H, P, N, G = dims.nheads, dims.headdim, dims.d_state, dims.n_groups
    for n, t in (("x", x), ("B", B), ("C", C), ("dt", dt), ("y", y)):
        _check(t, n, io)
    for n, t in (("dt_bias", dt_bias), ("A", A), ("D", D), ("state_in", state_in), ("state_out", state_out)):
        _check(t, n, torch.float32)
    for n, t in (("dt_bias", dt_bias), ("A", A), ("D", D)):
        if t is not None and (not t.is_contiguous() or t.numel() != H):
            raise ValueError("%s must be contiguous [nheads]" % n)
    for n, t in (("state_in", state_in), ("state_out", state_out)):
        if t is not None and (not t.is_contiguous() or tuple(t.shape) != (dims.batch, H, P, N)):
            raise ValueError("%s must be contiguous [batch, nheads, headdim, d_state]" % n)
    xs = _tok_stride(x, "x", dims, H * P)
    bs = _tok_stride(B, "B", dims, G * N)
    cs = _tok_stride(C, "C", dims, G * N)
    if bs != cs:
        raise ValueError("B and C must have the same token stride")
    dts = _tok_stride(dt, "dt", dims, H)
    ys = _tok_stride(y, "y", dims, H * P)
    return (_ptr(x), xs, _ptr(B), _ptr(C), bs, _ptr(dt), dts, _ptr(dt_bias), _ptr(A), _ptr(D)), \
        (_ptr(state_in), _ptr(state_out), _ptr(y), ys)


def m2_ssd_scan_fwd(dims: M2Dims, x, B, C, dt, dt_bias, A, D, y, state_in=None, state_out=None,
                    dt_min: float = 0.0, dt_max: float = float("inf"), workspace=None, stream=None,
                    seq_lens=None) -> None:
    """Chunked selective-SSM scan; see include/m2ssd.h.

    x [B, L, H, P] (or [B, L, H*P]), B/C [B, L, G, N] (or [B, L, G*N]), dt [B, L, H], y like x,
    all io dtype, token-strided views allowed (B and C must share one token stride);
    dt_bias, A, D [H] f32 (D may be None); state_in / state_out [B, H, P, N] f32 or None;
    workspace: a uint8 GPU tensor of at least m2_ssd_scan_workspace(dims) bytes, or None;
    seq_lens: int32 [B] GPU tensor of each right-padded sequence's length, or None."""
    ins, outs = _scan_args(dims, x, B, C, dt, dt_bias, A, D, y, state_in, state_out)
    need = m2_ssd_scan_workspace(dims)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    elif need > 0:
        raise ValueError("m2_ssd_scan_fwd needs a workspace of %d bytes" % need)
    _call("m2_ssd_scan_fwd", ctypes.byref(dims), *ins, float(dt_min), float(dt_max), *outs, ws_ptr, ws_bytes,
          _lens_ptr(seq_lens, dims), _stream(stream))


def m2_ssd_scan_fwd_noalloc(dims: M2Dims, x, B, C, dt, dt_bias, A, D, y, state_in=None, state_out=None,
                            dt_min: float = 0.0, dt_max: float = float("inf"), stream=None, seq_lens=None) -> None:
    """m2_ssd_scan_fwd with the library's static scratch buffer as its workspace (no allocation);
    see include/m2ssd.h.  Arguments as m2_ssd_scan_fwd without `workspace`."""
    ins, outs = _scan_args(dims, x, B, C, dt, dt_bias, A, D, y, state_in, state_out)
    _call("m2_ssd_scan_fwd_noalloc", ctypes.byref(dims), *ins, float(dt_min), float(dt_max), *outs,
          _lens_ptr(seq_lens, dims), _stream(stream))


def m2_mixer_prefill_workspace(dims: M2Dims) -> int:
    return int(_lib.m2_mixer_prefill_workspace(ctypes.byref(dims)))


def m2_mixer_prefill_fwd(dims: M2Dims, xbc, w, bias, dt, dt_bias, A, D, y, ring_in=None, ring_in_step: int = 0,
                         ring_out=None, state_in=None, state_out=None, dt_min: float = 0.0,
                         dt_max: float = float("inf"), workspace=None, stream=None, seq_lens=None) -> None:
    """conv1d + SiLU and the scan of a prompt in one pass; see include/m2ssd.h.

    xbc [B, L, conv_dim] raw conv input; w [conv_dim, W], bias [conv_dim] or None; ring_in / ring_out
    [B, W, conv_dim] or None; dt [B, L, H]; dt_bias, A, D [H]; y [B, L, H*P]; state_in / state_out
    [B, H, P, N] f32 or None; workspace: a uint8 GPU tensor of at least m2_mixer_prefill_workspace(dims)
    bytes; seq_lens: int32 [B] GPU tensor or None."""
    torch = _torch()
    io = _io_dtype(dims)
    H, P, N, Cd = dims.nheads, dims.headdim, dims.d_state, dims.conv_dim
    for n, t in (("xbc", xbc), ("dt", dt), ("y", y), ("ring_in", ring_in), ("ring_out", ring_out)):
        _check(t, n, io)
    for n, t in (("w", w), ("bias", bias), ("dt_bias", dt_bias), ("A", A), ("D", D), ("state_in", state_in),
                 ("state_out", state_out)):
        _check(t, n, torch.float32)
    if not w.is_contiguous() or tuple(w.shape) != (Cd, dims.d_conv):
        raise ValueError("w must be contiguous [conv_dim, d_conv]")
    if bias is not None and (not bias.is_contiguous() or bias.numel() != Cd):
        raise ValueError("bias must be contiguous [conv_dim]")
    for n, t in (("ring_in", ring_in), ("ring_out", ring_out)):
        if t is not None and (not t.is_contiguous() or tuple(t.shape) != (dims.batch, dims.d_conv, Cd)):
            raise ValueError("%s must be contiguous [batch, d_conv, conv_dim]" % n)
    for n, t in (("dt_bias", dt_bias), ("A", A), ("D", D)):
        if t is not None and (not t.is_contiguous() or t.numel() != H):
            raise ValueError("%s must be contiguous [nheads]" % n)
    for n, t in (("state_in", state_in), ("state_out", state_out)):
        if t is not None and (not t.is_contiguous() or tuple(t.shape) != (dims.batch, H, P, N)):
            raise ValueError("%s must be contiguous [batch, nheads, headdim, d_state]" % n)
    xs = _tok_stride(xbc, "xbc", dims, Cd)
    dts = _tok_stride(dt, "dt", dims, H)
    ys = _tok_stride(y, "y", dims, H * P)
    need = m2_mixer_prefill_workspace(dims)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    elif need > 0:
        raise ValueError("m2_mixer_prefill_fwd needs a workspace of %d bytes" % need)
    _call("m2_mixer_prefill_fwd", ctypes.byref(dims), _ptr(xbc), xs, _ptr(w), _ptr(bias), _ptr(ring_in),
          int(ring_in_step), _ptr(ring_out), _ptr(dt), dts, _ptr(dt_bias), _ptr(A), _ptr(D), float(dt_min),
          float(dt_max), _ptr(state_in), _ptr(state_out), _ptr(y), ys, ws_ptr, ws_bytes, _lens_ptr(seq_lens, dims),
          _stream(stream))


def _packed_stride(t, name, T, row: int) -> int:
    """Token stride of a packed [T, ...] tensor whose trailing dims pack `row` contiguous elements."""
    shape = tuple(t.shape)
    if t.dim() < 2 or shape[0] != T or math.prod(shape[1:]) != row:
        raise ValueError("%s: expected [%d, ...] with %d elements per token, got %s" % (name, T, row, shape))
    if T == 0:
        return row
    exp = 1
    for d in range(t.dim() - 1, 0, -1):
        if shape[d] != 1 and t.stride(d) != exp:
            raise ValueError("%s: trailing dims must be contiguous" % name)
        exp *= shape[d]
    return t.stride(0) if T > 1 else row


def _cu_ptr(cu_seqlens, dims: M2Dims):
    _check(cu_seqlens, "cu_seqlens", _torch().int32)
    if not cu_seqlens.is_contiguous() or tuple(cu_seqlens.shape) != (dims.batch + 1,):
        raise ValueError("cu_seqlens must be a contiguous int32 [batch + 1] tensor")
    return _ptr(cu_seqlens)


def m2_conv1d_fwd_packed(dims: M2Dims, cu_seqlens, xbc, w, bias, out, ring_in=None, ring_in_step: int = 0,
                         ring_out=None, stream=None) -> None:
    """Packed batch conv; see include/m2ssd.h.  dims.batch sequences, dims.seqlen the longest;
    xbc, out [T, conv_dim] (io dtype, token-strided views allowed); cu_seqlens int32 [batch + 1] on
    the GPU; ring_in / ring_out [batch, W, conv_dim] or None."""
    torch = _torch()
    io = _io_dtype(dims)
    Cd = dims.conv_dim
    for n, t in (("xbc", xbc), ("out", out), ("ring_in", ring_in), ("ring_out", ring_out)):
        _check(t, n, io)
    for n, t in (("w", w), ("bias", bias)):
        _check(t, n, torch.float32)
    if not w.is_contiguous() or tuple(w.shape) != (Cd, dims.d_conv):
        raise ValueError("w must be contiguous [conv_dim, d_conv]")
    if bias is not None and (not bias.is_contiguous() or bias.numel() != Cd):
        raise ValueError("bias must be contiguous [conv_dim]")
    for n, t in (("ring_in", ring_in), ("ring_out", ring_out)):
        if t is not None and (not t.is_contiguous() or tuple(t.shape) != (dims.batch, dims.d_conv, Cd)):
            raise ValueError("%s must be contiguous [batch, d_conv, conv_dim]" % n)
    T = int(xbc.shape[0])
    xs = _packed_stride(xbc, "xbc", T, Cd)
    os_ = _packed_stride(out, "out", T, Cd)
    _call("m2_conv1d_fwd_packed", ctypes.byref(dims), T, _cu_ptr(cu_seqlens, dims), _ptr(xbc), xs, _ptr(w),
          _ptr(bias), _ptr(ring_in), int(ring_in_step), _ptr(ring_out), _ptr(out), os_, _stream(stream))


def m2_ssd_scan_fwd_packed(dims: M2Dims, cu_seqlens, x, B, C, dt, dt_bias, A, D, y, state_in=None, state_out=None,
                           dt_min: float = 0.0, dt_max: float = float("inf"), workspace=None, stream=None) -> None:
    """Packed batch scan; see include/m2ssd.h.  dims.batch sequences, dims.seqlen the longest;
    x [T, H, P] (or [T, H*P]), B/C [T, G, N], dt [T, H], y like x (token-strided views allowed, B and C
    sharing one stride); cu_seqlens int32 [batch + 1] on the GPU; state_in / state_out
    [batch, H, P, N] f32 or None; workspace: a uint8 GPU tensor of at least
    m2_ssd_scan_workspace_packed(dims, T) bytes, or None."""
    torch = _torch()
    io = _io_dtype(dims)
    H, P, N, G = dims.nheads, dims.headdim, dims.d_state, dims.n_groups
    for n, t in (("x", x), ("B", B), ("C", C), ("dt", dt), ("y", y)):
        _check(t, n, io)
    for n, t in (("dt_bias", dt_bias), ("A", A), ("D", D), ("state_in", state_in), ("state_out", state_out)):
        _check(t, n, torch.float32)
    for n, t in (("dt_bias", dt_bias), ("A", A), ("D", D)):
        if t is not None and (not t.is_contiguous() or t.numel() != H):
            raise ValueError("%s must be contiguous [nheads]" % n)
    for n, t in (("state_in", state_in), ("state_out", state_out)):
        if t is not None and (not t.is_contiguous() or tuple(t.shape) != (dims.batch, H, P, N)):
            raise ValueError("%s must be contiguous [batch, nheads, headdim, d_state]" % n)
    T = int(x.shape[0])
    xs = _packed_stride(x, "x", T, H * P)
    bs = _packed_stride(B, "B", T, G * N)
    cs = _packed_stride(C, "C", T, G * N)
    if bs != cs:
        raise ValueError("B and C must have the same token stride")
    dts = _packed_stride(dt, "dt", T, H)
    ys = _packed_stride(y, "y", T, H * P)
    need = m2_ssd_scan_workspace_packed(dims, T)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    elif need > 0:
        raise ValueError("m2_ssd_scan_fwd_packed needs a workspace of %d bytes" % need)
    _call("m2_ssd_scan_fwd_packed", ctypes.byref(dims), T, _cu_ptr(cu_seqlens, dims), _ptr(x), xs, _ptr(B), _ptr(C),
          bs, _ptr(dt), dts, _ptr(dt_bias), _ptr(A), _ptr(D), float(dt_min), float(dt_max), _ptr(state_in),
          _ptr(state_out), _ptr(y), ys, ws_ptr, ws_bytes, _stream(stream))


def m2_mixer_prefill_workspace_packed(dims: M2Dims, total_tokens: int) -> int:
    return int(_lib.m2_mixer_prefill_workspace_packed(ctypes.byref(dims), int(total_tokens)))


def m2_mixer_prefill_fwd_packed(dims: M2Dims, cu_seqlens, xbc, w, bias, dt, dt_bias, A, D, y, ring_in=None,
                                ring_in_step: int = 0, ring_out=None, state_in=None, state_out=None,
                                dt_min: float = 0.0, dt_max: float = float("inf"), workspace=None,
                                stream=None) -> None:
    """Packed batch, one pass; see include/m2ssd.h.  dims.batch sequences, dims.seqlen the longest;
    xbc [T, conv_dim] raw conv input, dt [T, H], y [T, H*P] (token-strided views allowed); cu_seqlens
    int32 [batch + 1] on the GPU; w, bias, ring_in / ring_out, dt_bias, A, D and the states as in
    m2_mixer_prefill_fwd; workspace: a uint8 GPU tensor of at least
    m2_mixer_prefill_workspace_packed(dims, T) bytes."""
    torch = _torch()
    io = _io_dtype(dims)
    H, P, N, Cd = dims.nheads, dims.headdim, dims.d_state, dims.conv_dim
    for n, t in (("xbc", xbc), ("dt", dt), ("y", y), ("ring_in", ring_in), ("ring_out", ring_out)):
        _check(t, n, io)
    for n, t in (("w", w), ("bias", bias), ("dt_bias", dt_bias), ("A", A), ("D", D), ("state_in", state_in),
                 ("state_out", state_out)):
        _check(t, n, torch.float32)
    if not w.is_contiguous() or tuple(w.shape) != (Cd, dims.d_conv):
        raise ValueError("w must be contiguous [conv_dim, d_conv]")
    if bias is not None and (not bias.is_contiguous() or bias.numel() != Cd):
        raise ValueError("bias must be contiguous [conv_dim]")
    for n, t in (("ring_in", ring_in), ("ring_out", ring_out)):
        if t is not None and (not t.is_contiguous() or tuple(t.shape) != (dims.batch, dims.d_conv, Cd)):
            raise ValueError("%s must be contiguous [batch, d_conv, conv_dim]" % n)
    for n, t in (("dt_bias", dt_bias), ("A", A), ("D", D)):
        if t is not None and (not t.is_contiguous() or t.numel() != H):
            raise ValueError("%s must be contiguous [nheads]" % n)
    for n, t in (("state_in", state_in), ("state_out", state_out)):
        if t is not None and (not t.is_contiguous() or tuple(t.shape) != (dims.batch, H, P, N)):
            raise ValueError("%s must be contiguous [batch, nheads, headdim, d_state]" % n)
    T = int(xbc.shape[0])
    xs = _packed_stride(xbc, "xbc", T, Cd)
    dts = _packed_stride(dt, "dt", T, H)
    ys = _packed_stride(y, "y", T, H * P)
    need = m2_mixer_prefill_workspace_packed(dims, T)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    elif need > 0:
        raise ValueError("m2_mixer_prefill_fwd_packed needs a workspace of %d bytes" % need)
    _call("m2_mixer_prefill_fwd_packed", ctypes.byref(dims), T, _cu_ptr(cu_seqlens, dims), _ptr(xbc), xs, _ptr(w),
          _ptr(bias), _ptr(ring_in), int(ring_in_step), _ptr(ring_out), _ptr(dt), dts, _ptr(dt_bias), _ptr(A),
          _ptr(D), float(dt_min), float(dt_max), _ptr(state_in), _ptr(state_out), _ptr(y), ys, ws_ptr, ws_bytes,
          _stream(stream))


def m2_ssd_step(dims: M2Dims, xbc_tok, dt_tok, w, bias, dt_bias, A, D, ring, step: int, state, y,
                dt_min: float = 0.0, dt_max: float = float("inf"), stream=None) -> None:
    """One fused decode token; see include/m2ssd.h.

    xbc_tok [B, conv_dim], dt_tok [B, H] (io dtype, row-strided allowed); ring [B, W, conv_dim] io and
    state [B, H, P, N] f32 updated in place; y [B, H*P] io."""
    torch = _torch()
    io = _io_dtype(dims)
    H, P, N, Cd, W = dims.nheads, dims.headdim, dims.d_state, dims.conv_dim, dims.d_conv
    for n, t in (("xbc_tok", xbc_tok), ("dt_tok", dt_tok), ("ring", ring), ("y", y)):
        _check(t, n, io)
    for n, t in (("w", w), ("bias", bias), ("dt_bias", dt_bias), ("A", A), ("D", D), ("state", state)):
        _check(t, n, torch.float32)
    Bn = dims.batch
    for n, t, row in (("xbc_tok", xbc_tok, Cd), ("dt_tok", dt_tok, H)):
        if tuple(t.shape) != (Bn, row) or (row > 1 and t.stride(1) != 1):
            raise ValueError("%s must be [batch, %d] with contiguous rows" % (n, row))
    if not w.is_contiguous() or tuple(w.shape) != (Cd, W):
        raise ValueError("w must be contiguous [conv_dim, d_conv]")
    if bias is not None and (not bias.is_contiguous() or bias.numel() != Cd):
        raise ValueError("bias must be contiguous [conv_dim]")
    if not ring.is_contiguous() or tuple(ring.shape) != (Bn, W, Cd):
        raise ValueError("ring must be contiguous [batch, d_conv, conv_dim]")
    if not state.is_contiguous() or tuple(state.shape) != (Bn, H, P, N):
        raise ValueError("state must be contiguous [batch, nheads, headdim, d_state]")
    if not y.is_contiguous() or y.numel() != Bn * H * P:
        raise ValueError("y must be contiguous [batch, nheads*headdim]")
    xbs = xbc_tok.stride(0) if Bn > 1 else Cd
    dts = dt_tok.stride(0) if Bn > 1 else H
    _call("m2_ssd_step", ctypes.byref(dims), _ptr(xbc_tok), xbs, _ptr(dt_tok), dts, _ptr(w), _ptr(bias),
          _ptr(dt_bias), _ptr(A), _ptr(D), float(dt_min), float(dt_max), _ptr(ring), int(step), _ptr(state),
          _ptr(y), _stream(stream))


def _rows(t, name):
    """(rows, row stride) of a [..., D] tensor whose leading dims form one evenly strided run of rows."""
    if t.dim() < 1:
        raise ValueError("%s: expected at least one dim" % name)
    D = t.shape[-1]
    rows = 1
    for n in t.shape[:-1]:
        rows *= n
    if rows == 0 or D == 0:
        return 0, max(D, 1)  # empty: strides carry no meaning
    if t.stride(-1) != 1 and D > 1:
        raise ValueError("%s: the last dim must be contiguous" % name)
    if t.dim() == 1 or rows <= 1:
        return rows, D
    stride = t.stride(-2)
    expect = stride
    for i in range(t.dim() - 2, -1, -1):
        if t.shape[i] > 1 and t.stride(i) != expect:
            raise ValueError("%s: leading dims must be one evenly strided run of rows" % name)
        expect *= t.shape[i]
    return rows, stride


def m2_gated_rmsnorm(y, z, w, out, group_size: int, eps: float = 1e-5, norm_before_gate: bool = False,
                     stream=None) -> None:
    """Gated group RMSNorm after the scan; see include/m2ssd.h.

    y, z, out [..., d_inner] (bf16 or f32, same dtype; rows evenly strided, last dim contiguous);
    w [d_inner] f32.  out may be y itself."""
    torch = _torch()
    io = y.dtype
    if io not in (torch.bfloat16, torch.float32):
        raise TypeError("y: expected bfloat16 or float32, got %s" % io)
    for n, t in (("z", z), ("out", out)):
        _check(t, n, io)
    _check(y, "y", io)
    _check(w, "w", torch.float32)
    D = y.shape[-1]
    if tuple(z.shape) != tuple(y.shape) or tuple(out.shape) != tuple(y.shape):
        raise ValueError("y, z and out must have the same shape")
    if not w.is_contiguous() or w.numel() != D:
        raise ValueError("w must be contiguous [d_inner]")
    ntok, ys = _rows(y, "y")
    _, zs = _rows(z, "z")
    _, os_ = _rows(out, "out")
    _call("m2_gated_rmsnorm", int(ntok), int(D), int(group_size), M2_BF16 if io == torch.bfloat16 else M2_F32,
          _ptr(y), ys, _ptr(z), zs, _ptr(w), float(eps), int(bool(norm_before_gate)), _ptr(out), os_,
          _stream(stream))


def m2_ssd_scan_bwd_workspace(dims: M2Dims) -> int:
    """Bytes of workspace m2_ssd_scan_bwd needs (0: not built for these dims)."""
    return int(_lib.m2_ssd_scan_bwd_workspace(ctypes.byref(dims)))


def m2_ssd_scan_bwd(dims: M2Dims, x, B, C, dt, dt_bias, A, D, dy, dx, dB, dC, ddt, ddt_bias, dA, dD,
                    state_in=None, dstate_out=None, dstate_in=None, dt_min: float = 0.0, dt_max: float = float("inf"),
                    workspace=None, stream=None, seq_lens=None) -> None:
    """Backward of the scan; see include/m2ssd.h.

    Inputs as m2_ssd_scan_fwd plus dy (like y) and dstate_out [B, H, P, N] f32 or None; outputs dx (like x),
    dB/dC (like B/C, sharing one token stride), ddt (like dt), ddt_bias/dA/dD [H] f32 and dstate_in
    [B, H, P, N] f32 or None; workspace: a uint8 GPU tensor of at least m2_ssd_scan_bwd_workspace(dims)
    bytes; seq_lens: int32 [B] GPU tensor of each right-padded sequence's length, or None."""
    torch = _torch()
    ins, _ = _scan_args(dims, x, B, C, dt, dt_bias, A, D, dy, state_in, None)
    io = _io_dtype(dims)
    H, P, N, G = dims.nheads, dims.headdim, dims.d_state, dims.n_groups
    for n, t in (("dx", dx), ("dB", dB), ("dC", dC), ("ddt", ddt)):
        _check(t, n, io)
    for n, t in (("ddt_bias", ddt_bias), ("dA", dA), ("dD", dD), ("dstate_out", dstate_out), ("dstate_in", dstate_in)):
        _check(t, n, torch.float32)
    for n, t in (("ddt_bias", ddt_bias), ("dA", dA), ("dD", dD)):
        if t is None or not t.is_contiguous() or t.numel() != H:
            raise ValueError("%s must be a contiguous [nheads] tensor" % n)
    for n, t in (("dstate_out", dstate_out), ("dstate_in", dstate_in)):
        if t is not None and (not t.is_contiguous() or tuple(t.shape) != (dims.batch, H, P, N)):
            raise ValueError("%s must be contiguous [batch, nheads, headdim, d_state]" % n)
    dys = _tok_stride(dy, "dy", dims, H * P)
    dxs = _tok_stride(dx, "dx", dims, H * P)
    dbs = _tok_stride(dB, "dB", dims, G * N)
    if _tok_stride(dC, "dC", dims, G * N) != dbs:
        raise ValueError("dB and dC must have the same token stride")
    ddts = _tok_stride(ddt, "ddt", dims, H)
    if workspace is None:
        raise ValueError("m2_ssd_scan_bwd needs a workspace of %d bytes" % m2_ssd_scan_bwd_workspace(dims))
    _call("m2_ssd_scan_bwd", ctypes.byref(dims), *ins, float(dt_min), float(dt_max), _ptr(state_in), _ptr(dy), dys,
          _ptr(dstate_out), _ptr(dx), dxs, _ptr(dB), _ptr(dC), dbs, _ptr(ddt), ddts, _ptr(ddt_bias), _ptr(dA),
          _ptr(dD), _ptr(dstate_in), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
          _lens_ptr(seq_lens, dims), _stream(stream))


def m2_ssd_scan_bwd_packed(dims: M2Dims, cu_seqlens, x, B, C, dt, dt_bias, A, D, dy, dx, dB, dC, ddt, ddt_bias, dA,
                           dD, state_in=None, dstate_out=None, dstate_in=None, dt_min: float = 0.0,
                           dt_max: float = float("inf"), workspace=None, stream=None) -> None:
    """Backward of the packed scan; see include/m2ssd.h.  dims.batch sequences, dims.seqlen the longest;
    x/dy/dx [T, H, P] (or [T, H*P]), B/C/dB/dC [T, G, N], dt/ddt [T, H] (token-strided views allowed, B and
    C sharing one stride, dB and dC another); cu_seqlens int32 [batch + 1] on the GPU; state_in,
    dstate_out, dstate_in [batch, H, P, N] f32 or None; ddt_bias/dA/dD [H] f32; workspace: a uint8 GPU
    tensor of at least m2_ssd_scan_bwd_workspace(dims) bytes."""
    torch = _torch()
    io = _io_dtype(dims)
    H, P, N, G = dims.nheads, dims.headdim, dims.d_state, dims.n_groups
    for n, t in (("x", x), ("B", B), ("C", C), ("dt", dt), ("dy", dy), ("dx", dx), ("dB", dB), ("dC", dC),
                 ("ddt", ddt)):
        _check(t, n, io)
    for n, t in (("dt_bias", dt_bias), ("A", A), ("D", D), ("ddt_bias", ddt_bias), ("dA", dA), ("dD", dD),
                 ("state_in", state_in), ("dstate_out", dstate_out), ("dstate_in", dstate_in)):
        _check(t, n, torch.float32)
    for n, t in (("dt_bias", dt_bias), ("A", A), ("D", D), ("ddt_bias", ddt_bias), ("dA", dA), ("dD", dD)):
        if (t is None and n != "D") or (t is not None and (not t.is_contiguous() or t.numel() != H)):
            raise ValueError("%s must be a contiguous [nheads] tensor" % n)
    for n, t in (("state_in", state_in), ("dstate_out", dstate_out), ("dstate_in", dstate_in)):
        if t is not None and (not t.is_contiguous() or tuple(t.shape) != (dims.batch, H, P, N)):
            raise ValueError("%s must be contiguous [batch, nheads, headdim, d_state]" % n)
    T = int(x.shape[0])
    xs = _packed_stride(x, "x", T, H * P)
    bs = _packed_stride(B, "B", T, G * N)
    if _packed_stride(C, "C", T, G * N) != bs:
        raise ValueError("B and C must have the same token stride")
    dts = _packed_stride(dt, "dt", T, H)
    dys = _packed_stride(dy, "dy", T, H * P)
    dxs = _packed_stride(dx, "dx", T, H * P)
    dbs = _packed_stride(dB, "dB", T, G * N)
    if _packed_stride(dC, "dC", T, G * N) != dbs:
        raise ValueError("dB and dC must have the same token stride")
    ddts = _packed_stride(ddt, "ddt", T, H)
    if workspace is None:
        raise ValueError("m2_ssd_scan_bwd_packed needs a workspace of %d bytes" % m2_ssd_scan_bwd_workspace(dims))
    _call("m2_ssd_scan_bwd_packed", ctypes.byref(dims), T, _cu_ptr(cu_seqlens, dims), _ptr(x), xs, _ptr(B), _ptr(C),
          bs, _ptr(dt), dts, _ptr(dt_bias), _ptr(A), _ptr(D), float(dt_min), float(dt_max), _ptr(state_in), _ptr(dy),
          dys, _ptr(dstate_out), _ptr(dx), dxs, _ptr(dB), _ptr(dC), dbs, _ptr(ddt), ddts, _ptr(ddt_bias), _ptr(dA),
          _ptr(dD), _ptr(dstate_in), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
          _stream(stream))


def m2_stream_copy(dst, src, stream=None) -> None:
    """Copy src into dst (same byte size, 16-byte aligned GPU tensors) with the library's streaming copy
    kernel; see include/m2ssd.h."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n or not dst.is_cuda or not src.is_cuda:
        raise ValueError("dst and src must be GPU tensors of the same byte size")
    if not dst.is_contiguous() or not src.is_contiguous():
        raise ValueError("dst and src must be contiguous")
    _call("m2_stream_copy", _ptr(dst), _ptr(src), n, _stream(stream))
