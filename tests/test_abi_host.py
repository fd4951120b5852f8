"""Host-side checks of the C-ABI library (no GPU needed, no kernel is launched).

The library must load, export every function include/m2ssd.h declares, and
reject invalid arguments with the documented status before anything is
enqueued.  All argument sets used here fail validation, so no device memory is
touched (the pointers are placeholders that are never dereferenced).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "m2ssd.h")

m2 = pytest.importorskip("selective_state_space_mixer_amd")

FAKE = 0x7000_0000_0000   # placeholder device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(m2_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(m2.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(m2.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    assert m2.m2_abi_version() == m2.ABI_VERSION
    for s in range(9):
        assert m2.m2_status_str(s)
    assert m2.m2_status_str(99) == "unknown status"


def dims(**kw):
    base = dict(batch=2, seqlen=128, d_model=2560, expand=2, headdim=64, d_state=64, n_groups=1, d_conv=4,
                chunk_size=0, io=m2.M2_BF16)
    base.update(kw)
    return m2.M2Dims(**base)


def conv(d, xbc=FAKE, xs=None, w=FAKE + 0x100000, bias=None, ring_in=None, step=0, ring_out=None,
         out=FAKE + 0x4000_0000, os_=None, lens=None):
    lib = m2.lib()
    cd = d.conv_dim if d.expand > 0 else 1
    return lib.m2_conv1d_fwd(ctypes.byref(d) if d is not None else None, xbc, xs or cd, w, bias, ring_in, step,
                             ring_out, out, os_ or cd, lens, None)


def scan(d, x=FAKE, xs=None, B=FAKE + 0x10000000, C=FAKE + 0x10000100, bcs=None, dt=FAKE + 0x20000000, dts=None,
         dt_bias=FAKE + 0x30000000, A=FAKE + 0x30001000, D=None, dt_min=0.0, dt_max=float("inf"),
         s_in=None, s_out=None, y=FAKE + 0x4000_0000_00, ys=None, ws=None, ws_bytes=0, lens=None):
    lib = m2.lib()
    di = d.expand * d.d_model
    return lib.m2_ssd_scan_fwd(ctypes.byref(d), x, xs or di, B, C, bcs or d.n_groups * d.d_state, dt,
                               dts or max(di // max(d.headdim, 1), 1), dt_bias, A, D, dt_min, dt_max, s_in, s_out,
                               y, ys or di, ws, ws_bytes, lens, None)


def step(d, xbc=FAKE, xs=None, dt=FAKE + 0x1000000, dts=None, w=FAKE + 0x2000000, bias=None,
         dt_bias=FAKE + 0x3000000, A=FAKE + 0x3001000, D=None, ring=FAKE + 0x4000000, stepi=0,
         state=FAKE + 0x1_0000_0000, y=FAKE + 0x9_0000_0000, dt_min=0.0, dt_max=float("inf")):
    lib = m2.lib()
    return lib.m2_ssd_step(ctypes.byref(d), xbc, xs or d.conv_dim, dt, dts or d.nheads, w, bias, dt_bias, A, D,
                           dt_min, dt_max, ring, stepi, state, y, None)


def test_null_dims():
    assert m2.lib().m2_conv1d_fwd(None, FAKE, 1, FAKE, None, None, 0, None, FAKE, 1, None, None) == m2.M2_ERR_NULL
    assert m2.lib().m2_ssd_scan_workspace(None) == 0


def test_conv_validation():
    assert conv(dims(io=7)) == m2.M2_ERR_DTYPE
    assert conv(dims(batch=-1)) == m2.M2_ERR_SHAPE
    assert conv(dims(d_conv=5)) == m2.M2_ERR_UNSUPPORTED
    assert conv(dims(d_conv=1)) == m2.M2_ERR_UNSUPPORTED
    assert conv(dims(headdim=48)) == m2.M2_ERR_SHAPE            # 5120 % 48 != 0
    assert conv(dims(n_groups=3)) == m2.M2_ERR_SHAPE            # 80 heads % 3 != 0
    assert conv(dims(), w=None) == m2.M2_ERR_NULL
    assert conv(dims(), xbc=None) == m2.M2_ERR_NULL
    assert conv(dims(), out=None) == m2.M2_ERR_NULL
    d = dims()
    assert conv(d, xs=d.conv_dim - 1) == m2.M2_ERR_SHAPE
    assert conv(d, os_=d.conv_dim - 8) == m2.M2_ERR_SHAPE
    assert conv(d, out=FAKE + 64) == m2.M2_ERR_ALIAS             # out overlaps xbc
    assert conv(d, ring_in=FAKE + 0x2000_0000_0, ring_out=FAKE + 0x2000_0000_0 + 16) == m2.M2_ERR_ALIAS


def test_seq_lens_validation():
    d = dims()
    assert conv(d, lens=FAKE + 0x6_0000_0002) == m2.M2_ERR_UNSUPPORTED          # misaligned lengths
    assert conv(d, lens=FAKE + 0x4000_0000 + 4) == m2.M2_ERR_ALIAS              # lengths inside out
    assert conv(d, ring_out=FAKE + 0x7_0000_0000, lens=FAKE + 0x7_0000_0000) == m2.M2_ERR_ALIAS
    ws = dict(ws=FAKE + 0x9_0000_0000, ws_bytes=m2.m2_ssd_scan_workspace(d))
    assert scan(d, lens=FAKE + 0x6_0000_0002, **ws) == m2.M2_ERR_UNSUPPORTED
    assert scan(d, lens=FAKE + 0x4000_0000_00 + 8, **ws) == m2.M2_ERR_ALIAS       # lengths inside y
    assert scan(d, s_out=FAKE + 0x5_0000_0000, lens=FAKE + 0x5_0000_0000 + 64, **ws) == m2.M2_ERR_ALIAS
    big = dims(batch=1, seqlen=32768)
    need = m2.m2_ssd_scan_workspace(big)
    if need:
        assert scan(big, ws=FAKE + 0x8_0000_0000, ws_bytes=need, lens=FAKE + 0x8_0000_0000 + 256) == m2.M2_ERR_ALIAS


def test_packed_validation():
    lib = m2.lib()
    d = dims()
    cd, di = d.conv_dim, d.expand * d.d_model
    out = FAKE + 0x4000_0000
    conv_p = lambda T, cu, o=out: lib.m2_conv1d_fwd_packed(ctypes.byref(d), T, cu, FAKE, cd, FAKE + 0x100000, None,
                                                           None, 0, None, o, cd, None)
    assert conv_p(256, None) == m2.M2_ERR_NULL
    assert conv_p(-1, FAKE + 0x6_0000_0000) == m2.M2_ERR_SHAPE
    assert conv_p(256, FAKE + 0x6_0000_0002) == m2.M2_ERR_UNSUPPORTED             # misaligned offsets
    assert conv_p(256, out + 64) == m2.M2_ERR_ALIAS                               # offsets inside out
    ws = max(m2.m2_ssd_scan_workspace_packed(d, 256), m2.m2_ssd_scan_workspace(d))
    scan_p = lambda T, cu: lib.m2_ssd_scan_fwd_packed(ctypes.byref(d), T, cu, FAKE, di, FAKE + 0x10000000,
                                                      FAKE + 0x10000100, 128, FAKE + 0x20000000, 80,
                                                      FAKE + 0x30000000, FAKE + 0x30001000, None, 0.0,
                                                      float("inf"), None, None, FAKE + 0x4000_0000_00, di,
                                                      FAKE + 0x9_0000_0000, ws, None)
    assert scan_p(256, None) == m2.M2_ERR_NULL
    assert scan_p(-5, FAKE + 0x6_0000_0000) == m2.M2_ERR_SHAPE
    assert scan_p(256, FAKE + 0x6_0000_0001) == m2.M2_ERR_UNSUPPORTED
    assert scan_p(256, FAKE + 0x4000_0000_00 + 32) == m2.M2_ERR_ALIAS             # offsets inside y


def test_packed_workspace_follows_the_total():
    # eight prompts of 32768 tokens in all, the longest 8192: the packed plan sizes segments from the
    # total, the padded plan from batch x longest; both report sizes for their own plans
    d = dims(batch=8, seqlen=8192)
    assert m2.m2_ssd_scan_workspace_packed(d, 32768) > 0
    assert m2.m2_ssd_scan_workspace_packed(d, -1) == 0
    assert m2.m2_ssd_scan_workspace_packed(dims(io=7), 100) == 0
    needed = m2.m2_ssd_scan_workspace_packed(d, 32768)
    lib = m2.lib()
    di = d.expand * d.d_model
    st = lib.m2_ssd_scan_fwd_packed(ctypes.byref(d), 32768, FAKE + 0x6_0000_0000, FAKE, di, FAKE + 0x10000000,
                                    FAKE + 0x10000100, 128, FAKE + 0x20000000, 80, FAKE + 0x30000000,
                                    FAKE + 0x30001000, None, 0.0, float("inf"), None, None, FAKE + 0x4000_0000_00,
                                    di, FAKE + 0x9_0000_0000, needed - 1, None)
    assert st == m2.M2_ERR_WORKSPACE


def test_empty_batch_is_a_no_op():
    assert conv(dims(batch=0), xbc=None, out=None) == m2.M2_OK
    assert scan(dims(batch=0), x=None, B=None, C=None, dt=None, y=None) == m2.M2_OK
    assert step(dims(batch=0), xbc=None, dt=None, ring=None, state=None, y=None) == m2.M2_OK


def test_scan_validation():
    assert scan(dims(), dt_bias=None) == m2.M2_ERR_NULL
    assert scan(dims(), A=None) == m2.M2_ERR_NULL
    assert scan(dims(), y=None) == m2.M2_ERR_NULL
    assert scan(dims(), xs=100) == m2.M2_ERR_SHAPE
    assert scan(dims(), dts=79) == m2.M2_ERR_SHAPE
    assert scan(dims(), dt_min=1.0, dt_max=0.5) == m2.M2_ERR_SHAPE
    assert scan(dims(), dt_min=float("nan")) == m2.M2_ERR_SHAPE
    assert scan(dims(d_state=24, d_model=2560)) == m2.M2_ERR_UNSUPPORTED
    assert scan(dims(), y=FAKE + 128) == m2.M2_ERR_ALIAS                       # y overlaps x
    assert scan(dims(), s_in=FAKE + 0x5_0000_0000, s_out=FAKE + 0x5_0000_0000) == m2.M2_ERR_ALIAS
    assert scan(dims(), s_in=FAKE + 0x5_0000_0004) == m2.M2_ERR_UNSUPPORTED    # misaligned state
    assert scan(dims(), x=FAKE + 8) == m2.M2_ERR_UNSUPPORTED                    # misaligned x
    assert scan(dims(), C=FAKE + 0x10000100 + 2) == m2.M2_ERR_UNSUPPORTED       # misaligned C
    assert scan(dims(), bcs=5252) == m2.M2_ERR_UNSUPPORTED                      # B/C rows not 16-byte multiples
    assert scan(dims(), ys=5124) == m2.M2_ERR_UNSUPPORTED                       # y rows not 16-byte multiples


def test_chunk_size_outside_the_built_set_is_a_hint():
    """A chunk_size the kernels are not built for (Zamba2's configuration uses 256) means the library's
    choice: the same workspace as chunk_size 0, and the call gets past the chunk check (here it stops at
    the missing workspace, before any launch)."""
    base = m2.m2_ssd_scan_workspace(dims(batch=1, seqlen=32768))
    assert base > 0
    for q in (48, 128, 256, 1 << 20):
        assert m2.m2_ssd_scan_workspace(dims(batch=1, seqlen=32768, chunk_size=q)) == base
        assert scan(dims(batch=1, seqlen=32768, chunk_size=q), ws=None) == m2.M2_ERR_WORKSPACE
    # a built chunk length is honoured (a different plan, so a different workspace)
    assert m2.m2_ssd_scan_workspace(dims(batch=1, seqlen=32768, chunk_size=64)) != base
    assert scan(dims(chunk_size=-1)) == m2.M2_ERR_SHAPE


def test_scan_workspace_required_when_reported():
    d = dims(batch=1, seqlen=32768)
    need = m2.m2_ssd_scan_workspace(d)
    if need == 0:
        pytest.skip("no workspace needed at this shape")
    assert scan(d, ws=None) == m2.M2_ERR_WORKSPACE
    assert scan(d, ws=FAKE + 0x8_0000_0000, ws_bytes=need - 1) == m2.M2_ERR_WORKSPACE


def test_step_validation():
    assert step(dims(), stepi=-1) == m2.M2_ERR_SHAPE
    assert step(dims(), ring=None) == m2.M2_ERR_NULL
    assert step(dims(), state=None) == m2.M2_ERR_NULL
    assert step(dims(), xs=100) == m2.M2_ERR_SHAPE
    assert step(dims(d_state=24, d_model=2560)) == m2.M2_ERR_UNSUPPORTED
    assert step(dims(), y=FAKE + 0x4000000 + 64) == m2.M2_ERR_ALIAS           # y overlaps ring
    assert step(dims(), state=FAKE + 0x1_0000_0008) == m2.M2_ERR_UNSUPPORTED  # misaligned state


def norm(ntok=4, D=5120, gs=5120, io=m2.M2_BF16, y=FAKE, ys=None, z=FAKE + 0x1000_0000, zs=None,
         w=FAKE + 0x2000_0000, eps=1e-5, nbg=0, out=FAKE + 0x3000_0000, os_=None):
    return m2.lib().m2_gated_rmsnorm(ntok, D, gs, io, y, ys or D, z, zs or D, w, eps, nbg, out, os_ or D, None)


def test_gated_rmsnorm_validation():
    assert norm(io=5) == m2.M2_ERR_DTYPE
    assert norm(ntok=-1) == m2.M2_ERR_SHAPE
    assert norm(gs=3000) == m2.M2_ERR_SHAPE                     # does not divide d_inner
    assert norm(eps=-1.0) == m2.M2_ERR_SHAPE
    assert norm(eps=float("nan")) == m2.M2_ERR_SHAPE
    assert norm(w=None) == m2.M2_ERR_NULL
    assert norm(y=None) == m2.M2_ERR_NULL
    assert norm(ntok=0, y=None, z=None, out=None) == m2.M2_OK    # nothing to do
    assert norm(ys=5000) == m2.M2_ERR_SHAPE
    assert norm(D=5124, gs=1281) == m2.M2_ERR_UNSUPPORTED        # not a whole number of 16-byte pieces
    assert norm(D=16384, gs=16384) == m2.M2_ERR_UNSUPPORTED      # group longer than the kernel holds
    assert norm(out=FAKE + 0x1000_0000 + 256) == m2.M2_ERR_ALIAS  # out overlaps z
    assert norm(out=FAKE + 64) == m2.M2_ERR_ALIAS                # out overlaps y without being y
    assert norm(y=FAKE + 8) == m2.M2_ERR_UNSUPPORTED             # misaligned


def test_noalloc_scan_rejects_oversize_calls_before_any_launch():
    """m2_ssd_scan_fwd_noalloc compares the workspace a call needs with its static buffer on the host and
    returns M2_ERR_TOO_LARGE (nothing launched, no device touched) when it does not fit."""
    lib = m2.lib()
    d = dims(batch=1, seqlen=1 << 24)
    assert m2.m2_ssd_scan_workspace(d) > m2.M2_STATIC_SCRATCH_BYTES
    di = d.expand * d.d_model
    st = lib.m2_ssd_scan_fwd_noalloc(ctypes.byref(d), FAKE, di, FAKE + 0x10000000, FAKE + 0x10000100, 64,
                                     FAKE + 0x20000000, 80, FAKE + 0x30000000, FAKE + 0x30001000, None, 0.0,
                                     float("inf"), None, None, FAKE + 0x4000_0000_00, di, None, None)
    assert st == m2.M2_ERR_TOO_LARGE
    # argument errors are still reported first
    assert lib.m2_ssd_scan_fwd_noalloc(None, FAKE, di, FAKE, FAKE, 64, FAKE, 80, FAKE, FAKE, None, 0.0,
                                       float("inf"), None, None, FAKE, di, None, None) == m2.M2_ERR_NULL


def test_fused_prefill_shapes_and_validation():
    """The one-pass prompt path is built for bf16 headdim 64 / d_state 64; elsewhere it reports no
    workspace and M2_ERR_UNSUPPORTED, before anything is launched."""
    lib = m2.lib()
    assert m2.m2_mixer_prefill_workspace(dims(batch=1, seqlen=32768)) > m2.m2_ssd_scan_workspace(dims(batch=1, seqlen=32768))
    for bad in (dict(d_state=128), dict(headdim=32), dict(io=m2.M2_F32), dict(n_groups=40)):
        assert m2.m2_mixer_prefill_workspace(dims(**bad)) == 0, bad

    def call(d, xbc=FAKE, dt=FAKE + 0x2000_0000_0, y=FAKE + 0x4000_0000_00, ws=None, wsb=0, dts=None):
        return lib.m2_mixer_prefill_fwd(ctypes.byref(d), xbc, d.conv_dim, FAKE + 0x1000_0000_0, None, None, 0, None,
                                        dt, dts or d.expand * d.d_model // d.headdim, FAKE + 0x3000_0000_0,
                                        FAKE + 0x3000_1000_0, None, 0.0, float("inf"), None, None, y,
                                        d.expand * d.d_model, ws, wsb, None, None)
    assert call(dims(d_state=128)) == m2.M2_ERR_UNSUPPORTED
    assert call(dims(), xbc=None) == m2.M2_ERR_NULL
    assert call(dims(), dt=FAKE + 0x2000_0000_2) == m2.M2_ERR_UNSUPPORTED     # dt not on a dword
    assert call(dims(), dts=81) == m2.M2_ERR_UNSUPPORTED                       # odd dt token stride
    assert call(dims(), y=FAKE + 64) == m2.M2_ERR_ALIAS                         # y overlaps xbc
    assert call(dims(batch=1, seqlen=32768)) == m2.M2_ERR_WORKSPACE


def test_packed_fused_prefill_shapes_and_validation():
    """The packed one-pass path: its workspace follows the total (B/C activation rows plus the packed
    scan's plan), it is built where the one-pass path is, and it checks its token count, offsets and
    packed rows before any launch."""
    lib = m2.lib()
    d = dims(batch=8, seqlen=8192)
    need = m2.m2_mixer_prefill_workspace_packed(d, 32768)
    assert need >= m2.m2_ssd_scan_workspace_packed(d, 32768) + 32768 * 2 * d.n_groups * d.d_state * 2
    assert m2.m2_mixer_prefill_workspace_packed(d, -1) == 0
    for bad in (dict(d_state=128), dict(headdim=32), dict(io=m2.M2_F32)):
        assert m2.m2_mixer_prefill_workspace_packed(dims(**bad), 100) == 0, bad

    def call(d, T=256, cu=FAKE + 0x5000_0000_0, xbc=FAKE, y=FAKE + 0x4000_0000_00, ws=FAKE + 0x6000_0000_00,
             wsb=1 << 40):
        di = d.expand * d.d_model
        return lib.m2_mixer_prefill_fwd_packed(ctypes.byref(d), T, cu, xbc, d.conv_dim, FAKE + 0x1000_0000_0, None,
                                               None, 0, None, FAKE + 0x2000_0000_0, di // d.headdim,
                                               FAKE + 0x3000_0000_0, FAKE + 0x3000_1000_0, None, 0.0, float("inf"),
                                               None, None, y, di, ws, wsb, None)
    assert call(dims(d_state=128)) == m2.M2_ERR_UNSUPPORTED
    assert call(dims(), T=-1) == m2.M2_ERR_SHAPE
    assert call(dims(), cu=None) == m2.M2_ERR_NULL
    assert call(dims(), cu=FAKE + 0x5000_0000_2) == m2.M2_ERR_UNSUPPORTED     # offsets off a 4-byte boundary
    assert call(dims(), y=FAKE + 64) == m2.M2_ERR_ALIAS                         # y overlaps xbc
    assert call(dims(), cu=FAKE + 0x4000_0000_00 + 64) == m2.M2_ERR_ALIAS       # offsets inside y
    assert call(dims(batch=8, seqlen=8192), T=32768, wsb=1 << 20) == m2.M2_ERR_WORKSPACE


def test_scan_backward_shapes_and_validation():
    """The scan's backward is built for bf16 headdim 64 / d_state 64: elsewhere it reports no workspace
    and M2_ERR_UNSUPPORTED; argument, alignment, overlap and workspace errors come back before any
    launch."""
    lib = m2.lib()
    assert m2.m2_ssd_scan_bwd_workspace(dims(batch=1, seqlen=32768)) > 0
    for bad in (dict(d_state=128), dict(headdim=32), dict(io=m2.M2_F32)):
        assert m2.m2_ssd_scan_bwd_workspace(dims(**bad)) == 0, bad
    MB = 1 << 28

    def call(d, x=FAKE, dx=FAKE + 5 * MB, dB=FAKE + 6 * MB, ws=FAKE + 9 * MB, wsb=1 << 40, dA=FAKE + 8 * MB,
             xs=None, dt=FAKE + 3 * MB, lens=None):
        di = d.expand * d.d_model
        H, GN = di // d.headdim, d.n_groups * d.d_state
        return lib.m2_ssd_scan_bwd(ctypes.byref(d), x, xs or di, FAKE + 1 * MB, FAKE + 2 * MB, GN, dt, H,
                                   FAKE + 4 * MB, FAKE + 4 * MB + 4096, None, 0.0, float("inf"), None,
                                   FAKE + 10 * MB, di, None, dx, di, dB, FAKE + 7 * MB, GN, FAKE + 11 * MB, H,
                                   dA - 8192, dA, dA + 8192, None, ws, wsb, lens, None)
    assert call(dims(d_state=128)) == m2.M2_ERR_UNSUPPORTED
    assert call(dims(io=m2.M2_F32)) == m2.M2_ERR_UNSUPPORTED
    assert call(dims(), x=None) == m2.M2_ERR_NULL
    assert call(dims(), dA=0) == m2.M2_ERR_NULL
    assert call(dims(), xs=8) == m2.M2_ERR_SHAPE                        # token stride below the row
    assert call(dims(), x=FAKE + 8) == m2.M2_ERR_UNSUPPORTED            # x off a 16-byte boundary
    assert call(dims(), dt=FAKE + 3 * MB + 1) == m2.M2_ERR_UNSUPPORTED  # dt off a bf16 boundary
    assert call(dims(), dx=FAKE + 64) == m2.M2_ERR_ALIAS                 # dx overlaps x
    assert call(dims(), dB=FAKE + 5 * MB + 128) == m2.M2_ERR_ALIAS       # dB overlaps dx
    assert call(dims(), ws=FAKE + 6 * MB) == m2.M2_ERR_ALIAS             # workspace overlaps dB
    assert call(dims(), ws=None) == m2.M2_ERR_WORKSPACE
    assert call(dims(batch=1, seqlen=32768), wsb=1 << 20) == m2.M2_ERR_WORKSPACE
    assert call(dims(), lens=FAKE + 12 * MB + 2) == m2.M2_ERR_UNSUPPORTED  # lengths off a 4-byte boundary
    assert call(dims(), lens=FAKE + 5 * MB + 64) == m2.M2_ERR_ALIAS        # lengths inside dx


def test_packed_scan_backward_validation():
    """The packed backward checks its token count, offsets pointer and packed rows before any launch;
    an empty batch, or a batch with no tokens, is a valid no-op."""
    lib = m2.lib()
    MB = 1 << 28

    def call(d, T=4096, cu=FAKE + 12 * MB, x=FAKE, dx=FAKE + 5 * MB, xs=None, ws=FAKE + 9 * MB, wsb=1 << 40):
        di = d.expand * d.d_model
        H, GN = di // d.headdim, d.n_groups * d.d_state
        return lib.m2_ssd_scan_bwd_packed(ctypes.byref(d), T, cu, x, xs or di, FAKE + 1 * MB, FAKE + 2 * MB, GN,
                                          FAKE + 3 * MB, H, FAKE + 4 * MB, FAKE + 4 * MB + 4096, None, 0.0,
                                          float("inf"), None, FAKE + 10 * MB, di, None, dx, di, FAKE + 6 * MB,
                                          FAKE + 7 * MB, GN, FAKE + 11 * MB, H, FAKE + 8 * MB - 8192, FAKE + 8 * MB,
                                          FAKE + 8 * MB + 8192, None, ws, wsb, None)
    assert call(dims(), T=-1) == m2.M2_ERR_SHAPE
    assert call(dims(), cu=None) == m2.M2_ERR_NULL
    assert call(dims(), cu=FAKE + 12 * MB + 2) == m2.M2_ERR_UNSUPPORTED  # offsets off a 4-byte boundary
    assert call(dims(), cu=FAKE + 5 * MB + 64) == m2.M2_ERR_ALIAS        # offsets inside dx
    assert call(dims(), x=None) == m2.M2_ERR_NULL
    assert call(dims(), xs=8) == m2.M2_ERR_SHAPE
    assert call(dims(d_state=128)) == m2.M2_ERR_UNSUPPORTED
    assert call(dims(), ws=None) == m2.M2_ERR_WORKSPACE
    # dx spans the packed rows: an x starting in its last of 512 rows overlaps it
    assert call(dims(batch=8, seqlen=4096), T=512, dx=FAKE, x=FAKE + 511 * 5120 * 2) == m2.M2_ERR_ALIAS
