"""GPU parity of the conv on long prompts (the kernel that sizes its token tile at launch) against
the fp64 oracle.

The conv of the Zamba2 mixer (article "Transformers 中 Zamba2 混合架构模型解析", §三: depthwise
conv over the token axis, width mamba_d_conv, SiLU, its state carried as the last W inputs).  A
launch takes the long-prompt kernel when the grid, made one resident round, would give every lane
at least two turns of its load ring (32 tokens for bf16, 16 for fp32).  Every case below is sized so
that this holds at any occupancy up to 8 blocks per CU on 256 CUs (more tokens per lane on fewer
CUs), and so that the last tile of a sequence ends part-way through a ring turn:
  - the 2.7B channel count (5248) at 16461 tokens, conv widths 4, 3 and 2, with ring history at a
    non-zero phase;
  - fp32 activations (io "f32");
  - a right-padded batch (one sequence ends mid-tile, the other is full);
  - a packed batch with a 3-token sequence (shorter than the window) and an empty one;
  - one call against the same prompt in two calls continued through the ring, the second short
    enough for the fixed-tile kernel: bit-identical outputs and rings;
  - input and output as column slices of wider rows (token strides above conv_dim).
Outputs within the floored max-relative bound (2e-2 bf16, 1e-4 fp32); rings bit-exact; padding left
untouched.  Each test prints the error it reaches.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import selective_state_space_mixer_amd as m2
    from gpu_util import dev, dev32, dims_of, host, nan_like, tol_for

BASE = workloads.CONFIGS[3].dims   # d_model 2560: conv_dim 5248


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")


@pytest.mark.parametrize("width,io", [(4, "bf16"), (3, "bf16"), (2, "bf16"), (4, "f32")])
def test_long_prompt_conv(width, io):
    _need_gpu()
    d = BASE.replace(batch=1, seqlen=16461, d_conv=width, io=io)
    inp = workloads.generate(d, 8100 + width, True)
    phase = 2
    ref, ref_ring = oracle.conv1d(inp.xbc, inp.conv_w, inp.conv_b, inp.ring0, phase)
    out = nan_like((d.batch, d.seqlen, d.conv_dim), io)
    ring_out = nan_like((d.batch, width, d.conv_dim), io)
    m2.m2_conv1d_fwd(dims_of(d), dev(inp.xbc, io), dev32(inp.conv_w), dev32(inp.conv_b), out,
                     dev(inp.ring0, io), phase, ring_out)
    torch.cuda.synchronize()
    e = oracle.max_rel_err(host(out), ref)
    print("long conv W=%d %s, %d tokens x %d channels: %.2e" % (width, io, d.seqlen, d.conv_dim, e))
    assert e <= tol_for(io)
    np.testing.assert_array_equal(host(ring_out), ref_ring)


def test_long_prompt_conv_right_padded():
    _need_gpu()
    d = BASE.replace(batch=2, seqlen=12000)
    lens = np.array([7777, 12000], np.int32)
    inp = workloads.generate(d, 8201, True)
    ref, ref_ring = oracle.conv1d(inp.xbc, inp.conv_w, inp.conv_b, inp.ring0, 1, seq_lens=lens)
    out = nan_like((d.batch, d.seqlen, d.conv_dim), "bf16")
    ring_out = nan_like((d.batch, d.d_conv, d.conv_dim), "bf16")
    m2.m2_conv1d_fwd(dims_of(d), dev(inp.xbc, "bf16"), dev32(inp.conv_w), dev32(inp.conv_b), out,
                     dev(inp.ring0, "bf16"), 1, ring_out, seq_lens=torch.as_tensor(lens, device="cuda"))
    torch.cuda.synchronize()
    got = host(out)
    errs = []
    for b, n in enumerate(lens):
        errs.append(oracle.max_rel_err(got[b, :n], ref[b, :n]))
        assert np.isnan(got[b, n:]).all(), "padding of sequence %d written" % b
    print("long conv, right-padded %s: %s" % (lens.tolist(), " ".join("%.2e" % e for e in errs)))
    assert max(errs) <= tol_for("bf16")
    np.testing.assert_array_equal(host(ring_out), ref_ring)


def test_long_prompt_conv_packed():
    _need_gpu()
    lens = [9000, 3, 0, 6000]
    d = BASE.replace(batch=len(lens), seqlen=max(lens))
    inp = workloads.generate(d, 8301, True)
    xp = np.concatenate([inp.xbc[b, :n] for b, n in enumerate(lens)], 0)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ref, ref_ring = oracle.conv1d_packed(xp, cu, inp.conv_w, inp.conv_b, inp.ring0, 3)
    out = nan_like((len(xp), d.conv_dim), "bf16")
    ring_out = nan_like((len(lens), d.d_conv, d.conv_dim), "bf16")
    m2.m2_conv1d_fwd_packed(dims_of(d), torch.as_tensor(cu, device="cuda"), dev(xp, "bf16"), dev32(inp.conv_w),
                            dev32(inp.conv_b), out, dev(inp.ring0, "bf16"), 3, ring_out)
    torch.cuda.synchronize()
    e = oracle.max_rel_err(host(out), ref)
    print("long conv, packed %s: %.2e" % (lens, e))
    assert e <= tol_for("bf16")
    np.testing.assert_array_equal(host(ring_out), ref_ring)


def test_long_prompt_conv_split_matches_whole_bit_for_bit():
    """Both conv kernels form each output with the same taps in the same order, so a prompt convolved in
    one call (16461 tokens: the long-prompt kernel) equals, bit for bit, the same prompt in two calls
    continued through the ring: 9000 tokens (the long-prompt kernel), then 7461 tokens (at the five or
    more resident blocks per CU the long-prompt kernel gets, one round would give fewer than 32 tokens
    per lane there, so the fixed-tile kernel runs)."""
    _need_gpu()
    d = BASE.replace(batch=1, seqlen=16461)
    inp = workloads.generate(d, 8401, True)
    xbc = dev(inp.xbc, "bf16")
    w, bias = dev32(inp.conv_w), dev32(inp.conv_b)
    ring0 = dev(inp.ring0, "bf16")
    whole = nan_like((1, d.seqlen, d.conv_dim), "bf16")
    ring_whole = nan_like((1, d.d_conv, d.conv_dim), "bf16")
    m2.m2_conv1d_fwd(dims_of(d), xbc, w, bias, whole, ring0, 1, ring_whole)
    cut = 9000
    d1, d2 = d.replace(seqlen=cut), d.replace(seqlen=d.seqlen - cut)
    part = nan_like((1, d.seqlen, d.conv_dim), "bf16")
    ring_mid = nan_like((1, d.d_conv, d.conv_dim), "bf16")
    ring_end = nan_like((1, d.d_conv, d.conv_dim), "bf16")
    m2.m2_conv1d_fwd(dims_of(d1), xbc[:, :cut], w, bias, part[:, :cut], ring0, 1, ring_mid)
    m2.m2_conv1d_fwd(dims_of(d2), xbc[:, cut:], w, bias, part[:, cut:], ring_mid, 0, ring_end)
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int16), part.view(torch.int16))
    assert torch.equal(ring_whole.view(torch.int16), ring_end.view(torch.int16))
    ref, _ = oracle.conv1d(inp.xbc, inp.conv_w, inp.conv_b, inp.ring0, 1)
    e = oracle.max_rel_err(host(whole), ref)
    print("long conv, one call vs two: bit-identical; against the oracle %.2e" % e)
    assert e <= tol_for("bf16")


def test_long_prompt_conv_strided_views():
    """The conv input as a column slice of a wider row (as xBC sits between the gate and dt in the
    input projection's output) and the output written into a slice of a wider buffer: token strides
    5248 + 512 and 5248 + 256 elements, both multiples of 8, so the vector path and the long-prompt
    kernel run; the padding columns of the output buffer stay untouched."""
    _need_gpu()
    d = BASE.replace(batch=1, seqlen=12345)
    inp = workloads.generate(d, 8501, True)
    Cd, L = d.conv_dim, d.seqlen
    src = np.zeros((1, L, Cd + 512), np.float32)
    src[:, :, 256:256 + Cd] = inp.xbc
    xbig = dev(src, "bf16")
    obig = nan_like((1, L, Cd + 256), "bf16")
    ring_out = nan_like((1, d.d_conv, Cd), "bf16")
    m2.m2_conv1d_fwd(dims_of(d), xbig[:, :, 256:256 + Cd], dev32(inp.conv_w), dev32(inp.conv_b), obig[:, :, 128:128 + Cd],
                     dev(inp.ring0, "bf16"), 2, ring_out)
    torch.cuda.synchronize()
    ref, ref_ring = oracle.conv1d(inp.xbc, inp.conv_w, inp.conv_b, inp.ring0, 2)
    got = host(obig)
    e = oracle.max_rel_err(got[:, :, 128:128 + Cd], ref)
    print("long conv, strided views (token strides %d and %d): %.2e" % (Cd + 512, Cd + 256, e))
    assert e <= tol_for("bf16")
    assert np.isnan(got[:, :, :128]).all() and np.isnan(got[:, :, 128 + Cd:]).all(), "padding written"
    np.testing.assert_array_equal(host(ring_out), ref_ring)
