"""The scan entry point that allocates nothing (m2_ssd_scan_fwd_noalloc), through the C ABI, against
m2_ssd_scan_fwd with a caller-owned workspace: two calls in a row on one GPU, the second smaller, each
bit-identical to the workspace entry point and within the bf16 bar of the fp64 oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import selective_state_space_mixer_amd as m2
    from gpu_util import dev, dev32, dims_of, host, nan_like, workspace


def _inputs(d, seed, cached):
    inp = workloads.generate(d, seed, cached)
    x, b, c = inp.split()
    lead = (d.batch, d.seqlen)
    return (inp, x.reshape(lead + (d.nheads, d.headdim)), b.reshape(lead + (d.n_groups, d.d_state)),
            c.reshape(lead + (d.n_groups, d.d_state)))


def _run(d, inp, x, b, c, noalloc):
    Bn, L, H, P, N = d.batch, d.seqlen, d.nheads, d.headdim, d.d_state
    dims = dims_of(d)
    y = nan_like((Bn, L, H * P), d.io)
    s_out = torch.full((Bn, H, P, N), float("nan"), device="cuda")
    args = (dims, dev(x, d.io), dev(b, d.io), dev(c, d.io), dev(inp.dt_raw, d.io), dev32(inp.dt_bias), dev32(inp.A),
            dev32(inp.D), y, dev32(inp.state0), s_out)
    if noalloc:
        m2.m2_ssd_scan_fwd_noalloc(*args)
    else:
        m2.m2_ssd_scan_fwd(*args, workspace=workspace(dims))
    torch.cuda.synchronize()
    return host(y).reshape(Bn, L, H, P), host(s_out)


def test_noalloc_scan_matches_the_workspace_entry_point_twice():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")
    cases = [
        # Zamba2-2.7B mixer shape, one 8192-token sequence: a plan of several segments (chain + fix-up)
        (workloads.CONFIGS[3].dims.replace(seqlen=8192), 7101, False),
        # then a smaller call with a cached state: the scratch array keeps the first call's contents
        (workloads.CONFIGS[2].dims.replace(batch=2, seqlen=1000), 7102, True),
    ]
    for d, seed, cached in cases:
        dims = dims_of(d)
        assert 0 < m2.m2_ssd_scan_workspace(dims) <= m2.M2_STATIC_SCRATCH_BYTES
        inp, x, b, c = _inputs(d, seed, cached)
        y0, s0 = _run(d, inp, x, b, c, noalloc=False)
        y1, s1 = _run(d, inp, x, b, c, noalloc=True)
        np.testing.assert_array_equal(y1, y0)
        np.testing.assert_array_equal(s1, s0)
        yr, sr = oracle.ssd_scan(x, b, c, inp.dt_raw, inp.dt_bias, inp.A, inp.D, inp.state0)
        ey, es = oracle.max_rel_err(y1, yr), oracle.max_rel_err(s1, sr)
        print("noalloc %s: y %.2e state %.2e" % ((d.batch, d.seqlen), ey, es))
        assert ey <= 2e-2 and es <= 2e-2
