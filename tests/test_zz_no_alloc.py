"""gdn_recurrence_seq_noalloc on the GPU: the sequence recurrence with its
workspace in the library's static scratch array.

Calls go straight through the C ABI.  Each result is compared with
gdn_recurrence_seq_ws on the same inputs (same kernels, so bit for bit) and
with the oracle; two calls in a row, the second smaller, so the second runs on
a scratch array that still holds the first call's records.
"""
import sys

import numpy as np
import pytest

import oracle as orc
from gated_deltanet_decode_delta_amd import inputs
from gpu_util import dev, host, out_err, tile_err

pytestmark = pytest.mark.gpu

TOL_CHAIN = 1e-4


@pytest.fixture(scope="module")
def g():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_decode_delta_amd as gdn
    gdn.lib()
    return gdn


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _call(g, which, c, st, d, out, norm, ws=None):
    """One C-ABI call of the sequence entry point `which` on case c."""
    import torch
    lib = g.lib()
    NK, NV, D, B, T = c.NK, c.NV, c.D, c.B, c.T
    z, zs, gn = (d["z"].data_ptr(), NV * D, d["gn"].data_ptr()) if norm else (None, 0, None)
    args = [st.data_ptr(), st.stride(0), d["q"].data_ptr(), d["k"].data_ptr(), NK * D,
            d["v"].data_ptr(), NV * D, d["alpha"].data_ptr(), d["beta"].data_ptr(), NV,
            z, zs, gn, c.eps, out.data_ptr(), NV * D, B, T, NK, NV, D, D]
    stream = torch.cuda.current_stream().cuda_stream
    if which == "ws":
        return lib.gdn_recurrence_seq_ws(*args, ws.data_ptr(), ws.numel(), stream)
    return lib.gdn_recurrence_seq_noalloc(*args, stream)


def _run_pair(g, c, norm):
    """(noalloc o, noalloc state, ws o, ws state) on case c."""
    import torch
    d = {n: dev(getattr(c, n)) for n in ("q", "k", "v", "z", "alpha", "beta", "gn")}
    rows, vw = c.B * c.T, c.NV * c.D
    st_a, st_b = dev(c.state), dev(c.state)
    out_a = torch.full((rows, vw), float("nan"), device="cuda:0")
    out_b = torch.full((rows, vw), float("nan"), device="cuda:0")
    assert _call(g, "noalloc", c, st_a, d, out_a, norm) == 0
    need = g.lib().gdn_seq_workspace_bytes(c.B, c.T, c.NV, c.D, c.D)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda:0")
    assert _call(g, "ws", c, st_b, d, out_b, norm, ws) == 0
    return host(out_a), host(st_a), host(out_b), host(st_b)


def _oracle(c, norm):
    st = c.state.copy()
    kw = dict(z=c.z, gn=c.gn, eps=c.eps) if norm else {}
    o = orc.seq(st, c.q, c.k, c.v, c.alpha, c.beta, B=c.B, T=c.T, NK=c.NK, NV=c.NV, Dk=c.D,
                Dv=c.D, **kw)
    return o, st


def test_noalloc_two_calls_second_smaller(g):
    """Call 1: two sequences of 300 tokens (raw o); call 2: one sequence of 37
    tokens with the gated norm, on the scratch call 1 left behind."""
    first = inputs.make_case(2500, B=2, NK=16, NV=48, D=128, T=300)
    second = inputs.make_case(2501, B=1, NK=16, NV=48, D=128, T=37)
    for c, norm in ((first, False), (second, True)):
        say("noalloc", c.B, c.T, "norm" if norm else "raw")
        oa, sa, ob, sb = _run_pair(g, c, norm)
        assert np.array_equal(oa.view(np.uint32), ob.view(np.uint32))
        assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
        ref_o, ref_s = _oracle(c, norm)
        assert out_err(oa, ref_o, c.NV, c.D) < TOL_CHAIN
        assert tile_err(sa, ref_s, c.NV, c.D) < TOL_CHAIN


def test_noalloc_at_the_scratch_limit_then_small(g):
    """A shape whose records fill the scratch almost to its end (one sequence,
    48 heads, 9696 tokens: 67.0 MB of 67.1 MB), then a 5-token call; both bit
    for bit equal to the workspace entry point."""
    T = 16 * (g.SEQ_NOALLOC_MAX_BYTES // (48 * 2304))
    assert g.lib().gdn_seq_workspace_bytes(1, T, 48, 128, 128) <= g.SEQ_NOALLOC_MAX_BYTES
    for c in (inputs.make_case(2502, B=1, NK=16, NV=48, D=128, T=T),
              inputs.make_case(2503, B=1, NK=16, NV=48, D=128, T=5)):
        say("noalloc limit", c.B, c.T)
        oa, sa, ob, sb = _run_pair(g, c, False)
        assert np.array_equal(oa.view(np.uint32), ob.view(np.uint32))
        assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
        assert np.isfinite(oa).all()
    ref_o, ref_s = _oracle(c, False)
    assert out_err(oa, ref_o, c.NV, c.D) < TOL_CHAIN
    assert tile_err(sa, ref_s, c.NV, c.D) < TOL_CHAIN


def test_noalloc_rejects_beyond_the_limit(g):
    """One record past the scratch: GDN_ERR_SCRATCH, and nothing is written."""
    import torch
    T = 16 * (g.SEQ_NOALLOC_MAX_BYTES // (48 * 2304)) + 1
    c = inputs.make_case(2504, B=1, NK=16, NV=48, D=128, T=T)
    say("noalloc too large", T)
    d = {n: dev(getattr(c, n)) for n in ("q", "k", "v", "z", "alpha", "beta", "gn")}
    st = dev(c.state)
    out = torch.full((T, 48 * 128), float("nan"), device="cuda:0")
    assert _call(g, "noalloc", c, st, d, out, False) == 9
    assert bool(torch.isnan(out).all())
    assert np.array_equal(host(st).view(np.uint32), c.state.view(np.uint32))


def test_noalloc_other_head_dim_needs_no_scratch(g):
    """D = 64 runs without a workspace; the entry point takes it as the plain
    sequence call does."""
    c = inputs.make_case(2505, B=2, NK=2, NV=6, D=64, T=21)
    say("noalloc D=64")
    d = {n: dev(getattr(c, n)) for n in ("q", "k", "v", "z", "alpha", "beta", "gn")}
    import torch
    st = dev(c.state)
    out = torch.empty((c.B * c.T, c.NV * c.D), device="cuda:0")
    assert _call(g, "noalloc", c, st, d, out, True) == 0
    ref_o, ref_s = _oracle(c, True)
    assert out_err(host(out), ref_o, c.NV, c.D) < TOL_CHAIN
    assert tile_err(host(st), ref_s, c.NV, c.D) < TOL_CHAIN


def test_noalloc_on_a_side_stream(g):
    """A stream of the current device other than the null stream passes the
    device check; the results match the workspace entry point on that stream
    bit for bit, and the oracle."""
    import torch
    c = inputs.make_case(2506, B=2, NK=16, NV=48, D=128, T=40)
    say("noalloc on a side stream")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        oa, sa, ob, sb = _run_pair(g, c, False)
    assert np.array_equal(oa.view(np.uint32), ob.view(np.uint32))
    assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
    ref_o, ref_s = _oracle(c, False)
    assert out_err(oa, ref_o, c.NV, c.D) < TOL_CHAIN
    assert tile_err(sa, ref_s, c.NV, c.D) < TOL_CHAIN


def test_noalloc_captured_in_a_graph(g):
    """The entry point for callers that cannot allocate, captured once in a HIP
    graph after a first eager call (which resolves the scratch address), then
    replayed three times with eager work and synchronisation in between: every
    replay's output and state equal the same calls made eagerly, bit for bit."""
    import torch
    c = inputs.make_case(2507, B=1, NK=16, NV=48, D=128, T=40)
    say("noalloc in a graph")
    d = {n: dev(getattr(c, n)) for n in ("q", "k", "v", "z", "alpha", "beta", "gn")}
    rows, vw = c.B * c.T, c.NV * c.D
    st_g, st_e = dev(c.state), dev(c.state)
    out_g = torch.empty((rows, vw), device="cuda:0")
    out_e = torch.empty((rows, vw), device="cuda:0")

    def call(st, out):
        assert _call(g, "noalloc", c, st, d, out, False) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(st_g, out_g)                      # first call outside the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(st_g, out_g)
    call(st_e, out_e)                          # the eager copy catches up with the warm-up
    for rep in range(3):
        graph.replay()
        call(st_e, out_e)
        scratch = torch.randn(1 << 20, device="cuda:0").sum()
        torch.cuda.synchronize()
        assert bool(torch.isfinite(scratch))
        assert torch.equal(out_g, out_e), rep
        assert torch.equal(st_g, st_e), rep
