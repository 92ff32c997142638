"""Calls on several streams at once.

Apart from the no-allocation entry point's documented static scratch, a call
keeps nothing between calls and shares nothing with another call: every array
it touches is the caller's.  So calls on different buffers may run on different
streams at the same time.  Here three streams (default priority) each run a
chain of calls on their own buffers -- fused-norm decodes, the workspace
sequence path and the workspace-free one, the binary16 decode -- interleaved
call by call from the host, and every result must equal, bit for bit, the same
chains run one after the other on one stream.
"""
import sys

import numpy as np
import pytest

from gated_deltanet_decode_delta_amd import inputs
from gpu_util import dev, host

pytestmark = pytest.mark.gpu

NK, NV, D = 16, 48, 128


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


def _chains(g):
    """Three chains of calls: (inputs, a factory for the buffers they write,
    one step of the chain on those buffers)."""
    import torch
    names = ("q", "k", "v", "z", "alpha", "beta", "gn")
    dec = inputs.make_case(3600, B=16, NK=NK, NV=NV, D=D)
    seq = inputs.make_case(3700, B=2, NK=NK, NV=NV, D=D, T=45)
    f16 = inputs.make_case(3800, B=24, NK=NK, NV=NV, D=D)
    di, si, fi = ({n: dev(getattr(c, n)) for n in names} for c in (dec, seq, f16))
    need = g.gdn_seq_workspace_bytes(seq.B, seq.T, NV, D)
    nan = float("nan")

    def bufs():
        return {"dec": dev(dec.state), "dec_out": torch.full((16, NV * D), nan, device="cuda:0"),
                "seq_ws": dev(seq.state), "seq": dev(seq.state),
                "seq_ws_out": torch.full((seq.B * seq.T, NV * D), nan, device="cuda:0"),
                "seq_out": torch.full((seq.B * seq.T, NV * D), nan, device="cuda:0"),
                "ws": torch.empty(max(need, 16), dtype=torch.uint8, device="cuda:0"),
                "f16": g.gdn_state_f32_to_f16(dev(f16.state)),
                "f16_out": torch.full((24, NV * D), nan, device="cuda:0").to(torch.bfloat16)}

    def step_dec(w):
        d = di
        g.gdn_decode_norm(w["dec"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                          dec.eps, out=w["dec_out"], num_k_heads=NK, num_v_heads=NV)

    def step_seq(w):
        d = si
        g.gdn_recurrence_seq_ws(w["seq_ws"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"],
                                d["gn"], seq.eps, out=w["seq_ws_out"], workspace=w["ws"],
                                seq_len=seq.T, num_k_heads=NK, num_v_heads=NV, head_dim=D)
        g.gdn_recurrence_seq(w["seq"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], None, None,
                             seq.eps, out=w["seq_out"], seq_len=seq.T, num_k_heads=NK,
                             num_v_heads=NV, head_dim=D)

    def step_f16(w):
        d = fi
        g.gdn_decode_f16state(w["f16"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"],
                              d["gn"], f16.eps, out=w["f16_out"], num_k_heads=NK, num_v_heads=NV)

    return bufs, (step_dec, step_seq, step_f16)


def test_three_streams_match_one_stream(g):
    import torch
    bufs, steps = _chains(g)
    ref, par = bufs(), bufs()
    torch.cuda.synchronize()
    rounds = 12
    say("one stream,", rounds, "rounds of each chain")
    for step in steps:
        for _ in range(rounds):
            step(ref)
    torch.cuda.synchronize()
    say("three streams, interleaved")
    streams = [torch.cuda.Stream() for _ in steps]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(rounds):
        for s, step in zip(streams, steps):
            with torch.cuda.stream(s):
                step(par)
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for k in ref:
        if k == "ws":
            continue
        a, b = host(ref[k]).view(np.uint8), host(par[k]).view(np.uint8)
        assert np.array_equal(a, b), k
