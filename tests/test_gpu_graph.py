"""The entry points replayed from a HIP graph.

A serving loop captures a decode token once and replays it.  Here one graph
holds a fused-norm decode per layer, the int8-quantised epilogue, a
binary16-state decode, a draft verify, the decode with the fused input stage in
both ring modes and both D = 128 sequence entry points (with z: the chunked
kernels and the norm pass).  It is replayed three times, with eager work of the
program between the replays, and after every replay each output and each state
must equal, bit for bit, the same calls made eagerly on copies of the same
buffers: the graph runs the same kernels on the same inputs, and no call
records a memset.
"""
import sys

import numpy as np
import pytest

from gated_deltanet_decode_delta_amd import inputs
from gpu_util import dev, host

pytestmark = pytest.mark.gpu


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


def _buffers(g):
    """Inputs (shared by both copies) and one set of the buffers the calls
    write: states and outputs."""
    import torch
    NK, NV, D = 16, 48, 128
    layers = [inputs.make_case(3100 + l, B=3, NK=NK, NV=NV, D=D) for l in range(3)]
    f16 = inputs.make_case(3200, B=5, NK=NK, NV=NV, D=D)
    ver = inputs.make_case(3300, B=2, NK=NK, NV=NV, D=D, T=3)
    seq = inputs.make_case(3400, B=2, NK=NK, NV=NV, D=D, T=37)
    names = ("q", "k", "v", "z", "alpha", "beta", "gn")
    ins = {"layers": [{n: dev(getattr(c, n)) for n in names} for c in layers],
           "f16": {n: dev(getattr(f16, n)) for n in names},
           "ver": {n: dev(getattr(ver, n)) for n in names},
           "seq": {n: dev(getattr(seq, n)) for n in names}}
    need = g.gdn_seq_workspace_bytes(seq.B, seq.T, NV, D)
    fr = inputs.make_frontend_case(3500, B=3, NK=NK, NV=NV, D=D, taps=4)
    ins["front"] = {n: dev(getattr(fr, n)) for n in ("x", "w", "br", "ar", "dt", "rate", "z", "gn")}

    def fresh():
        nan = float("nan")
        return {
            "layers": [dev(c.state) for c in layers],
            "layer_out": [torch.full((3, NV * D), nan, device="cuda:0") for _ in layers],
            "f16": g.gdn_state_f32_to_f16(dev(f16.state)),
            "f16_out": torch.full((5, NV * D), nan, device="cuda:0").to(torch.bfloat16),
            "ver": dev(ver.state),
            "ver_inter": torch.full((2 * 2, NV * D * D), nan, device="cuda:0"),
            "ver_out": torch.full((2 * 3, NV * D), nan, device="cuda:0"),
            "seq": dev(seq.state),
            "seq_out": torch.full((2 * 37, NV * D), nan, device="cuda:0"),
            "seq_ws_state": dev(seq.state),
            "seq_ws_out": torch.full((2 * 37, NV * D), nan, device="cuda:0"),
            "ws": torch.empty(max(need, 16), dtype=torch.uint8, device="cuda:0"),
            "q8_state": dev(layers[0].state),
            "q8_codes": torch.zeros((3, NV * D), dtype=torch.int8, device="cuda:0"),
            "q8_scales": torch.full((3, NV * D // 32), nan, device="cuda:0"),
            "fr_state": dev(fr.state),
            "fr_ring": dev(fr.ring),
            "fr_out": torch.full((3, NV * D), nan, device="cuda:0"),
            "fr2_state": dev(fr.state),
            "fr2_ring_a": dev(fr.ring),
            "fr2_ring_b": torch.full_like(dev(fr.ring), nan),
            "fr2_out": torch.full((3, NV * D), nan, device="cuda:0"),
        }
    return ins, fresh, (NK, NV, D), seq.eps


def _token(g, ins, w, dims, eps):
    """Every call of one step, on the written buffers `w`."""
    NK, NV, D = dims
    for d, st, out in zip(ins["layers"], w["layers"], w["layer_out"]):
        g.gdn_decode_norm(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"], eps,
                          out=out, num_k_heads=NK, num_v_heads=NV)
    d = ins["layers"][0]
    g.gdn_decode_norm_q(w["q8_state"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"],
                        d["gn"], eps, codes=w["q8_codes"], scales=w["q8_scales"], write_y=False,
                        num_k_heads=NK, num_v_heads=NV)
    f = ins["front"]
    g.gdn_decode_fused(w["fr_state"], w["fr_ring"], f["x"], f["w"], f["br"], f["ar"], f["dt"],
                       f["rate"], f["z"], f["gn"], eps, 1e-6, out=w["fr_out"], num_k_heads=NK,
                       num_v_heads=NV)
    # two ring buffers: one step reads ring a and writes ring b, the next reads b
    # and writes a, so each replay leaves the rings where the next one reads them
    g.gdn_decode_fused(w["fr2_state"], w["fr2_ring_a"], f["x"], f["w"], f["br"], f["ar"], f["dt"],
                       f["rate"], f["z"], f["gn"], eps, 1e-6, out=w["fr2_out"],
                       conv_state_out=w["fr2_ring_b"], num_k_heads=NK, num_v_heads=NV)
    g.gdn_decode_fused(w["fr2_state"], w["fr2_ring_b"], f["x"], f["w"], f["br"], f["ar"], f["dt"],
                       f["rate"], f["z"], f["gn"], eps, 1e-6, out=w["fr2_out"],
                       conv_state_out=w["fr2_ring_a"], num_k_heads=NK, num_v_heads=NV)
    d = ins["f16"]
    g.gdn_decode_f16state(w["f16"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                          eps, out=w["f16_out"], num_k_heads=NK, num_v_heads=NV)
    d = ins["ver"]
    g.gdn_decode_verify(w["ver"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                        eps, out=w["ver_out"], inter_state=w["ver_inter"], num_tokens=3,
                        num_k_heads=NK, num_v_heads=NV, head_dim=D)
    d = ins["seq"]
    g.gdn_recurrence_seq(w["seq"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                         eps, out=w["seq_out"], seq_len=37, num_k_heads=NK, num_v_heads=NV,
                         head_dim=D)
    g.gdn_recurrence_seq_ws(w["seq_ws_state"], d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                            d["z"], d["gn"], eps, out=w["seq_ws_out"], workspace=w["ws"],
                            seq_len=37, num_k_heads=NK, num_v_heads=NV, head_dim=D)


def _same(a, b, what):
    x, y = host(a).view(np.uint8), host(b).view(np.uint8)
    assert x.shape == y.shape and np.array_equal(x, y), what


def _compare(gw, ew, rep):
    for i, (a, b) in enumerate(zip(gw["layers"], ew["layers"])):
        _same(a, b, f"replay {rep}: layer {i} state")
    for i, (a, b) in enumerate(zip(gw["layer_out"], ew["layer_out"])):
        _same(a, b, f"replay {rep}: layer {i} y")
    for k in ("f16", "f16_out", "ver", "ver_inter", "ver_out", "seq", "seq_out", "seq_ws_state",
              "seq_ws_out", "q8_state", "q8_codes", "q8_scales", "fr_state", "fr_ring", "fr_out",
              "fr2_state", "fr2_ring_a", "fr2_ring_b", "fr2_out"):
        _same(gw[k], ew[k], f"replay {rep}: {k}")


def test_graph_replays_match_eager_calls(g):
    import torch
    ins, fresh, dims, eps = _buffers(g)
    gw, ew = fresh(), fresh()          # graph's buffers, eager reference buffers
    torch.cuda.synchronize()
    # warm-up on a side stream (as torch asks before capture), mirrored eagerly
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _token(g, ins, gw, dims, eps)
    torch.cuda.current_stream().wait_stream(side)
    _token(g, ins, ew, dims, eps)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _token(g, ins, gw, dims, eps)   # recorded, not run
    torch.cuda.synchronize()
    _compare(gw, ew, "after capture")
    for rep in range(3):
        say("graph replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        # the program's own eager work between replays
        _token(g, ins, ew, dims, eps)
        scratch = torch.randn(1 << 20, device="cuda:0")
        float(scratch.sum())
        torch.cuda.synchronize()
        _compare(gw, ew, rep)
