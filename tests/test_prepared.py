"""``prepare``: one entry-point call marshalled once and launched again by the
returned object.  On the CPU: the capture itself, through a call that the
library accepts without a launch (an empty batch), and its error cases.  On
the GPU: prepared calls give the bits of direct calls."""
import sys

import numpy as np
import pytest

import gated_deltanet_decode_delta_amd as gdn


def _empty_decode(marker):
    """Stands in for an entry point: marshals an empty gdn_decode (batch 0, no
    launch, GDN_OK) through the binding's capture path and returns marker."""
    gdn._invoke("gdn_decode", (None, 0, None, None, 0, None, 0, None, None, 0, None, 0,
                               0, 1, 1, 128, 128, None))
    return marker


def test_prepare_records_and_repeats_a_call():
    gdn.lib()
    call = gdn.prepare(_empty_decode, "result")
    assert isinstance(call, gdn.PreparedCall)
    assert call() == "result" and call() == "result"
    assert not gdn._CAPTURE.active          # the capture ended with prepare


def test_prepare_of_a_call_the_library_rejects_raises_when_called():
    gdn.lib()

    def bad():
        gdn._invoke("gdn_decode", (None, 0, None, None, 0, None, 0, None, None, 0, None, 0,
                                   -1, 1, 1, 128, 128, None))

    call = gdn.prepare(bad)                   # marshalled, not launched
    with pytest.raises(gdn.GdnError, match="GDN_ERR_SHAPE"):
        call()


def test_prepare_needs_a_launch_and_does_not_nest():
    gdn.lib()
    with pytest.raises(ValueError, match="launches nothing"):
        gdn.prepare(lambda: None)
    with pytest.raises(RuntimeError, match="nested"):
        gdn.prepare(lambda: gdn.prepare(_empty_decode, 1))
    assert not gdn._CAPTURE.active


@pytest.mark.gpu
def test_prepared_calls_match_direct_calls():
    """gdn_decode_norm and gdn_recurrence_seq_ws (its workspace made inside the
    binding and kept by the prepared call), each twice prepared and twice
    direct on copies of the same state: the same bits."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_decode_delta_amd import inputs
    from gpu_util import dev, host
    print("[case] prepared calls", file=sys.stderr, flush=True)
    c = inputs.make_case(2300, B=4, NK=16, NV=48, D=128, T=1)
    d = {n: dev(getattr(c, n)) for n in ("q", "k", "v", "z", "alpha", "beta", "gn")}
    st_a, st_b = dev(c.state), dev(c.state)
    y_b = torch.empty((4, 48 * 128), device="cuda:0")
    call = gdn.prepare(gdn.gdn_decode_norm, st_a, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                       d["z"], d["gn"], c.eps, num_k_heads=16, num_v_heads=48)
    for _ in range(2):
        y_a = call()
        gdn.gdn_decode_norm(st_b, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                            c.eps, out=y_b, num_k_heads=16, num_v_heads=48)
    assert np.array_equal(host(y_a).view(np.uint32), host(y_b).view(np.uint32))
    assert np.array_equal(host(st_a).view(np.uint32), host(st_b).view(np.uint32))

    s = inputs.make_case(2301, B=2, NK=16, NV=48, D=128, T=40)
    e = {n: dev(getattr(s, n)) for n in ("q", "k", "v", "alpha", "beta")}
    st_a, st_b = dev(s.state), dev(s.state)
    call = gdn.prepare(gdn.gdn_recurrence_seq_ws, st_a, e["q"], e["k"], e["v"], e["alpha"],
                       e["beta"], seq_len=40, num_k_heads=16, num_v_heads=48, head_dim=128)
    for _ in range(2):
        o_a = call()
        o_b = gdn.gdn_recurrence_seq_ws(st_b, e["q"], e["k"], e["v"], e["alpha"], e["beta"],
                                        seq_len=40, num_k_heads=16, num_v_heads=48, head_dim=128)
    assert np.array_equal(host(o_a).view(np.uint32), host(o_b).view(np.uint32))
    assert np.array_equal(host(st_a).view(np.uint32), host(st_b).view(np.uint32))
