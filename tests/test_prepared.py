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


def _bits(t):
    from gpu_util import host
    return host(t).view(np.uint16 if t.dtype in (_torch().float16, _torch().bfloat16) else
                        (np.uint8 if t.dtype == _torch().int8 else np.uint32))


def _torch():
    import torch
    return torch


@pytest.mark.gpu
@pytest.mark.parametrize("entry", ["gdn_decode", "gdn_decode_norm_bf16", "gdn_decode_norm_q",
                                   "gdn_decode_f16state", "gdn_recurrence_seq",
                                   "gdn_recurrence_seq_noalloc", "gdn_decode_verify",
                                   "gdn_decode_fused", "gdn_state_f32_to_f16"])
def test_prepared_call_of_every_entry_point(entry):
    """Each entry point twice through a prepared call and twice directly, on
    copies of the same inputs and state: the same bits in every output and in
    the state."""
    torch = _torch()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_decode_delta_amd import inputs
    from gpu_util import dev
    print("[case] prepared", entry, file=sys.stderr, flush=True)
    B, NK, NV, D = 3, 2, 6, 128
    T = 5 if entry in ("gdn_recurrence_seq", "gdn_recurrence_seq_noalloc", "gdn_decode_verify") else 1
    if entry == "gdn_decode_fused":
        c = inputs.make_frontend_case(2310, B=B, NK=NK, NV=NV, D=D)
        names = ("x", "w", "br", "ar", "dt", "rate", "z", "gn")
    else:
        c = inputs.make_case(2311, B=B, NK=NK, NV=NV, D=D, T=T)
        names = ("q", "k", "v", "z", "alpha", "beta", "gn")
    d = {n: dev(getattr(c, n)) for n in names}

    def run(state, ring=None):
        """The entry point's call on this state (and ring), as (fn, args, kwargs)."""
        if entry == "gdn_decode":
            return gdn.gdn_decode, (state, d["q"], d["k"], d["v"], d["alpha"], d["beta"]), \
                dict(num_k_heads=NK, num_v_heads=NV, head_dim=D)
        if entry == "gdn_decode_norm_bf16":
            return gdn.gdn_decode_norm, (state, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"],
                                         d["gn"], c.eps), \
                dict(out_dtype=torch.bfloat16, num_k_heads=NK, num_v_heads=NV)
        if entry == "gdn_decode_norm_q":
            return gdn.gdn_decode_norm_q, (state, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"],
                                           d["gn"], c.eps), dict(num_k_heads=NK, num_v_heads=NV)
        if entry == "gdn_decode_f16state":
            return gdn.gdn_decode_f16state, (state, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                             d["z"], d["gn"], c.eps), \
                dict(out_dtype=torch.bfloat16, num_k_heads=NK, num_v_heads=NV)
        if entry in ("gdn_recurrence_seq", "gdn_recurrence_seq_noalloc"):
            return getattr(gdn, entry), (state, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"],
                                         d["gn"], c.eps), \
                dict(seq_len=T, num_k_heads=NK, num_v_heads=NV)
        if entry == "gdn_decode_verify":
            return gdn.gdn_decode_verify, (state, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"],
                                           d["gn"], c.eps), \
                dict(num_tokens=T, num_k_heads=NK, num_v_heads=NV)
        if entry == "gdn_decode_fused":
            return gdn.gdn_decode_fused, (state, ring, d["x"], d["w"], d["br"], d["ar"], d["dt"],
                                          d["rate"], d["z"], d["gn"], 1e-6, 1e-6), \
                dict(num_k_heads=NK, num_v_heads=NV)
        return gdn.gdn_state_f32_to_f16, (state,), {}

    def fresh():
        st = dev(c.state)
        if entry == "gdn_decode_f16state":
            st = gdn.gdn_state_f32_to_f16(st)
        ring = dev(c.ring) if entry == "gdn_decode_fused" else None
        return st, ring

    def flat(res):
        return [r for r in (res if isinstance(res, tuple) else (res,)) if r is not None]

    st_a, ring_a = fresh()
    fn, args, kw = run(st_a, ring_a)
    call = gdn.prepare(fn, *args, **kw)
    st_b, ring_b = fresh()
    for _ in range(2):
        got_a = flat(call())
        fn, args, kw = run(st_b, ring_b)
        got_b = flat(fn(*args, **kw))
    pairs = list(zip(got_a, got_b)) + [(st_a, st_b)]
    if ring_a is not None:
        pairs.append((ring_a, ring_b))
    for x, y in pairs:
        assert np.array_equal(_bits(x), _bits(y))
