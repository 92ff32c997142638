"""GPU parity of gdn_decode_verify (several draft tokens per launch, with the
state after each token kept for rollback) against the CPU oracle.

Token t of sequence b sits in row b*T + t, as in the oracle's sequence layout,
so the oracle run over the first t + 1 tokens of every sequence gives both the
output rows up to t and the rollback state after token t.
"""
import ctypes
import sys

import numpy as np
import pytest

import oracle as orc
from gated_deltanet_decode_delta_amd import inputs
from gpu_util import dev, host, out_err, tile_err

pytestmark = pytest.mark.gpu

TOL_STEP = 1e-5
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


def _prefix(a, B, T, n):
    """Rows of the first n tokens of every sequence, in b*n + t order."""
    return np.ascontiguousarray(a.reshape(B, T, -1)[:, :n].reshape(B * n, -1))


def _oracle_prefix(c, n, norm):
    """(state after n tokens, outputs of those n tokens) from the oracle."""
    B, T = c.B, c.T
    st = c.state.copy()
    kw = dict(z=_prefix(c.z, B, T, n), gn=c.gn, eps=1e-6) if norm else {}
    out = orc.seq(st, _prefix(c.q, B, T, n), _prefix(c.k, B, T, n), _prefix(c.v, B, T, n),
                  _prefix(c.alpha, B, T, n), _prefix(c.beta, B, T, n), B=B, T=n, NK=c.NK,
                  NV=c.NV, Dk=c.D, Dv=c.D, **kw)
    return st, out


def _run_verify(g, c, norm, T):
    d = {n: dev(getattr(c, n)) for n in ("q", "k", "v", "alpha", "beta", "z", "gn")}
    st = dev(c.state)
    out, inter = g.gdn_decode_verify(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                     d["z"] if norm else None, d["gn"] if norm else None, 1e-6,
                                     num_tokens=T, num_k_heads=c.NK, num_v_heads=c.NV,
                                     head_dim=c.D)
    return st, out, inter


@pytest.mark.parametrize("D", [4, 16, 64, 128, 256])
@pytest.mark.parametrize("T", [1, 2, 5, 8])
@pytest.mark.parametrize("norm", [False, True])
def test_verify_against_oracle_prefixes(g, D, T, norm):
    """Every rollback slot equals the oracle's state after that many tokens, the
    final state the state after all T, and each output row the oracle's."""
    B, NK, NV = 3, 2, 6
    c = inputs.make_case(700 + D + 10 * T, B=B, NK=NK, NV=NV, D=D, T=T)
    say("verify", D, T, "norm" if norm else "raw")
    st, out, inter = _run_verify(g, c, norm, T)
    ref_state, ref_out = _oracle_prefix(c, T, norm)
    assert out_err(host(out), ref_out, NV, D) < TOL_STEP * T
    assert tile_err(host(st), ref_state, NV, D) < TOL_STEP * T
    if T > 1:
        got = host(inter).reshape(B, T - 1, -1)
        for t in range(T - 1):
            ref_t, _ = _oracle_prefix(c, t + 1, norm)
            assert tile_err(got[:, t], ref_t, NV, D) < TOL_STEP * (t + 1), t
    else:
        assert inter is None


def test_verify_two_tokens_full_batch_padded_pool(g):
    """The two-token draft check on the decode workload's shapes: 64 sequences of
    48 value heads over 16 key heads, D = 128, slots 983040 floats apart (a pad
    that must stay untouched); sampled heads against the oracle."""
    B, NK, NV, D, T = 64, 16, 48, 128, 2
    c = inputs.make_case(71, B=B, NK=NK, NV=NV, D=D, T=T, pitch=983040)
    say("verify full batch", B, T)
    st, out, inter = _run_verify(g, c, True, T)
    got_state, got_out, got_inter = host(st), host(out), host(inter)
    dense = NV * D * D
    assert np.isnan(got_state[:, dense:]).all()           # the pad is never touched
    r = np.random.Generator(np.random.PCG64(17))
    for b in sorted(r.choice(B, size=6, replace=False)):
        one = inputs.Case(B=1, T=T, NK=NK, NV=NV, D=D, pitch=c.pitch,
                          state=c.state[b:b + 1].copy(),
                          q=c.q[b * T:(b + 1) * T], k=c.k[b * T:(b + 1) * T],
                          v=c.v[b * T:(b + 1) * T], z=c.z[b * T:(b + 1) * T],
                          alpha=c.alpha[b * T:(b + 1) * T], beta=c.beta[b * T:(b + 1) * T],
                          gn=c.gn)
        ref_state, ref_out = _oracle_prefix(one, T, True)
        ref_1, _ = _oracle_prefix(one, 1, True)
        assert out_err(got_out[b * T:(b + 1) * T], ref_out, NV, D) < TOL_STEP * T, b
        assert tile_err(got_state[b:b + 1], ref_state, NV, D) < TOL_STEP * T, b
        assert tile_err(got_inter[b:b + 1], ref_1, NV, D) < TOL_STEP, b


def test_verify_equals_chained_decode(g):
    """Eight tokens in one verify launch == eight chained single-token calls: the
    final state, every rollback slot and every output (fp32 rounding only)."""
    B, NK, NV, D, T = 4, 4, 8, 128, 8
    c = inputs.make_case(72, B=B, NK=NK, NV=NV, D=D, T=T)
    say("verify == chained decode")
    d = {n: dev(getattr(c, n)) for n in ("q", "k", "v", "alpha", "beta", "z", "gn")}
    st_v, out_v, inter_v = _run_verify(g, c, True, T)
    st = dev(c.state)
    got_inter = host(inter_v).reshape(B, T - 1, -1)
    got_out = host(out_v)
    for t in range(T):
        rows = [b * T + t for b in range(B)]
        y = host(g.gdn_decode_norm(st, d["q"][rows], d["k"][rows], d["v"][rows], d["alpha"][rows],
                                   d["beta"][rows], d["z"][rows], d["gn"], 1e-6, num_k_heads=NK,
                                   num_v_heads=NV))
        assert out_err(got_out[rows], y, NV, D) < 1e-6, t
        if t + 1 < T:
            assert tile_err(got_inter[:, t], host(st), NV, D) < 1e-6, t
    assert tile_err(host(st_v), host(st), NV, D) < 1e-6


def test_verify_rollback_then_continue(g):
    """Speculative use: verify 4 draft tokens, reject after the second, restore
    the rollback slot and decode the corrected token from it."""
    import torch
    B, NK, NV, D, T = 2, 2, 4, 64, 4
    c = inputs.make_case(73, B=B, NK=NK, NV=NV, D=D, T=T)
    fix = inputs.make_case(74, B=B, NK=NK, NV=NV, D=D, T=1)
    say("verify rollback")
    st, _, inter = _run_verify(g, c, False, T)
    keep = 2                                     # tokens 0 and 1 accepted
    st.copy_(inter.view(B, T - 1, -1)[:, keep - 1])
    o = g.gdn_decode(st, dev(fix.q), dev(fix.k), dev(fix.v), dev(fix.alpha), dev(fix.beta),
                     num_k_heads=NK, num_v_heads=NV, head_dim=D)
    ref_state, _ = _oracle_prefix(c, keep, False)
    ref_o = orc.seq(ref_state, fix.q, fix.k, fix.v, fix.alpha, fix.beta, B=B, T=1, NK=NK, NV=NV,
                    Dk=D, Dv=D)
    torch.cuda.synchronize()
    assert out_err(host(o), ref_o, NV, D) < TOL_STEP * 3
    assert tile_err(host(st), ref_state, NV, D) < TOL_STEP * 3


def test_verify_validation(g):
    """Token count outside 1..8, a missing or overlapping rollback buffer and a
    short rollback pitch come back as status codes before any launch."""
    import torch
    B, NK, NV, D = 2, 2, 4, 16
    c = inputs.make_case(75, B=B, NK=NK, NV=NV, D=D, T=9)
    d = {n: dev(getattr(c, n)) for n in ("q", "k", "v", "alpha", "beta")}
    st = dev(c.state)
    slot = NV * D * D
    lib = g.lib()
    vp = ctypes.c_void_p

    def call(T, inter, pitch, state=st):
        return lib.gdn_decode_verify(vp(state.data_ptr()), slot, inter, pitch,
                                     vp(d["q"].data_ptr()), vp(d["k"].data_ptr()), NK * D,
                                     vp(d["v"].data_ptr()), NV * D, vp(d["alpha"].data_ptr()),
                                     vp(d["beta"].data_ptr()), NV, None, 0, None, 1e-6,
                                     vp(out.data_ptr()), NV * D, B, T, NK, NV, D, D, None)

    out = torch.zeros(B * 9, NV * D, device="cuda:0")
    inter = torch.zeros(B * 8, slot, device="cuda:0")
    ip = vp(inter.data_ptr())
    say("verify validation")
    assert call(9, ip, slot) == 2                    # more than 8 tokens
    assert call(0, ip, slot) == 2                    # no token
    assert call(3, None, slot) == 1                  # rollback buffer required
    assert call(3, ip, slot - 4) == 3                # slots overlap each other
    assert call(3, vp(inter.data_ptr() + 4), slot) == 3   # misaligned
    assert call(3, vp(st.data_ptr()), slot) == 5     # rollback over the state
    assert (host(inter) == 0).all() and (host(out) == 0).all()
    assert np.array_equal(host(st), c.state)
    assert call(1, None, 0) == 0                     # one token needs no rollback buffer
