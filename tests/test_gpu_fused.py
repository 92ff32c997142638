"""GPU parity of gdn_decode_fused (the input stage -- conv ring, silu, L2 of
q/k, gates -- fused in front of the decode step) against the CPU oracle.

The oracle runs the same front end in double and the pinned step; the ring is
pure data movement and must match bit for bit; o / y and the state must agree
to the one-step fp32 tolerance (1e-5 per head), like the plain decode.
"""
import sys

import numpy as np
import pytest

import oracle as orc
from gated_deltanet_decode_delta_amd import inputs
from gpu_util import dev, host, out_err, tile_err

pytestmark = pytest.mark.gpu

TOL_STEP = 1e-5


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


def _gpu(g, c, norm, split=False):
    """Run the fused step; returns the device arrays and the output.  With
    split, the new ring goes to d["ring_out"] (NaN-filled beforehand) and
    d["ring"] must stay as it was."""
    import torch
    d = {n: dev(getattr(c, n)) for n in ("state", "ring", "x", "w", "br", "ar", "dt", "rate", "z", "gn")}
    d["ring_out"] = torch.full_like(d["ring"], float("nan")) if split else None
    o = g.gdn_decode_fused(d["state"], d["ring"], d["x"], d["w"], d["br"], d["ar"], d["dt"], d["rate"],
                           d["z"] if norm else None, d["gn"] if norm else None, c.eps, c.l2_eps,
                           conv_state_out=d["ring_out"], num_k_heads=c.NK, num_v_heads=c.NV,
                           head_dim=c.D)
    return d, o


def _new_ring(d, c):
    """The ring after the call (taps*C live columns), from wherever it went."""
    live = c.taps * c.C
    if d["ring_out"] is not None:
        assert np.array_equal(host(d["ring"]), c.ring, equal_nan=True)   # old ring only read
        got = host(d["ring_out"])
        assert np.isnan(got[:, live:]).all()                            # pads not written
        return got[:, :live]
    got = host(d["ring"])
    assert np.array_equal(got[:, live:], c.ring[:, live:], equal_nan=True)
    return got[:, :live]


def _oracle(c, norm):
    st, ring = c.state.copy(), c.ring.copy()
    kw = dict(z=c.z, gn=c.gn, eps=c.eps) if norm else {}
    y = orc.fused_decode(st, ring, c.x, c.w, c.br, c.ar, c.dt, c.rate, B=c.B, NK=c.NK, NV=c.NV,
                         D=c.D, taps=c.taps, l2_eps=c.l2_eps, **kw)
    return st, ring, y


@pytest.mark.parametrize("D", [4, 16, 64, 128, 256])
@pytest.mark.parametrize("NV,NK,taps", [(2, 2, 4), (6, 2, 4), (8, 4, 1), (6, 3, 8)])
@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("split", [False, True])
def test_fused_against_oracle(g, D, NV, NK, taps, norm, split):
    B = 3
    c = inputs.make_frontend_case(900 + D + NV + taps, B=B, NK=NK, NV=NV, D=D, taps=taps,
                                  pitch=NV * D * D + 64, ring_pitch=taps * (2 * NK + NV) * D + 12)
    say("fused", D, NV, NK, taps, "norm" if norm else "raw", "split" if split else "in place")
    d, o = _gpu(g, c, norm, split)
    st, ring, y = _oracle(c, norm)
    assert np.array_equal(_new_ring(d, c), ring[:, :c.taps * c.C])
    assert out_err(host(o), y, NV, D) < TOL_STEP
    got = host(d["state"])
    assert tile_err(got, st, NV, D) < TOL_STEP
    assert np.isnan(got[:, NV * D * D:]).all()


@pytest.mark.parametrize("taps", [2, 3, 5, 6, 7])
@pytest.mark.parametrize("split", [False, True])
def test_fused_every_ring_depth(g, taps, split):
    """The ring depths not covered above, on both sides of the short-ring variant
    (taps <= 4): D = 128, the decode's 3:1 pairing, fused norm, a wide enough
    launch (B = 64) that the two-buffer kernel takes its 256-workgroup shape."""
    B, NK, NV, D = 64, 2, 6, 128
    c = inputs.make_frontend_case(940 + taps, B=B, NK=NK, NV=NV, D=D, taps=taps,
                                  ring_pitch=taps * (2 * NK + NV) * D + 4)
    say("fused ring depth", taps, "split" if split else "in place")
    d, o = _gpu(g, c, True, split)
    st, ring, y = _oracle(c, True)
    assert np.array_equal(_new_ring(d, c), ring[:, :c.taps * c.C])
    assert out_err(host(o), y, NV, D) < TOL_STEP
    assert tile_err(host(d["state"]), st, NV, D) < TOL_STEP


@pytest.mark.parametrize("split", [False, True])
def test_fused_real_shape_full_batch(g, split):
    """The decode workload's shapes (B=64, 48 value heads over 16 key heads,
    D=128, 4-tap ring, 1.25x state slot pitch), fused norm: the ring bitwise,
    all outputs and sampled state tiles against the oracle."""
    B, NK, NV, D = 64, 16, 48, 128
    c = inputs.make_frontend_case(950, B=B, NK=NK, NV=NV, D=D, taps=4, pitch=983040)
    say("fused real shape", "split" if split else "in place")
    d, o = _gpu(g, c, True, split)
    st, ring, y = _oracle(c, True)
    assert np.array_equal(_new_ring(d, c), ring)
    assert out_err(host(o), y, NV, D) < TOL_STEP
    got = host(d["state"])
    r = np.random.Generator(np.random.PCG64(31))
    for b in sorted(r.choice(B, 8, replace=False)):
        assert tile_err(got[b:b + 1], st[b:b + 1], NV, D) < TOL_STEP, b
    assert np.isnan(got[:, NV * D * D:]).all()


@pytest.mark.parametrize("split", [False, True])
def test_fused_three_tokens_chain(g, split):
    """Three tokens in a row: the ring carries each token's row into the next
    tokens' convs (with two buffers, they alternate); all steps against the
    oracle, the rings bitwise."""
    import torch
    B, NK, NV, D, taps = 2, 2, 4, 32, 3
    cases = [inputs.make_frontend_case(960 + i, B=B, NK=NK, NV=NV, D=D, taps=taps) for i in range(3)]
    c = cases[0]
    say("fused chain", "split" if split else "in place")
    d = {n: dev(getattr(c, n)) for n in ("state", "ring", "w", "dt", "rate", "gn")}
    rings = [d["ring"], torch.empty_like(d["ring"])] if split else [d["ring"]]
    st, ring = c.state.copy(), c.ring.copy()
    for i, cc in enumerate(cases):
        src = rings[i % len(rings)]
        dst = rings[(i + 1) % 2] if split else None
        o = g.gdn_decode_fused(d["state"], src, dev(cc.x), d["w"], dev(cc.br), dev(cc.ar),
                               d["dt"], d["rate"], dev(cc.z), d["gn"], c.eps, c.l2_eps,
                               conv_state_out=dst, num_k_heads=NK, num_v_heads=NV)
        y = orc.fused_decode(st, ring, cc.x, c.w, cc.br, cc.ar, c.dt, c.rate, B=B, NK=NK, NV=NV, D=D,
                             taps=taps, z=cc.z, gn=c.gn)
        assert out_err(host(o), y, NV, D) < 3 * TOL_STEP, i
        got = rings[(i + 1) % len(rings)]
        assert np.array_equal(host(got), ring), i
    assert tile_err(host(d["state"]), st, NV, D) < 3 * TOL_STEP


def test_fused_equals_frontend_then_decode(g):
    """The fused launch equals the plain decode fed with the oracle's front-end
    outputs rounded to fp32 (the step itself is the same arithmetic)."""
    B, NK, NV, D = 4, 4, 8, 128
    c = inputs.make_frontend_case(970, B=B, NK=NK, NV=NV, D=D, taps=4)
    say("fused == front end + decode")
    d, o = _gpu(g, c, True)
    st, ring = c.state.copy(), c.ring.copy()
    _, q, k, v, al, be = orc.fused_decode(st, ring, c.x, c.w, c.br, c.ar, c.dt, c.rate, B=B, NK=NK,
                                          NV=NV, D=D, taps=4, return_inputs=True)
    st2 = dev(c.state)
    y = g.gdn_decode_norm(st2, dev(q.astype(np.float32)), dev(k.astype(np.float32)),
                          dev(v.astype(np.float32)), dev(al.astype(np.float32)),
                          dev(be.astype(np.float32)), dev(c.z), dev(c.gn), c.eps,
                          num_k_heads=NK, num_v_heads=NV)
    assert out_err(host(o), host(y), NV, D) < 2e-6
    assert tile_err(host(d["state"]), host(st2), NV, D) < 2e-6


def test_fused_validation(g):
    """Bad tap counts, overlapping ring and an LDS need beyond 64 KiB come back
    as status codes before any launch, leaving every buffer untouched."""
    import torch
    c = inputs.make_frontend_case(980, B=2, NK=2, NV=4, D=16, taps=4)
    d = {n: dev(getattr(c, n)) for n in ("state", "ring", "x", "w", "br", "ar", "dt", "rate")}
    say("fused validation")
    w9 = torch.zeros((9, c.C), device="cuda:0")
    with pytest.raises(g.GdnError) as e:
        g.gdn_decode_fused(d["state"], torch.zeros((2, 9 * c.C), device="cuda:0"), d["x"], w9,
                           d["br"], d["ar"], d["dt"], d["rate"], num_k_heads=2, num_v_heads=4,
                           head_dim=16)
    assert e.value.status == 2
    with pytest.raises(g.GdnError) as e:        # ring over the state
        g.gdn_decode_fused(d["state"], d["state"][:, :4 * c.C], d["x"], d["w"], d["br"], d["ar"],
                           d["dt"], d["rate"], num_k_heads=2, num_v_heads=4, head_dim=16)
    assert e.value.status == 5
    with pytest.raises(g.GdnError) as e:        # output over the conv weights
        g.gdn_decode_fused(d["state"], d["ring"], d["x"], d["w"], d["br"], d["ar"], d["dt"],
                           d["rate"], out=d["w"][:2, :64], num_k_heads=2, num_v_heads=4,
                           head_dim=16)
    assert e.value.status == 5
    big = inputs.make_frontend_case(981, B=1, NK=1, NV=64, D=256, taps=1)
    db = {n: dev(getattr(big, n)) for n in ("state", "ring", "x", "w", "br", "ar", "dt", "rate")}
    with pytest.raises(g.GdnError) as e:        # (2 + 64) * 256 floats of LDS features
        g.gdn_decode_fused(db["state"], db["ring"], db["x"], db["w"], db["br"], db["ar"], db["dt"],
                           db["rate"], num_k_heads=1, num_v_heads=64, head_dim=256)
    assert e.value.status == 4
    assert np.array_equal(host(d["state"]), c.state, equal_nan=True)
    assert np.array_equal(host(d["ring"]), c.ring, equal_nan=True)
