"""GPU parity on a state pool larger than 2**31 elements.

2800 sequences of 48 value heads at D = 128 make a dense pool of 2.2e9 state
elements (8.8 GB in fp32, 4.4 GB in binary16), so slot offsets, rollback-slot
offsets and the converters' element counts need 64-bit arithmetic: slot 2730
crosses element 2**31 at its head 32, and slot 2731 starts past it.  Every
sequence takes its token inputs from one of four seeded sequences (b mod 4);
sampled slots hold seeded states and one keeps a zero state.  The sampled
sequences are checked against the oracle one by one, at the one-step tolerance.
"""
import sys

import numpy as np
import pytest

import oracle as orc
from gated_deltanet_decode_delta_amd import inputs
from gpu_util import DEV, bf16_ok, dev, host, out_err, tile_err

pytestmark = pytest.mark.gpu

TOL_STEP = 1e-5
TOL_F16 = 3e-3

BIG_B = 2800
NK, NV, D = 16, 48, 128
SLOT = NV * D * D
# sequence -> the seeded sequence (row of a four-sequence case) it takes its
# inputs and initial state from
SAMPLES = {0: 0, 1501: 1, 2730: 2, 2731: 3, 2798: 2}
ZERO = 2799            # keeps a zero initial state; inputs of sequence 3

assert 2730 * SLOT < 2 ** 31 < 2731 * SLOT and (2 ** 31 - 2730 * SLOT) % (D * D) == 0
assert all(b % 4 == r for b, r in SAMPLES.items()) and ZERO % 4 == 3


@pytest.fixture(scope="module")
def g():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_decode_delta_amd as gdn
    gdn.lib()
    return gdn


@pytest.fixture(scope="module", params=["gdn_recurrence_seq", "gdn_recurrence_seq_ws"])
def seq(g, request):
    """Both sequence entry points: without and with the chunk workspace."""
    return getattr(g, request.param)


@pytest.fixture(autouse=True)
def _release():
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _rows(T):
    """Row of the four-sequence case that feeds row b*T + t of the big batch."""
    import torch
    r = torch.arange(BIG_B, device=DEV) % 4
    return (r[:, None] * T + torch.arange(T, device=DEV)[None, :]).reshape(-1)


def _tiled(c, T, names):
    ix = _rows(T)
    return {n: dev(getattr(c, n))[ix].contiguous() for n in names}


def _checked():
    return list(SAMPLES.items()) + [(ZERO, ZERO % 4)]


def _init_state(c, b, r, dtype_bits=False):
    """Initial state of sequence b on the host (row r's seeded state, or zero)."""
    s = np.zeros((1, SLOT), np.float32) if b == ZERO else c.state[r:r + 1].copy()
    return orc.f32_to_f16_bits(s) if dtype_bits else s


def _case_rows(c, r, T):
    sl = slice(r * T, (r + 1) * T)
    names = ("q", "k", "v", "z", "alpha", "beta")
    return {n: np.ascontiguousarray(getattr(c, n)[sl]) for n in names}


def test_large_pool_decode_norm(g):
    import torch
    c = inputs.make_case(2101, B=4, NK=NK, NV=NV, D=D, T=1)
    say("large pool decode_norm", BIG_B)
    st = torch.zeros((BIG_B, SLOT), dtype=torch.float32, device=DEV)
    for b, r in SAMPLES.items():
        st[b] = dev(c.state[r])
    d = _tiled(c, 1, ("q", "k", "v", "z", "alpha", "beta"))
    y = g.gdn_decode_norm(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], dev(c.gn),
                          c.eps, num_k_heads=NK, num_v_heads=NV, head_dim=D)
    got_y = host(y)
    for b, r in _checked():
        ref_st = _init_state(c, b, r)
        x = _case_rows(c, r, 1)
        ref = orc.decode(ref_st, x["q"], x["k"], x["v"], x["alpha"], x["beta"], B=1, NK=NK, NV=NV,
                         Dk=D, Dv=D, z=x["z"], gn=c.gn, eps=c.eps)
        assert out_err(got_y[b:b + 1], ref, NV, D) < TOL_STEP, b
        assert tile_err(host(st[b:b + 1]), ref_st, NV, D) < TOL_STEP, b


def test_large_pool_f16_state(g):
    import torch
    c = inputs.make_case(2102, B=4, NK=NK, NV=NV, D=D, T=1)
    say("large pool f16 state", BIG_B)
    st = torch.zeros((BIG_B, SLOT), dtype=torch.float16, device=DEV)
    for b, r in SAMPLES.items():
        st[b] = dev(orc.f32_to_f16_bits(c.state[r:r + 1])[0].view(np.float16))
    d = _tiled(c, 1, ("q", "k", "v", "z", "alpha", "beta"))
    y = g.gdn_decode_f16state(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], dev(c.gn),
                              c.eps, out_dtype=torch.bfloat16, num_k_heads=NK, num_v_heads=NV,
                              head_dim=D)
    got_y = host(y)
    for b, r in _checked():
        ref16 = _init_state(c, b, r, dtype_bits=True)
        x = _case_rows(c, r, 1)
        ref = orc.decode(ref16, x["q"], x["k"], x["v"], x["alpha"], x["beta"], B=1, NK=NK, NV=NV,
                         Dk=D, Dv=D, z=x["z"], gn=c.gn, eps=c.eps, state_kind=orc.STATE_F16)
        assert bf16_ok(got_y[b:b + 1], ref, NV, D, TOL_F16) <= 1.0, b
        gs = host(st[b:b + 1]).view(np.float16).astype(np.float64)
        assert tile_err(gs, ref16.view(np.float16).astype(np.float64), NV, D) < TOL_F16, b


def test_large_pool_sequence(g, seq):
    """Three tokens per sequence through the chunked sequence kernel."""
    import torch
    T = 3
    c = inputs.make_case(2103, B=4, NK=NK, NV=NV, D=D, T=T)
    say("large pool sequence", BIG_B, T)
    st = torch.zeros((BIG_B, SLOT), dtype=torch.float32, device=DEV)
    for b, r in SAMPLES.items():
        st[b] = dev(c.state[r])
    d = _tiled(c, T, ("q", "k", "v", "alpha", "beta"))
    o = seq(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], seq_len=T,
            num_k_heads=NK, num_v_heads=NV, head_dim=D)
    got_o = host(o)
    for b, r in _checked():
        ref_st = _init_state(c, b, r)
        x = _case_rows(c, r, T)
        ref = orc.seq(ref_st, x["q"], x["k"], x["v"], x["alpha"], x["beta"], B=1, T=T, NK=NK,
                      NV=NV, Dk=D, Dv=D)
        assert out_err(got_o[b * T:(b + 1) * T], ref, NV, D) < TOL_STEP * T, b
        assert tile_err(host(st[b:b + 1]), ref_st, NV, D) < TOL_STEP * T, b


def test_large_pool_verify_rollback(g):
    """Two draft tokens: the rollback slots (one per sequence, 2.2e9 elements in
    all) and the final states, both past element 2**31."""
    import torch
    T = 2
    c = inputs.make_case(2104, B=4, NK=NK, NV=NV, D=D, T=T)
    say("large pool verify", BIG_B, T)
    st = torch.zeros((BIG_B, SLOT), dtype=torch.float32, device=DEV)
    for b, r in SAMPLES.items():
        st[b] = dev(c.state[r])
    d = _tiled(c, T, ("q", "k", "v", "z", "alpha", "beta"))
    out, inter = g.gdn_decode_verify(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"],
                                     dev(c.gn), c.eps, num_tokens=T, num_k_heads=NK,
                                     num_v_heads=NV, head_dim=D)
    got_o = host(out)
    for b, r in _checked():
        x = _case_rows(c, r, T)
        first = _init_state(c, b, r)
        orc.seq(first, x["q"][:1], x["k"][:1], x["v"][:1], x["alpha"][:1], x["beta"][:1], B=1, T=1,
                NK=NK, NV=NV, Dk=D, Dv=D, z=x["z"][:1], gn=c.gn, eps=c.eps)
        ref_st = _init_state(c, b, r)
        ref = orc.seq(ref_st, x["q"], x["k"], x["v"], x["alpha"], x["beta"], B=1, T=T, NK=NK,
                      NV=NV, Dk=D, Dv=D, z=x["z"], gn=c.gn, eps=c.eps)
        assert out_err(got_o[b * T:(b + 1) * T], ref, NV, D) < TOL_STEP * T, b
        assert tile_err(host(inter[b:b + 1]), first, NV, D) < TOL_STEP, b
        assert tile_err(host(st[b:b + 1]), ref_st, NV, D) < TOL_STEP * T, b


def test_large_pool_fused_two_buffers(g):
    """The fused input stage with two ring buffers: the new rings bitwise, the
    outputs and states of the sampled sequences against the oracle."""
    import torch
    c = inputs.make_frontend_case(2105, B=4, NK=NK, NV=NV, D=D, taps=4)
    assert c.state.shape[1] == SLOT
    say("large pool fused", BIG_B)
    st = torch.zeros((BIG_B, SLOT), dtype=torch.float32, device=DEV)
    for b, r in SAMPLES.items():
        st[b] = dev(c.state[r])
    ix = torch.arange(BIG_B, device=DEV) % 4
    d = {n: dev(getattr(c, n))[ix].contiguous() for n in ("ring", "x", "br", "ar", "z")}
    ring_out = torch.full_like(d["ring"], float("nan"))
    y = g.gdn_decode_fused(st, d["ring"], d["x"], dev(c.w), d["br"], d["ar"], dev(c.dt),
                           dev(c.rate), d["z"], dev(c.gn), c.eps, c.l2_eps, conv_state_out=ring_out,
                           num_k_heads=NK, num_v_heads=NV, head_dim=D)
    got_y = host(y)
    live = c.taps * c.C
    for b, r in _checked():
        ref_st = _init_state(c, b, r)
        ring = c.ring[r:r + 1].copy()
        ref = orc.fused_decode(ref_st, ring, c.x[r:r + 1], c.w, c.br[r:r + 1], c.ar[r:r + 1], c.dt,
                               c.rate, B=1, NK=NK, NV=NV, D=D, taps=c.taps, l2_eps=c.l2_eps,
                               z=c.z[r:r + 1], gn=c.gn, eps=c.eps)
        assert np.array_equal(host(ring_out[b:b + 1])[:, :live], ring[:, :live]), b
        assert out_err(got_y[b:b + 1], ref, NV, D) < TOL_STEP, b
        assert tile_err(host(st[b:b + 1]), ref_st, NV, D) < TOL_STEP, b


def test_sequence_rows_past_2_31_bytes(g, seq):
    """The rows of one sequence span more than 2**31 bytes of v: 40 tokens
    with a v row stride of 2**24 + 256 elements.  The workspace entry point
    then runs without its workspace (its state pass addresses a sequence's
    rows with 32-bit byte offsets); both entry points match the oracle."""
    import torch
    T, nk, nv = 40, 1, 2
    vs = 2 ** 24 + 256
    assert T * vs * 4 > 2 ** 31 - 1
    c = inputs.make_case(2107, B=1, NK=nk, NV=nv, D=D, T=T)
    say("sequence, v rows past 2**31 bytes", T, vs)
    big = torch.zeros((T, vs), dtype=torch.float32, device=DEV)   # 2.7 GB
    big[:, :nv * D] = dev(np.ascontiguousarray(c.v.reshape(T, nv * D)))
    v = big[:, :nv * D]
    st = dev(c.state)
    q, k, al, be = (dev(getattr(c, n)) for n in ("q", "k", "alpha", "beta"))
    o = seq(st, q, k, v, al, be, seq_len=T, num_k_heads=nk, num_v_heads=nv, head_dim=D)
    ref_st = c.state.copy()
    ref = orc.seq(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=1, T=T, NK=nk, NV=nv, Dk=D, Dv=D)
    assert out_err(host(o), ref, nv, D) < TOL_STEP * T
    assert tile_err(host(st), ref_st, nv, D) < TOL_STEP * T
