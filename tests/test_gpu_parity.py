"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every case draws seeded inputs, runs the library on cuda:0 and the oracle on
the host on the same arrays, and compares per head (tile or output vector):
max |gpu - oracle| / max |oracle| must stay under the stated tolerance --
1e-5 for one fp32 step, 1e-4 after chained steps (up to 4096), 3e-3 for a
binary16 state; bf16 outputs may also differ by half a bf16 ulp.  Full-size
workloads are checked on every head when the oracle is fast enough, otherwise
on sampled heads that the oracle computes one by one.
"""
import functools
import os
import sys

import numpy as np
import pytest

import oracle as orc
from gated_deltanet_decode_delta_amd import inputs
from gpu_util import bf16_ok, dev, host, normed_output_errors, out_err, tile_err

pytestmark = pytest.mark.gpu

TOL_STEP = 1e-5
TOL_CHAIN = 1e-4
TOL_F16 = 3e-3


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


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _dev_case(c):
    return dict(q=dev(c.q), k=dev(c.k), v=dev(c.v), z=dev(c.z), alpha=dev(c.alpha),
                beta=dev(c.beta), gn=dev(c.gn))


# host threads for the oracle over full-size workloads (distinct heads run on
# distinct threads; the result is the same oracle's, head by head)
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def _all_heads(B, NV):
    return [(b, h) for b in range(B) for h in range(NV)]


def _repeat_rows(a, B, n):
    """Row b of a [B, W] array repeated n times: rows b*n .. b*n + n - 1 (the
    same inputs on every call, as one n-token sequence per b)."""
    return np.ascontiguousarray(np.repeat(a, n, axis=0))


@functools.lru_cache(maxsize=3)
def _sequence_reference(init, norm):
    """The sequence workload and the oracle's outputs and final state over
    every head and all 4096 tokens, computed once for both entry points."""
    c = inputs.config_case("sequence", state_init=init)
    ref_state = c.state.copy()
    kw = dict(z=c.z, gn=c.gn, eps=c.eps) if norm else {}
    ref = orc.seq_head_threaded(ref_state, c.q, c.k, c.v, c.alpha, c.beta, B=c.B, T=c.T,
                                NK=c.NK, NV=c.NV, Dk=c.D, Dv=c.D, heads=_all_heads(c.B, c.NV),
                                threads=ORACLE_THREADS, **kw)
    return c, ref, ref_state


# --------------------------------------------------------------------------- 1
def test_tiny_config_all_paths(g):
    """Miniature (NV=2, NK=1, D=4, 8 tokens): decode, decode_norm and the
    sequence kernel (raw and normed) against the oracle token by token."""
    c = inputs.config_case("tiny")
    B, T, NK, NV, D = c.B, c.T, c.NK, c.NV, c.D
    say("tiny", B, T, NK, NV, D)
    ref_state = c.state.copy()
    ref_y = orc.seq(ref_state, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D, Dv=D,
                    z=c.z, gn=c.gn)
    ref_state_raw = c.state.copy()
    ref_o = orc.seq(ref_state_raw, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D,
                    Dv=D)
    d = _dev_case(c)
    st_n, st_r = dev(c.state), dev(c.state)
    for t in range(T):
        sl = slice(t, t + 1)
        y = g.gdn_decode_norm(st_n, d["q"][sl], d["k"][sl], d["v"][sl], d["alpha"][sl],
                              d["beta"][sl], d["z"][sl], d["gn"], c.eps, num_k_heads=NK,
                              num_v_heads=NV)
        o = g.gdn_decode(st_r, d["q"][sl], d["k"][sl], d["v"][sl], d["alpha"][sl], d["beta"][sl],
                         num_k_heads=NK, num_v_heads=NV, head_dim=D)
        st_ref_t = c.state.copy()
        orc.seq(st_ref_t, c.q[:t + 1], c.k[:t + 1], c.v[:t + 1], c.alpha[:t + 1], c.beta[:t + 1],
                B=1, T=t + 1, NK=NK, NV=NV, Dk=D, Dv=D)
        assert out_err(host(y), ref_y[sl], NV, D) < TOL_STEP, t
        assert out_err(host(o), ref_o[sl], NV, D) < TOL_STEP, t
        assert tile_err(host(st_r), st_ref_t, NV, D) < TOL_STEP, t
        assert tile_err(host(st_n), st_ref_t, NV, D) < TOL_STEP, t
    st_s = dev(c.state)
    o_seq = g.gdn_recurrence_seq(st_s, d["q"], d["k"], d["v"], d["alpha"], d["beta"], seq_len=T,
                                 num_k_heads=NK, num_v_heads=NV, head_dim=D)
    assert out_err(host(o_seq), ref_o, NV, D) < TOL_STEP
    assert tile_err(host(st_s), ref_state_raw, NV, D) < TOL_STEP
    st_s = dev(c.state)
    y_seq = g.gdn_recurrence_seq(st_s, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"],
                                 d["gn"], c.eps, seq_len=T, num_k_heads=NK, num_v_heads=NV)
    assert out_err(host(y_seq), ref_y, NV, D) < TOL_STEP
    assert tile_err(host(st_s), ref_state, NV, D) < TOL_STEP


# --------------------------------------------------------------------------- 2
def test_real_head_layers(g):
    """Real head shape (B=1, NV=48, NK=16, D=128), fused norm fp32: one token
    over all 48 independent layer states (the timed workload's inputs), every
    head of every layer checked."""
    for layer in range(inputs.CONFIGS["real_head"]["layers"]):
        c = inputs.real_head_layer(layer)
        say("real_head layer", layer)
        ref_state = c.state.copy()
        ref = orc.decode(ref_state, c.q, c.k, c.v, c.alpha, c.beta, B=1, NK=16, NV=48, Dk=128,
                         Dv=128, z=c.z, gn=c.gn, eps=c.eps)
        d = _dev_case(c)
        st = dev(c.state)
        y = g.gdn_decode_norm(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                              c.eps, num_k_heads=16, num_v_heads=48)
        assert out_err(host(y), ref, 48, 128) < TOL_STEP
        assert tile_err(host(st), ref_state, 48, 128) < TOL_STEP


# --------------------------------------------------------------------------- 3
def test_batched_padded_pool_100_calls(g):
    """B=64 with a 1.25x slot pitch (NaN pads), fused norm fp32: every head after
    call 1 and after call 100; pads untouched."""
    import torch
    c = inputs.config_case("batched")
    B, NK, NV, D = c.B, c.NK, c.NV, c.D
    say("batched B=64 pitch", c.pitch)
    d = _dev_case(c)
    st = dev(c.state)
    ref_state = c.state.copy()
    ref = orc.decode(ref_state, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D,
                     z=c.z, gn=c.gn, eps=c.eps)
    y = g.gdn_decode_norm(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                          c.eps, num_k_heads=NK, num_v_heads=NV)
    got_state = host(st)
    assert out_err(host(y), ref, NV, D) < TOL_STEP
    assert tile_err(got_state, ref_state, NV, D) < TOL_STEP
    assert np.isnan(got_state[:, NV * D * D:]).all()
    for _ in range(99):
        y = g.gdn_decode_norm(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                              c.eps, out=y, num_k_heads=NK, num_v_heads=NV)
    # calls 2 .. 100 repeat the same inputs: 99 more oracle steps on every head,
    # run as one 99-token sequence per batch entry (rows b*99 .. b*99 + 98)
    n = 99
    rep = {name: _repeat_rows(getattr(c, name), B, n) for name in ("q", "k", "v", "z", "alpha", "beta")}
    ref = orc.seq_head_threaded(ref_state, rep["q"], rep["k"], rep["v"], rep["alpha"], rep["beta"],
                                B=B, T=n, NK=NK, NV=NV, Dk=D, Dv=D, heads=_all_heads(B, NV),
                                threads=ORACLE_THREADS, z=rep["z"], gn=c.gn, eps=c.eps)
    ref_last = ref[n - 1::n]   # the output of call 100 for every sequence
    got_state, got_y = host(st), host(y)
    assert np.isnan(got_state[:, NV * D * D:]).all()
    assert tile_err(got_state, ref_state, NV, D) < TOL_CHAIN
    # The same inputs 100 times drive each head's state toward v k^T, so o = S'q
    # becomes a cancellation where k.q is near 0 (condition numbers up to ~2e4
    # here): fp32 evaluation of any order then errs by ~1e-3 relative to |o|.
    # Every head is held to the tolerance relative to the size of o's summands;
    # heads whose output is not such a cancellation (kappa <= 100) also to the
    # plain measure relative to |y|.
    plain, scaled, kappa = normed_output_errors(got_y, ref_last, ref_state, c.q, c.z, c.gn, NV,
                                                NK, D, c.eps)
    assert scaled.max() < TOL_CHAIN, (scaled.max(), int(scaled.argmax()))
    well = kappa <= 100
    assert well.sum() > 0.9 * well.size
    assert plain[well].max() < TOL_CHAIN, (plain[well].max(), kappa[well].max())
    del torch


def test_batched_raw_decode_and_packed_rows(g):
    """gdn_decode (raw o) at B=64, and q|k|v read from one packed projection row
    ([B, 2*NK*D + NV*D]) with z from a wider row, through element strides."""
    c = inputs.config_case("batched")
    B, NK, NV, D = c.B, c.NK, c.NV, c.D
    say("batched raw + packed rows")
    ref_state = c.state.copy()
    ref_o = orc.decode(ref_state, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D)
    d = _dev_case(c)
    st = dev(c.state)
    o = g.gdn_decode(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], num_k_heads=NK,
                     num_v_heads=NV, head_dim=D)
    assert out_err(host(o), ref_o, NV, D) < TOL_STEP
    assert tile_err(host(st), ref_state, NV, D) < TOL_STEP

    qk = NK * D
    W = 2 * qk + NV * D
    packed = np.zeros((B, W), np.float32)
    packed[:, :qk], packed[:, qk:2 * qk], packed[:, 2 * qk:] = c.q, c.k, c.v
    zrow = np.zeros((B, 2 * qk + 2 * NV * D), np.float32)
    zrow[:, 2 * qk + NV * D:] = c.z
    ab = np.zeros((B, 2 * NV), np.float32)
    ab[:, :NV], ab[:, NV:] = c.beta, c.alpha
    pk, zr, abd = dev(packed), dev(zrow), dev(ab)
    ref_state = c.state.copy()
    ref_y = orc.decode(ref_state, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D,
                       z=c.z, gn=c.gn, eps=c.eps)
    st = dev(c.state)
    y = g.gdn_decode_norm(st, pk[:, :qk], pk[:, qk:2 * qk], pk[:, 2 * qk:], abd[:, NV:],
                          abd[:, :NV], zr[:, 2 * qk + NV * D:], d["gn"], c.eps, num_k_heads=NK,
                          num_v_heads=NV)
    assert out_err(host(y), ref_y, NV, D) < TOL_STEP
    assert tile_err(host(st), ref_state, NV, D) < TOL_STEP

    # raw o from the packed rows into a window of a wider NaN-filled buffer (the
    # wide raw launch splits each head's rows over two workgroups)
    import torch
    ref_state = c.state.copy()
    ref_o = orc.decode(ref_state, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D)
    st = dev(c.state)
    wide = torch.full((B, NV * D + 36), float("nan"), device="cuda:0")
    g.gdn_decode(st, pk[:, :qk], pk[:, qk:2 * qk], pk[:, 2 * qk:], abd[:, NV:], abd[:, :NV],
                 out=wide[:, 4:4 + NV * D], num_k_heads=NK, num_v_heads=NV, head_dim=D)
    w = host(wide)
    assert out_err(w[:, 4:4 + NV * D], ref_o, NV, D) < TOL_STEP
    assert np.isnan(w[:, :4]).all() and np.isnan(w[:, 4 + NV * D:]).all()
    assert tile_err(host(st), ref_state, NV, D) < TOL_STEP


# --------------------------------------------------------------------------- 4
def test_fp16_state_full_batch(g):
    """B=256 binary16 pool from an fp32 N(0, 0.02) init through the converter
    (bitwise against the oracle's RNE), then one fused-norm step with bf16 out."""
    import torch
    c = inputs.config_case("fp16_state")
    B, NK, NV, D = c.B, c.NK, c.NV, c.D
    say("fp16 state B=256")
    st32 = dev(c.state)
    st16 = g.gdn_state_f32_to_f16(st32)
    ref16 = orc.f32_to_f16_bits(c.state)
    got16 = host(st16)
    assert np.array_equal(got16, ref16)
    del st32
    d = _dev_case(c)
    y = g.gdn_decode_f16state(st16, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"],
                              d["gn"], c.eps, out_dtype=torch.bfloat16, num_k_heads=NK,
                              num_v_heads=NV)
    ref_y = orc.seq_head_threaded(ref16, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=1, NK=NK, NV=NV,
                                  Dk=D, Dv=D, heads=_all_heads(B, NV), threads=ORACLE_THREADS,
                                  z=c.z, gn=c.gn, eps=c.eps, state_kind=orc.STATE_F16)
    got16, got_y = host(st16), host(y)
    for b0 in range(0, B, 32):   # every head, 32 sequences at a time (bounded host memory)
        sl = slice(b0, b0 + 32)
        gs = got16[sl].view(np.float16).astype(np.float64)
        rs = ref16[sl].view(np.float16).astype(np.float64)
        assert tile_err(gs, rs, NV, D) < TOL_F16, b0
        assert bf16_ok(got_y[sl], ref_y[sl], NV, D, TOL_F16) <= 1.0, b0


def test_fp16_state_padded_pitch_raw_and_f32(g):
    """binary16 pool with a padded pitch (pads hold a canary pattern), raw o and
    fp32 y outputs, several steps."""
    import torch
    B, NK, NV, D = 3, 2, 4, 64
    c = inputs.make_case(45, B=B, NK=NK, NV=NV, D=D, T=1)
    pitch = NV * D * D + 24
    s16 = np.full((B, pitch), 0x7E01, np.uint16)
    s16[:, :NV * D * D] = orc.f32_to_f16_bits(c.state)
    st = dev(s16.view(np.float16))
    ref = s16.copy()
    d = _dev_case(c)
    say("fp16 padded pitch")
    for step in range(3):
        o = g.gdn_decode_f16state(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                  num_k_heads=NK, num_v_heads=NV, head_dim=D)
        ref_o = orc.decode(ref, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D,
                           state_kind=orc.STATE_F16)
        assert out_err(host(o), ref_o, NV, D) < TOL_F16, step
    y = g.gdn_decode_f16state(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                              c.eps, out_dtype=torch.float32, num_k_heads=NK, num_v_heads=NV)
    ref_y = orc.decode(ref, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D, z=c.z,
                       gn=c.gn, eps=c.eps, state_kind=orc.STATE_F16)
    assert out_err(host(y), ref_y, NV, D) < TOL_F16
    got = host(st)
    assert (got[:, NV * D * D:] == 0x7E01).all()
    assert tile_err(got[:, :NV * D * D].view(np.float16).astype(np.float64),
                    ref[:, :NV * D * D].view(np.float16).astype(np.float64), NV, D) < TOL_F16


# --------------------------------------------------------------------------- 5
def _check_sequence(got_o, got_s, ref, ref_state, T, NV, D):
    """Every head: each token's output vector and the final state tile."""
    for r0 in range(0, got_o.shape[0], T):   # one sequence at a time (bounded host memory)
        assert out_err(got_o[r0:r0 + T], ref[r0:r0 + T], NV, D) < TOL_CHAIN, r0 // T
    assert tile_err(got_s, ref_state, NV, D) < TOL_CHAIN


@pytest.mark.parametrize("init", ["zero", "normal"])
def test_sequence_4096_tokens(g, seq, init):
    """B=4, T=4096, NV=48, NK=16, D=128: every head through 4096 oracle steps
    (every token's output and the final state)."""
    c, ref, ref_state = _sequence_reference(init, False)
    B, T, NK, NV, D = c.B, c.T, c.NK, c.NV, c.D
    say("sequence", init, B, T)
    d = _dev_case(c)
    st = dev(c.state)
    o = seq(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], seq_len=T,
            num_k_heads=NK, num_v_heads=NV, head_dim=D)
    _check_sequence(host(o), host(st), ref, ref_state, T, NV, D)


def test_sequence_4096_tokens_fused_norm(g, seq):
    """The full sequence workload with z (the raw pass, then the gated norm over
    the output rows): every head through 4096 oracle steps, every token's y and
    the final state."""
    c, ref, ref_state = _sequence_reference("normal", True)
    B, T, NK, NV, D = c.B, c.T, c.NK, c.NV, c.D
    say("sequence norm", B, T)
    d = _dev_case(c)
    st = dev(c.state)
    y = seq(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"], c.eps,
            seq_len=T, num_k_heads=NK, num_v_heads=NV)
    _check_sequence(host(y), host(st), ref, ref_state, T, NV, D)


def test_sequence_fused_norm_ragged(g, seq):
    """Sequence kernel with z (fused gated norm), a length that is not a multiple
    of the staging chunk, every head."""
    B, T, NK, NV, D = 2, 37, 16, 48, 128
    c = inputs.make_case(57, B=B, NK=NK, NV=NV, D=D, T=T)
    say("sequence norm ragged T=37")
    d = _dev_case(c)
    st = dev(c.state)
    y = seq(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
            c.eps, seq_len=T, num_k_heads=NK, num_v_heads=NV)
    ref_state = c.state.copy()
    ref = orc.seq(ref_state, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D, Dv=D,
                  z=c.z, gn=c.gn, eps=c.eps)
    assert out_err(host(y), ref, NV, D) < TOL_CHAIN
    assert tile_err(host(st), ref_state, NV, D) < TOL_CHAIN


def test_sequence_norm_five_sequences(g, seq):
    """With z at B=5 (960 state-pass workgroups of the workspace path at NV=48,
    more than the device holds at once, and 320 quarters in the kernel without
    a workspace): every head's outputs and state against the oracle."""
    B, T, NK, NV, D = 5, 40, 16, 48, 128
    c = inputs.make_case(58, B=B, NK=NK, NV=NV, D=D, T=T)
    say("sequence norm B=5 T=40")
    d = _dev_case(c)
    st = dev(c.state)
    y = seq(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
            c.eps, seq_len=T, num_k_heads=NK, num_v_heads=NV)
    ref_state = c.state.copy()
    ref = orc.seq(ref_state, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D, Dv=D,
                  z=c.z, gn=c.gn, eps=c.eps)
    assert out_err(host(y), ref, NV, D) < TOL_CHAIN
    assert tile_err(host(st), ref_state, NV, D) < TOL_CHAIN


def test_sequence_equals_chained_decode(g, seq):
    """T tokens in one sequence launch == T chained single-token launches (1e-4)."""
    B, T, NK, NV, D = 3, 20, 4, 8, 128
    c = inputs.make_case(58, B=B, NK=NK, NV=NV, D=D, T=T)
    say("seq == chained decode")
    d = _dev_case(c)
    st_seq = dev(c.state)
    o_seq = host(seq(st_seq, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                     seq_len=T, num_k_heads=NK, num_v_heads=NV, head_dim=D))
    st = dev(c.state)
    o_chain = np.zeros_like(o_seq)
    for t in range(T):
        rows = [b * T + t for b in range(B)]
        o_chain[rows] = host(g.gdn_decode(st, d["q"][rows], d["k"][rows], d["v"][rows],
                                          d["alpha"][rows], d["beta"][rows], num_k_heads=NK,
                                          num_v_heads=NV, head_dim=D))
    assert out_err(o_seq, o_chain, NV, D) < TOL_CHAIN
    assert tile_err(host(st_seq), host(st), NV, D) < TOL_CHAIN


# ------------------------------------------------------------ dims and shapes
@pytest.mark.parametrize("D", [4, 8, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("NV,NK", [(2, 2), (6, 2), (8, 4)])
def test_every_head_dim_all_entry_points(g, D, NV, NK):
    import torch
    B, T = 3, 19
    c = inputs.make_case(60 + D + NV, B=B, NK=NK, NV=NV, D=D, T=T)
    say("dims", D, NV, NK)
    d = _dev_case(c)
    # decode (raw), decode_norm (fp32 and bf16), f16 twin on token 0 rows
    rows = [b * T for b in range(B)]
    c1 = inputs.make_case(60 + D + NV, B=B, NK=NK, NV=NV, D=D, T=1)
    for kind in ("raw", "norm32", "norm16", "f16"):
        if kind == "f16":
            ref_state = orc.f32_to_f16_bits(c1.state)
            st = dev(ref_state.view(np.float16))
            ref = orc.decode(ref_state, c1.q, c1.k, c1.v, c1.alpha, c1.beta, B=B, NK=NK, NV=NV,
                             Dk=D, Dv=D, z=c1.z, gn=c1.gn, eps=c1.eps, state_kind=orc.STATE_F16)
            y = g.gdn_decode_f16state(st, dev(c1.q), dev(c1.k), dev(c1.v), dev(c1.alpha),
                                      dev(c1.beta), dev(c1.z), dev(c1.gn), c1.eps,
                                      out_dtype=torch.bfloat16, num_k_heads=NK, num_v_heads=NV)
            assert bf16_ok(host(y), ref, NV, D, TOL_F16) <= 1.0
            gs = host(st).view(np.float16).astype(np.float64)
            assert tile_err(gs, ref_state.view(np.float16).astype(np.float64), NV, D) < TOL_F16
            continue
        ref_state = c1.state.copy()
        norm = kind != "raw"
        ref = orc.decode(ref_state, c1.q, c1.k, c1.v, c1.alpha, c1.beta, B=B, NK=NK, NV=NV, Dk=D,
                         Dv=D, z=c1.z if norm else None, gn=c1.gn if norm else None, eps=c1.eps)
        st = dev(c1.state)
        if kind == "raw":
            o = g.gdn_decode(st, dev(c1.q), dev(c1.k), dev(c1.v), dev(c1.alpha), dev(c1.beta),
                             num_k_heads=NK, num_v_heads=NV, head_dim=D)
            assert out_err(host(o), ref, NV, D) < TOL_STEP
        else:
            dt = torch.float32 if kind == "norm32" else torch.bfloat16
            y = g.gdn_decode_norm(st, dev(c1.q), dev(c1.k), dev(c1.v), dev(c1.alpha),
                                  dev(c1.beta), dev(c1.z), dev(c1.gn), c1.eps, out_dtype=dt,
                                  num_k_heads=NK, num_v_heads=NV)
            if dt == torch.float32:
                assert out_err(host(y), ref, NV, D) < TOL_STEP
            else:
                assert bf16_ok(host(y), ref, NV, D, TOL_STEP) <= 1.0
        assert tile_err(host(st), ref_state, NV, D) < TOL_STEP
    del rows
    # the sequence kernel, raw and normed, ragged T
    for norm in (False, True):
        ref_state = c.state.copy()
        ref = orc.seq(ref_state, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D,
                      Dv=D, z=c.z if norm else None, gn=c.gn if norm else None, eps=c.eps)
        st = dev(c.state)
        o = g.gdn_recurrence_seq(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                 d["z"] if norm else None, d["gn"] if norm else None, c.eps,
                                 seq_len=T, num_k_heads=NK, num_v_heads=NV, head_dim=D)
        assert out_err(host(o), ref, NV, D) < TOL_CHAIN, norm
        assert tile_err(host(st), ref_state, NV, D) < TOL_CHAIN, norm


# ------------------------------------------------------------- special cases
@pytest.mark.parametrize("B,NK,NV", [(5, 16, 64), (33, 8, 8), (3, 1, 128), (64, 16, 48)])
def test_raw_decode_heads_split_over_two_workgroups(g, B, NK, NV):
    """The wide raw decode at D = 128 splits each head's rows over two
    workgroups: other pairings (four, one and 128 value heads per key head), a
    NaN-padded slot pitch and the output in a window of a wider NaN-filled
    buffer. Every head's output and state tile against the oracle; the pads
    stay NaN."""
    import torch
    D = 128
    pitch = NV * D * D + 64
    c = inputs.make_case(2400 + B + NV, B=B, NK=NK, NV=NV, D=D, pitch=pitch)
    say("raw split", B, NK, NV)
    d = _dev_case(c)
    st = dev(c.state)
    wide = torch.full((B, NV * D + 20), float("nan"), device="cuda:0")
    g.gdn_decode(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], out=wide[:, 12:12 + NV * D],
                 num_k_heads=NK, num_v_heads=NV, head_dim=D)
    ref_st = c.state.copy()
    ref = orc.decode(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D)
    w = host(wide)
    assert out_err(w[:, 12:12 + NV * D], ref, NV, D) < TOL_STEP
    assert np.isnan(w[:, :12]).all() and np.isnan(w[:, 12 + NV * D:]).all()
    got = host(st)
    assert tile_err(got, ref_st, NV, D) < TOL_STEP
    assert np.isnan(got[:, NV * D * D:]).all()


@pytest.mark.parametrize("D", [4, 8, 16, 32, 64, 128, 256])
def test_wide_launch_every_head_dim(g, D):
    """Launches of 256 or more workgroups use the wide single-token tile (16
    values per lane for fp32, 32 for binary16); smaller ones hold 32 values per
    lane.  Every decode mode at every D on a wide launch (B=32, NV=8, NK=4)."""
    import torch
    B, NK, NV = 32, 4, 8
    c = inputs.make_case(1100 + D, B=B, NK=NK, NV=NV, D=D)
    say("wide launch", D)
    d = _dev_case(c)
    ref_st = c.state.copy()
    o_ref = orc.decode(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D)
    y_ref = orc.decode(c.state.copy(), c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D,
                       Dv=D, z=c.z, gn=c.gn, eps=c.eps)
    st = dev(c.state)
    o = g.gdn_decode(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], num_k_heads=NK,
                     num_v_heads=NV, head_dim=D)
    assert out_err(host(o), o_ref, NV, D) < TOL_STEP
    assert tile_err(host(st), ref_st, NV, D) < TOL_STEP
    for dt in (torch.float32, torch.bfloat16):
        st = dev(c.state)
        y = g.gdn_decode_norm(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                              c.eps, out_dtype=dt, num_k_heads=NK, num_v_heads=NV)
        if dt == torch.float32:
            assert out_err(host(y), y_ref, NV, D) < TOL_STEP
        else:
            assert bf16_ok(host(y), y_ref, NV, D, TOL_STEP) <= 1.0
        assert tile_err(host(st), ref_st, NV, D) < TOL_STEP
    if D % 32 == 0:
        st = dev(c.state)
        y, codes, scales = g.gdn_decode_norm_q(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                               d["z"], d["gn"], c.eps, num_k_heads=NK,
                                               num_v_heads=NV)
        assert out_err(host(y), y_ref, NV, D) < TOL_STEP
        yh, ch, sh = host(y), host(codes), host(scales)
        am = np.abs(yh.reshape(-1, 32)).max(axis=1)
        want = np.where(am > 0, am / np.float32(127.0), np.float32(1.0)).astype(np.float32)
        assert np.array_equal(sh.reshape(-1), want)
        assert np.array_equal(ch.reshape(-1, 32), np.rint(yh.reshape(-1, 32) / want[:, None]).astype(np.int8))
    st16 = g.gdn_state_f32_to_f16(dev(c.state))
    ref16 = orc.f32_to_f16_bits(c.state)
    y16_ref = orc.decode(ref16, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D,
                         z=c.z, gn=c.gn, eps=c.eps, state_kind=orc.STATE_F16)
    y16 = g.gdn_decode_f16state(st16, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                                c.eps, out_dtype=torch.float32, num_k_heads=NK, num_v_heads=NV)
    assert out_err(host(y16), y16_ref, NV, D) < TOL_F16
    got16 = host(st16).view(np.float16).astype(np.float64)
    assert tile_err(got16, ref16.view(np.float16).astype(np.float64), NV, D) < TOL_F16


@pytest.mark.parametrize("B", [2, 32])
def test_pins_hold_on_gpu(g, B):
    """The closed-form cases of the oracle pins, on the GPU kernels:
    alpha=1/beta=0 leaves the state bit-identical; alpha=0/beta=1 writes v k^T;
    one-hot keys with alpha=beta=1 store v in column h mod NK. B = 2 runs the
    small-grid launch, B = 32 the wide one (each head's rows over two
    workgroups)."""
    NK, NV, D = 4, 8, 128
    c = inputs.make_case(61, B=B, NK=NK, NV=NV, D=D)
    say("gpu pins")
    ones = np.ones((B, NV), np.float32)
    zeros = np.zeros((B, NV), np.float32)
    st = dev(c.state)
    g.gdn_decode(st, dev(c.q), dev(c.k), dev(c.v), dev(ones), dev(zeros), num_k_heads=NK,
                 num_v_heads=NV, head_dim=D)
    assert np.array_equal(host(st), c.state)
    st = dev(c.state)
    g.gdn_decode(st, dev(c.q), dev(c.k), dev(c.v), dev(zeros), dev(ones), num_k_heads=NK,
                 num_v_heads=NV, head_dim=D)
    got = host(st).reshape(B, NV, D, D)
    for b in range(B):
        for h in range(NV):
            gk = c.k[b, (h % NK) * D:(h % NK + 1) * D]
            want = np.outer(c.v[b, h * D:(h + 1) * D], gk).astype(np.float32)
            assert np.array_equal(got[b, h], want), (b, h)
    q = np.zeros((B, NK * D), np.float32)
    for gg in range(NK):
        q[:, gg * D + gg] = 1.0
    v = np.repeat(np.arange(1, NV + 1, dtype=np.float32), D)[None, :].repeat(B, 0)
    st = dev(np.zeros((B, NV * D * D), np.float32))
    o = host(g.gdn_decode(st, dev(q), dev(q), dev(v), dev(ones), dev(ones), num_k_heads=NK,
                          num_v_heads=NV, head_dim=D))
    got = host(st).reshape(B, NV, D, D)
    for h in range(NV):
        want = np.zeros((D, D), np.float32)
        want[:, h % NK] = h + 1
        assert np.array_equal(got[0, h], want), h
        np.testing.assert_allclose(o[0, h * D:(h + 1) * D], (h + 1) / np.sqrt(D), rtol=1e-6)


def test_deterministic_bitwise(g):
    """Two runs on the same inputs give the same bits (no atomics, fixed orders)."""
    import torch
    c = inputs.make_case(62, B=16, NK=16, NV=48, D=128, T=1)
    say("determinism")
    d = _dev_case(c)
    outs = []
    for _ in range(2):
        st = dev(c.state)
        y = g.gdn_decode_norm(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                              c.eps, out_dtype=torch.bfloat16, num_k_heads=16, num_v_heads=48)
        outs.append((host(st).view(np.uint32), host(y)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_sequence_workspace_deterministic_bitwise(g):
    """The workspace sequence path twice on the same inputs (a fresh workspace
    each time, the first filled with NaN): the same bits, outputs and states."""
    import torch
    B, T, NK, NV, D = 4, 70, 16, 48, 128
    c = inputs.make_case(64, B=B, NK=NK, NV=NV, D=D, T=T)
    say("determinism, workspace sequence")
    d = _dev_case(c)
    outs = []
    for fill in (float("nan"), 0.0):
        ws = torch.full((g.gdn_seq_workspace_bytes(B, T, NV, D) // 4,), fill,
                        dtype=torch.float32, device="cuda:0")
        st = dev(c.state)
        o = g.gdn_recurrence_seq_ws(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                    workspace=ws.view(torch.uint8), seq_len=T, num_k_heads=NK,
                                    num_v_heads=NV, head_dim=D)
        outs.append((host(st).view(np.uint32), host(o).view(np.uint32)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("T", [70, 200])
def test_sequence_workspace_norm_two_calls_one_workspace(g, T):
    """The workspace path with z, twice in one workspace (first filled with NaN)
    on two different cases of the same shape: nothing the first call leaves in
    the workspace reaches the second. Each call against the oracle, and the
    first call's bits again on a fresh workspace."""
    import torch
    B, NK, NV, D = 4, 16, 48, 128
    cases = [inputs.make_case(65 + i, B=B, NK=NK, NV=NV, D=D, T=T) for i in range(2)]
    say("workspace norm, two calls", T)
    need = g.gdn_seq_workspace_bytes(B, T, NV, D)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda:0")

    def run(c, w):
        d = _dev_case(c)
        st = dev(c.state)
        y = g.gdn_recurrence_seq_ws(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"],
                                    d["gn"], c.eps, workspace=w.view(torch.uint8), seq_len=T,
                                    num_k_heads=NK, num_v_heads=NV)
        return host(y), host(st)

    got = [run(c, ws) for c in cases]
    for c, (y, st) in zip(cases, got):
        ref_state = c.state.copy()
        ref = orc.seq(ref_state, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D,
                      Dv=D, z=c.z, gn=c.gn, eps=c.eps)
        assert out_err(y, ref, NV, D) < TOL_CHAIN
        assert tile_err(st, ref_state, NV, D) < TOL_CHAIN
    y0, st0 = run(cases[0], torch.zeros_like(ws))
    assert np.array_equal(y0.view(np.uint32), got[0][0].view(np.uint32))
    assert np.array_equal(st0.view(np.uint32), got[0][1].view(np.uint32))


@pytest.mark.parametrize("kind", ["decode", "f16", "seq128", "seq64", "seq128ws", "seq128ws_norm"])
def test_batch_permutation_permutes_results_bitwise(g, kind):
    """Sequences are independent: running a permuted batch gives the permuted
    outputs and states bit for bit (a wide launch for every kernel family)."""
    import torch
    D = 64 if kind == "seq64" else 128
    T = 20 if kind.startswith("seq") else 1
    B, NK, NV = (8, 4, 8) if kind.startswith("seq") else (40, 4, 8)
    c = inputs.make_case(1900 + D + T, B=B, NK=NK, NV=NV, D=D, T=T)
    perm = np.random.Generator(np.random.PCG64(19)).permutation(B)
    rows = (perm[:, None] * T + np.arange(T)[None, :]).reshape(-1)
    say("batch permutation", kind)

    def run(order, row_order):
        d = {n: dev(np.ascontiguousarray(getattr(c, n)[row_order]))
             for n in ("q", "k", "v", "z", "alpha", "beta")}
        st32 = dev(np.ascontiguousarray(c.state[order]))
        if kind == "decode":
            y = g.gdn_decode_norm(st32, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"],
                                  dev(c.gn), c.eps, num_k_heads=NK, num_v_heads=NV)
            return host(y), host(st32).view(np.uint32)
        if kind == "f16":
            st16 = g.gdn_state_f32_to_f16(st32)
            y = g.gdn_decode_f16state(st16, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"],
                                      dev(c.gn), c.eps, out_dtype=torch.bfloat16, num_k_heads=NK,
                                      num_v_heads=NV)
            return host(y), host(st16)
        if kind.startswith("seq128ws"):   # pre-pass, four workgroups per head (and the norm pass)
            zkw = dict(z=d["z"], norm_weight=dev(c.gn), eps=c.eps) if kind.endswith("norm") else {}
            o = g.gdn_recurrence_seq_ws(st32, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                        seq_len=T, num_k_heads=NK, num_v_heads=NV, head_dim=D,
                                        **zkw)
            return host(o), host(st32).view(np.uint32)
        o = g.gdn_recurrence_seq(st32, d["q"], d["k"], d["v"], d["alpha"], d["beta"], seq_len=T,
                                 num_k_heads=NK, num_v_heads=NV, head_dim=D)
        return host(o), host(st32).view(np.uint32)

    base = np.arange(B)
    y0, s0 = run(base, np.arange(B * T))
    y1, s1 = run(perm, rows)
    assert np.array_equal(y1, y0[rows])
    assert np.array_equal(s1, s0[perm])


def test_empty_batch_and_length_are_noops(g, seq):
    import torch
    c = inputs.make_case(63, B=2, NK=2, NV=4, D=16, T=1)
    say("empty")
    d = _dev_case(c)
    st = dev(c.state)
    out = torch.full((2, 64), 7.0, device="cuda:0")
    seq(st, d["q"][:0], d["k"][:0], d["v"][:0], d["alpha"][:0], d["beta"][:0],
        out=out[:0], seq_len=0, num_k_heads=2, num_v_heads=4, head_dim=16)
    e = torch.empty((0, 4 * 16 * 16), device="cuda:0")
    o = g.gdn_decode(e, d["q"][:0], d["k"][:0], d["v"][:0], d["alpha"][:0], d["beta"][:0],
                     num_k_heads=2, num_v_heads=4, head_dim=16)
    assert o.shape[0] == 0
    assert np.array_equal(host(st), c.state)
    assert (host(out) == 7.0).all()


def test_converters_bitwise(g):
    """fp32 -> binary16 on special values, midpoints, subnormals and a random
    sample, bitwise against the oracle's RNE; binary16 -> fp32 on all 65536
    patterns; odd lengths exercise the scalar tail."""
    import torch
    r = np.random.Generator(np.random.PCG64(64))
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = h.view(np.float16).astype(np.float64)
    nxt = np.concatenate([f[1:], [np.inf]])
    mid = ((f + nxt) / 2)[np.isfinite(f) & np.isfinite(nxt)].astype(np.float32).view(np.uint32)
    pats = [r.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)]
    for base in (f[np.isfinite(f)].astype(np.float32).view(np.uint32), mid):
        for dd in (-1, 0, 1):
            pats.append((base.astype(np.int64) + dd).astype(np.uint32))
    x = np.concatenate(pats).view(np.float32)
    x = x[: x.size - (x.size % 8) + 5]          # an odd tail
    say("converters", x.size)
    got = host(g.gdn_state_f32_to_f16(dev(x)))
    want = orc.f32_to_f16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert ((got[nan] & 0x7C00) == 0x7C00).all() and (got[nan] & 0x03FF).all()
    hh = np.concatenate([h, h[:3]])
    back = host(g.gdn_state_f16_to_f32(dev(hh.view(np.float16))))
    ref = orc.f16_bits_to_f32(hh)
    fin = ~np.isnan(ref)
    assert np.array_equal(back[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.isnan(back[~fin]).all()
    del torch


def test_f32_to_f16_every_binary32_pattern(g):
    """The fp32 -> binary16 converter on all 2^32 binary32 bit patterns, in 16
    chunks, bitwise against the oracle's RNE (NaNs: any quiet binary16 NaN)."""
    from concurrent.futures import ThreadPoolExecutor
    import torch
    n = 1 << 28
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    src = torch.empty(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty(n, dtype=torch.float16, device="cuda:0")
    for chunk in range(16):
        x = np.arange(chunk * n, (chunk + 1) * n, dtype=np.uint32).view(np.float32)
        say("f32 -> f16 patterns", chunk, "of 16")
        src.copy_(torch.from_numpy(x))
        g.gdn_state_f32_to_f16(src, dst)
        got = host(dst)
        parts = np.array_split(np.arange(n), threads)
        with ThreadPoolExecutor(max_workers=threads) as ex:
            want = np.concatenate(list(ex.map(lambda ix: orc.f32_to_f16_bits(x[ix[0]:ix[-1] + 1]), parts)))
        nan = np.isnan(x)
        assert np.array_equal(got[~nan], want[~nan]), chunk
        assert ((got[nan] & 0x7C00) == 0x7C00).all() and (got[nan] & 0x03FF).all(), chunk


def test_f16_state_keeps_subnormals(g):
    """A state update whose results land in the binary16 subnormal range keeps
    them (no flush to zero), matching the oracle bitwise for exact cases."""
    B, NK, NV, D = 1, 1, 1, 16
    c = inputs.make_case(65, B=B, NK=NK, NV=NV, D=D)
    s16 = np.zeros((1, D * D), np.uint16)
    s16[0, ::3] = 0x0001        # smallest subnormal
    s16[0, 1::7] = 0x03FF       # largest subnormal
    st = dev(s16.view(np.float16))
    ones = np.ones((1, 1), np.float32)
    zeros = np.zeros((1, 1), np.float32)
    say("f16 subnormals")
    g.gdn_decode_f16state(st, dev(c.q), dev(c.k), dev(c.v), dev(ones), dev(zeros),
                          num_k_heads=NK, num_v_heads=NV, head_dim=D)
    assert np.array_equal(host(st), s16)
    half = np.full((1, 1), 0.5, np.float32)
    g.gdn_decode_f16state(st, dev(c.q), dev(c.k), dev(c.v), dev(half), dev(zeros),
                          num_k_heads=NK, num_v_heads=NV, head_dim=D)
    ref = s16.copy()
    orc.decode(ref, c.q, c.k, c.v, half, zeros, B=1, NK=1, NV=1, Dk=D, Dv=D,
               state_kind=orc.STATE_F16)
    assert np.array_equal(host(st), ref)
    assert (ref[0, 1::7] == 0x0200).all()   # 0x03FF / 2 rounds to even 0x0200


def test_validation_rejects_before_launch(g):
    """Bad arguments come back as status codes and leave buffers untouched."""
    import torch
    c = inputs.make_case(66, B=2, NK=2, NV=4, D=16)
    d = _dev_case(c)
    st = dev(c.state)
    say("validation")
    out = d["v"].clone()
    with pytest.raises(g.GdnError) as e:   # output aliases the state
        g.gdn_decode(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], out=st[:, :64],
                     num_k_heads=2, num_v_heads=4, head_dim=16)
    assert e.value.status == 5
    with pytest.raises(g.GdnError) as e:   # unsupported head dim
        g.gdn_decode(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], num_k_heads=2,
                     num_v_heads=4, head_dim=12)
    with pytest.raises(g.GdnError) as e:   # NV not a multiple of NK
        g.gdn_decode(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], num_k_heads=2,
                     num_v_heads=3, head_dim=16)
    assert e.value.status == 2
    mis = torch.zeros(2 * 32 + 1, device="cuda:0")[1:].view(2, 32)   # 4-byte offset
    with pytest.raises(g.GdnError) as e:
        g.gdn_decode(st, mis, mis, d["v"], d["alpha"], d["beta"], num_k_heads=2,
                     num_v_heads=4, head_dim=16)
    assert e.value.status == 3
    with pytest.raises(g.GdnError) as e:   # negative eps
        g.gdn_decode_norm(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                          -1.0, num_k_heads=2, num_v_heads=4)
    assert e.value.status == 8
    src = torch.zeros(64, device="cuda:0")
    with pytest.raises(g.GdnError) as e:   # converter in place
        g.gdn_state_f32_to_f16(src, src.view(torch.float16)[:64])
    assert e.value.status == 5
    assert np.array_equal(host(st), c.state)
    assert np.array_equal(host(out), c.v)


def test_graph_replay_matches_eager(g):
    """Decode calls captured once in a HIP graph (as the B=1 model token is
    timed) and replayed three times, with eager work and synchronisation
    between replays: every replay's outputs and states equal the same calls
    made eagerly on copies, bit for bit."""
    import torch
    B, NK, NV, D, L = 1, 16, 48, 128, 4
    cases = [inputs.make_case(1200 + l, B=B, NK=NK, NV=NV, D=D) for l in range(L)]
    say("graph replay")
    dg = [_dev_case(c) for c in cases]
    st_g = [dev(c.state) for c in cases]
    st_e = [dev(c.state) for c in cases]
    out_g = [torch.empty((B, NV * D), device="cuda:0") for _ in range(L)]

    def token(states, outs):
        for d, st, o in zip(dg, states, outs):
            g.gdn_decode_norm(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                              1e-6, out=o, num_k_heads=NK, num_v_heads=NV)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        token(st_g, out_g)                     # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        token(st_g, out_g)
    # the capture itself does not run the kernels: bring the eager copies to
    # the same point (one warm-up token)
    out_e = [torch.empty_like(o) for o in out_g]
    token(st_e, out_e)
    for rep in range(3):
        graph.replay()
        token(st_e, out_e)
        scratch = torch.randn(1 << 20, device="cuda:0").sum()   # eager work in between
        torch.cuda.synchronize()
        assert bool(torch.isfinite(scratch))
        for l in range(L):
            assert torch.equal(out_g[l], out_e[l]), (rep, l)
            assert torch.equal(st_g[l], st_e[l]), (rep, l)


def test_sequence_workspace_shared_and_odd_heads(g):
    """The workspace entry at one value head per key head and 15 heads (the
    workgroup mapping's partial group of eight), twice in a row on one shared
    workspace with different inputs, and the size check (a workspace one byte
    short is rejected before any launch, leaving the state untouched)."""
    import torch
    B, NK, NV, D = 3, 5, 5, 128
    ws = torch.empty(g.gdn_seq_workspace_bytes(B, 40, NV, D), dtype=torch.uint8, device="cuda:0")
    for T, seed in ((40, 1501), (23, 1502)):      # the second call leaves part of the workspace stale
        c = inputs.make_case(seed, B=B, NK=NK, NV=NV, D=D, T=T)
        say("seq workspace shared", T)
        d = _dev_case(c)
        st = dev(c.state)
        o = g.gdn_recurrence_seq_ws(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                    workspace=ws, seq_len=T, num_k_heads=NK, num_v_heads=NV,
                                    head_dim=D)
        ref_st = c.state.copy()
        ref = orc.seq(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D, Dv=D)
        assert out_err(host(o), ref, NV, D) < TOL_CHAIN, T
        assert tile_err(host(st), ref_st, NV, D) < TOL_CHAIN, T
    need = g.gdn_seq_workspace_bytes(B, 23, NV, D)
    before = host(st).copy()
    with pytest.raises(g.GdnError):
        g.gdn_recurrence_seq_ws(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                workspace=ws[:need - 1], seq_len=23, num_k_heads=NK,
                                num_v_heads=NV, head_dim=D)
    assert np.array_equal(host(st), before)


@pytest.mark.parametrize("B,NK,R,T", [(3, 11, 3, 37), (1, 16, 3, 40), (2, 16, 3, 17)])
def test_sequence_workspace_small_batches(g, B, NK, R, T):
    """The workspace path at 99 value heads in all, and at the real head shape
    with B = 1 and B = 2 (192 and 384 workgroups, fewer than three per CU),
    against the oracle on every head, with a ragged or short T."""
    NV, D = R * NK, 128
    c = inputs.make_case(3200 + B * NV + T, B=B, NK=NK, NV=NV, D=D, T=T)
    say("seq workspace row split", B, NK, R, T)
    d = _dev_case(c)
    st = dev(c.state)
    o = g.gdn_recurrence_seq_ws(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], seq_len=T,
                                num_k_heads=NK, num_v_heads=NV, head_dim=D)
    ref_st = c.state.copy()
    ref = orc.seq(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D, Dv=D)
    assert out_err(host(o), ref, NV, D) < TOL_CHAIN
    assert tile_err(host(st), ref_st, NV, D) < TOL_CHAIN


@pytest.mark.parametrize("NK,R", [(2, 2), (1, 4), (1, 5), (2, 8), (1, 17)])
def test_sequence_many_value_heads_per_key_head(g, seq, NK, R):
    """Both sequence entries at D = 128 with R = NV / NK value heads per key
    head: the pre-pass takes them four at a time (R = 5 leaves a group of one,
    R = 8 makes two full groups) inside groups of sixteen staged alpha / beta
    rows (R = 17 needs a second one); R >= 4 sends the plain entry to the
    one-workgroup-per-head kernel.  A ragged T puts a partial chunk last."""
    B, T, D = 2, 37, 128
    NV = R * NK
    c = inputs.make_case(2900 + 10 * R + NK, B=B, NK=NK, NV=NV, D=D, T=T)
    say("seq heads per key head", NK, R)
    d = _dev_case(c)
    st = dev(c.state)
    o = seq(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], seq_len=T, num_k_heads=NK,
            num_v_heads=NV, head_dim=D)
    ref_st = c.state.copy()
    ref = orc.seq(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D, Dv=D)
    assert out_err(host(o), ref, NV, D) < TOL_CHAIN
    assert tile_err(host(st), ref_st, NV, D) < TOL_CHAIN


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 32, 33, 48])
@pytest.mark.parametrize("norm", [False, True])
def test_sequence_chunk_boundaries(g, seq, D, T, norm):
    """Lengths around the 16-token chunk (and the two chunk buffers of the
    matrix-core kernel at D = 128): outputs and final state against the oracle."""
    B, NK, NV = 2, 2, 6
    c = inputs.make_case(1300 + T + D, B=B, NK=NK, NV=NV, D=D, T=T)
    say("seq boundary", D, T, norm)
    d = _dev_case(c)
    st = dev(c.state)
    kw = dict(z=d["z"], norm_weight=d["gn"], eps=c.eps) if norm else dict(head_dim=D)
    o = seq(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], seq_len=T,
            num_k_heads=NK, num_v_heads=NV, **kw)
    ref_st = c.state.copy()
    okw = dict(z=c.z, gn=c.gn, eps=c.eps) if norm else {}
    ref = orc.seq(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D, Dv=D, **okw)
    assert out_err(host(o), ref, NV, D) < TOL_CHAIN
    assert tile_err(host(st), ref_st, NV, D) < TOL_CHAIN


@pytest.mark.parametrize("D", [64, 128])
def test_sequence_extreme_decay(g, seq, D):
    """Decays of exactly 0 (the state is forgotten), 1e-8 (the running decay
    product leaves any fixed exponent range within a few tokens), 1 (no decay)
    and ordinary values, mixed within chunks, with write strengths of 0 and 1
    among them: outputs and final state against the oracle."""
    B, NK, NV, T = 2, 2, 4, 100
    c = inputs.make_case(1400 + D, B=B, NK=NK, NV=NV, D=D, T=T)
    r = np.random.Generator(np.random.PCG64(1401))
    pick = r.integers(0, 5, size=c.alpha.shape)
    c.alpha[:] = np.choose(pick, [np.float32(0.0), np.float32(1e-8), np.float32(1.0),
                                  np.float32(0.5), c.alpha]).astype(np.float32)
    c.beta[r.random(c.beta.shape) < 0.2] = 0.0
    c.beta[r.random(c.beta.shape) < 0.2] = 1.0
    say("seq extreme decay", D)
    d = _dev_case(c)
    st = dev(c.state)
    o = seq(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], seq_len=T,
            num_k_heads=NK, num_v_heads=NV, head_dim=D)
    ref_st = c.state.copy()
    ref = orc.seq(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D, Dv=D)
    got_o, got_st = host(o), host(st)
    assert np.isfinite(got_o).all() and np.isfinite(got_st).all()
    assert out_err(got_o, ref, NV, D) < TOL_CHAIN
    assert tile_err(got_st, ref_st, NV, D) < TOL_CHAIN


def test_calls_on_side_streams(g):
    """Calls run on the stream they are given: two pools advanced concurrently
    on two side streams (disjoint state and outputs) match the oracle, and an
    explicit stream handle works like the current-stream default."""
    import torch
    B, NK, NV, D = 8, 4, 8, 128
    ca = inputs.make_case(1500, B=B, NK=NK, NV=NV, D=D)
    cb = inputs.make_case(1501, B=B, NK=NK, NV=NV, D=D)
    say("side streams")
    da, db = _dev_case(ca), _dev_case(cb)
    sta, stb = dev(ca.state), dev(cb.state)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        ya = g.gdn_decode_norm(sta, da["q"], da["k"], da["v"], da["alpha"], da["beta"], da["z"],
                               da["gn"], ca.eps, num_k_heads=NK, num_v_heads=NV)
    yb = g.gdn_decode_norm(stb, db["q"], db["k"], db["v"], db["alpha"], db["beta"], db["z"],
                           db["gn"], cb.eps, num_k_heads=NK, num_v_heads=NV,
                           stream=s2.cuda_stream)
    torch.cuda.synchronize()
    for c, y, st in ((ca, ya, sta), (cb, yb, stb)):
        ref_st = c.state.copy()
        ref = orc.decode(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D,
                         z=c.z, gn=c.gn, eps=c.eps)
        assert out_err(host(y), ref, NV, D) < TOL_STEP
        assert tile_err(host(st), ref_st, NV, D) < TOL_STEP
