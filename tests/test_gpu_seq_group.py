"""GPU parity of the workspace-free sequence kernel at D = 128 that gives each
workgroup one quarter of the state rows of all value heads of a key head.

gdn_recurrence_seq runs it whenever a key head has at most three value heads
(with four, the one-workgroup-per-head kernel runs: the R = 4 cases below
check that route).  At three value heads per key head a grid of eighths (16
rows per workgroup) runs instead of quarters when it fits the 256 compute
units in one pass, B * NK <= 32: most small cases below take eighths, and the
ones marked "quarters" keep B * NK above 32 so that quarters run.
Every (value heads per key head, length) pairing below is compared head by head
with the oracle: ragged lengths (a partial last chunk), lengths under one and
two chunks, group counts that are and are not multiples of eight (the block
mapping keeps a key head's four quarters on one XCD and places the remainder
separately), raw o and the gated norm.
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


def _run(g, c, norm):
    d = {n: dev(getattr(c, n)) for n in ("q", "k", "v", "z", "alpha", "beta", "gn")}
    st = dev(c.state)
    if norm:
        o = g.gdn_recurrence_seq(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                                 c.eps, seq_len=c.T, num_k_heads=c.NK, num_v_heads=c.NV)
    else:
        o = g.gdn_recurrence_seq(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], seq_len=c.T,
                                 num_k_heads=c.NK, num_v_heads=c.NV, head_dim=c.D)
    ref_st = c.state.copy()
    kw = dict(z=c.z, gn=c.gn, eps=c.eps) if norm else {}
    ref = orc.seq(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=c.B, T=c.T, NK=c.NK, NV=c.NV, Dk=c.D,
                  Dv=c.D, **kw)
    return host(o), host(st), ref, ref_st


@pytest.mark.parametrize("R", [1, 2, 3, 4])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 37])
def test_group_kernel_heads_per_key_head(g, R, T):
    B, NK = 3, 2   # six key-head groups: fewer than eight, all in the remainder
    c = inputs.make_case(2600 + 10 * R + T, B=B, NK=NK, NV=R * NK, D=128, T=T)
    say("seq group R", R, "T", T)
    o, st, ref, ref_st = _run(g, c, False)
    assert out_err(o, ref, c.NV, 128) < TOL_CHAIN
    assert tile_err(st, ref_st, c.NV, 128) < TOL_CHAIN


@pytest.mark.parametrize("B,NK,R", [(4, 2, 3), (2, 16, 3), (3, 8, 2), (1, 12, 4)])
def test_group_kernel_block_mapping(g, B, NK, R):
    """8, 32, 24 and 12 key-head groups: whole sets of eight, and eight plus a
    remainder of four (B=1, NK=12)."""
    T = 40
    c = inputs.make_case(2700 + B * NK + R, B=B, NK=NK, NV=R * NK, D=128, T=T)
    say("seq group mapping", B, NK, R)
    o, st, ref, ref_st = _run(g, c, False)
    assert out_err(o, ref, c.NV, 128) < TOL_CHAIN
    assert tile_err(st, ref_st, c.NV, 128) < TOL_CHAIN


@pytest.mark.parametrize("R", [1, 3, 4])
def test_group_kernel_gated_norm(g, R):
    B, NK, T = 2, 3, 45
    c = inputs.make_case(2800 + R, B=B, NK=NK, NV=R * NK, D=128, T=T)
    say("seq group norm R", R)
    o, st, ref, ref_st = _run(g, c, True)
    assert out_err(o, ref, c.NV, 128) < TOL_CHAIN
    assert tile_err(st, ref_st, c.NV, 128) < TOL_CHAIN


def test_group_kernel_strong_decay_and_zero_alpha(g):
    """alpha = 0 on some tokens and tiny alphas elsewhere (the range products
    and the decay scale folded into the state); beta up to 1."""
    B, NK, R, T = 2, 2, 3, 50
    c = inputs.make_case(2900, B=B, NK=NK, NV=R * NK, D=128, T=T)
    c.alpha[::7] = 0.0
    c.alpha[3::11] = 1e-20
    c.beta[5::9] = 1.0
    say("seq group strong decay")
    o, st, ref, ref_st = _run(g, c, False)
    assert out_err(o, ref, c.NV, 128) < TOL_CHAIN
    assert tile_err(st, ref_st, c.NV, 128) < TOL_CHAIN
    assert np.isfinite(o).all() and np.isfinite(st).all()


@pytest.mark.parametrize("B,NK,T,norm", [(3, 12, 17, False), (3, 11, 37, False), (3, 11, 37, True)])
def test_group_kernel_quarters_at_three_heads(g, B, NK, T, norm):
    """Quarters at R = 3 (B * NK = 36 or 33, above the eighths limit): a ragged
    T, group counts with and without a remainder of the mapping's eight."""
    c = inputs.make_case(3000 + B * NK + T, B=B, NK=NK, NV=3 * NK, D=128, T=T)
    say("seq group quarters", B, NK, T, norm)
    o, st, ref, ref_st = _run(g, c, norm)
    assert out_err(o, ref, c.NV, 128) < TOL_CHAIN
    assert tile_err(st, ref_st, c.NV, 128) < TOL_CHAIN


@pytest.mark.parametrize("B,NK", [(1, 12), (1, 5), (2, 16), (1, 1)])
def test_group_kernel_eighths_mapping(g, B, NK):
    """Eighths at R = 3: 12 groups (eight plus a remainder of four), 5 (all in
    the remainder), 32 (the largest grid that takes eighths: 256 workgroups)
    and a single group."""
    T = 40
    c = inputs.make_case(3100 + B * NK, B=B, NK=NK, NV=3 * NK, D=128, T=T)
    say("seq group eighths", B, NK)
    o, st, ref, ref_st = _run(g, c, False)
    assert out_err(o, ref, c.NV, 128) < TOL_CHAIN
    assert tile_err(st, ref_st, c.NV, 128) < TOL_CHAIN
