"""GPU parity of gdn_decode_norm_q: the fused decode + gated norm with int8
quantisation of y in groups of 32.

The fp32 y is compared with the oracle as for gdn_decode_norm (1e-5 per head).
The integer decisions are checked twice:
* exactly, in binary32, on the kernel's own y: scale = fl(amax/127) and
  code = rne(fl(y/scale)), recomputed with numpy float32 (IEEE) arithmetic;
* against the oracle's quantiser run on the oracle's y rounded to fp32: scales
  within the y tolerance, codes equal except where the oracle's y/scale lies so
  close to a rounding boundary that the allowed y error can cross it (then +-1).
"""
import sys

import numpy as np
import pytest

import oracle as orc
from gated_deltanet_decode_delta_amd import inputs
from gpu_util import dev, host, out_err

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


def _run(g, c, write_y=True, state=None):
    d = {n: dev(getattr(c, n)) for n in ("q", "k", "v", "alpha", "beta", "z", "gn")}
    st = dev(c.state) if state is None else state
    y, codes, scales = g.gdn_decode_norm_q(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                           d["z"], d["gn"], c.eps, write_y=write_y,
                                           num_k_heads=c.NK, num_v_heads=c.NV)
    return st, (host(y) if y is not None else None), host(codes), host(scales)


def _exact_fp32_decisions(y, codes, scales):
    """The kernel's codes and scales are the binary32 quantisation of its own y."""
    yg = y.astype(np.float32).reshape(-1, 32)
    am = np.abs(yg).max(axis=1)
    want_s = np.where(am > 0, am / np.float32(127.0), np.float32(1.0)).astype(np.float32)
    assert np.array_equal(scales.reshape(-1), want_s)
    want_c = np.rint(yg / want_s[:, None]).astype(np.int8)
    assert np.array_equal(codes.reshape(-1, 32), want_c)
    nz = am > 0
    assert (np.abs(codes.reshape(-1, 32)[nz].astype(int)).max(axis=1) == 127).all()


def _against_oracle(y_ref, codes, scales, NV, D):
    """Codes and scales against the oracle's quantiser on its own fp32 y."""
    yr32 = y_ref.astype(np.float32)
    rc, rs = orc.quant_groups32(yr32)
    rc = rc.reshape(codes.shape)
    rs = rs.reshape(scales.shape)
    head_max = np.abs(y_ref).reshape(-1, NV, D).max(axis=2)           # [rows, NV]
    allow_y = TOL_STEP * np.repeat(head_max, D // 32, axis=1)          # per group
    assert (np.abs(scales - rs) <= allow_y / 127 + 1e-30).all()
    # codes: exact unless the allowed error in y/scale reaches a rounding boundary
    ratio = yr32.reshape(rc.shape[0], -1, 32) / rs[:, :, None]
    slack = (allow_y / rs)[:, :, None] * 1.01 + 2 * np.abs(ratio) * 2.0 ** -23
    frac = np.abs(ratio - np.floor(ratio) - 0.5)
    near = frac <= slack
    diff = codes.reshape(ratio.shape).astype(int) - rc.reshape(ratio.shape).astype(int)
    assert (np.abs(diff) <= 1).all()
    assert (diff[~near] == 0).all()
    return int(near.sum())


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_norm_q_against_oracle(g, D):
    B, NK, NV = 3, 2, 6
    c = inputs.make_case(800 + D, B=B, NK=NK, NV=NV, D=D)
    c.z[1, 2 * D:3 * D] = 0.0           # head 2 of sequence 1: y = 0, all-zero groups
    say("norm_q", D)
    st, y, codes, scales = _run(g, c)
    ref_state = c.state.copy()
    y_ref = orc.decode(ref_state, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D,
                       z=c.z, gn=c.gn, eps=c.eps)
    assert out_err(y, y_ref, NV, D) < TOL_STEP
    _exact_fp32_decisions(y, codes, scales)
    _against_oracle(y_ref, codes, scales, NV, D)
    zero = slice(2 * D // 32, 3 * D // 32)
    assert (scales[1, zero] == 1.0).all() and not codes[1, 2 * D:3 * D].any()
    ref_st = ref_state.reshape(B, -1)
    got_st = host(st)
    assert np.abs(got_st - ref_st).max() <= TOL_STEP * np.abs(ref_st).max()


def test_norm_q_without_y_matches_with_y(g):
    """Skipping the fp32 y changes nothing else: same codes, scales and state."""
    c = inputs.make_case(820, B=4, NK=4, NV=8, D=128)
    say("norm_q no y")
    st1, y1, c1, s1 = _run(g, c, write_y=True)
    st2, y2, c2, s2 = _run(g, c, write_y=False)
    assert y2 is None
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert np.array_equal(host(st1), host(st2))


def test_norm_q_full_batch_padded_pool(g):
    """The decode workload's shapes (B=64, NV=48, NK=16, D=128, 1.25x slot pitch):
    exact binary32 decisions everywhere, sampled heads against the oracle."""
    c = inputs.config_case("batched")
    B, NK, NV, D = c.B, c.NK, c.NV, c.D
    say("norm_q full batch")
    st, y, codes, scales = _run(g, c)
    _exact_fp32_decisions(y, codes, scales)
    assert np.isnan(host(st)[:, NV * D * D:]).all()
    r = np.random.Generator(np.random.PCG64(21))
    heads = sorted((int(i) // NV, int(i) % NV) for i in r.choice(B * NV, 24, replace=False))
    ref_state = c.state.copy()
    y_ref = orc.decode(ref_state, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D,
                       z=c.z, gn=c.gn, eps=c.eps, heads=heads)
    for b, h in heads:
        sl = slice(h * D, (h + 1) * D)
        assert out_err(y[b:b + 1, sl], y_ref[b:b + 1, sl], 1, D) < TOL_STEP
        _against_oracle(y_ref[b:b + 1, sl], codes[b:b + 1, sl], scales[b:b + 1, h * 4:(h + 1) * 4],
                        1, D)


def test_norm_q_validation(g):
    """Unsupported head dim, missing or overlapping code/scale buffers."""
    import torch
    c = inputs.make_case(830, B=2, NK=2, NV=4, D=16)
    d = {n: dev(getattr(c, n)) for n in ("q", "k", "v", "alpha", "beta", "z", "gn")}
    st = dev(c.state)
    say("norm_q validation")
    with pytest.raises(g.GdnError) as e:      # D = 16 is not a multiple of 32
        g.gdn_decode_norm_q(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                            num_k_heads=2, num_v_heads=4)
    assert e.value.status == 4
    c = inputs.make_case(831, B=2, NK=2, NV=4, D=32)
    d = {n: dev(getattr(c, n)) for n in ("q", "k", "v", "alpha", "beta", "z", "gn")}
    st = dev(c.state)
    buf = torch.zeros(2, 4 * 32, dtype=torch.int8, device="cuda:0")
    with pytest.raises(g.GdnError) as e:      # scales inside the codes buffer
        g.gdn_decode_norm_q(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                            codes=buf, scales=buf.view(torch.float32)[:, :4],
                            num_k_heads=2, num_v_heads=4)
    assert e.value.status == 5
    with pytest.raises(g.GdnError) as e:      # codes over the state
        g.gdn_decode_norm_q(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], d["gn"],
                            codes=st.view(torch.int8)[:, :128],
                            num_k_heads=2, num_v_heads=4)
    assert e.value.status == 5
    assert np.array_equal(host(st), c.state)
