"""GPU parity of the multi-token entry points on packed, strided rows.

q | k | v are column slices of one padded projection row, z sits at an offset in a
wider row, alpha and beta share one interleaved row, the output rows are a
window of a wider NaN-filled buffer and the state slots are padded with NaN.
Every stride goes through the C ABI as given; the pads must stay untouched.
Ragged token counts put a partial chunk at the end of the sequence kernels.
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


@pytest.fixture(scope="module", params=["gdn_recurrence_seq", "gdn_recurrence_seq_ws"])
def seq(g, request):
    """Both sequence entry points: without and with the chunk workspace."""
    return getattr(g, request.param)


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _packed(c, rows):
    """Device views of the case's token inputs laid out in shared wide rows."""
    import torch
    NK, NV, D = c.NK, c.NV, c.D
    qk, vw = NK * D, NV * D
    proj = np.zeros((rows, 2 * qk + vw + 12), np.float32)
    proj[:, :qk], proj[:, qk:2 * qk], proj[:, 2 * qk:2 * qk + vw] = c.q, c.k, c.v
    zrow = np.zeros((rows, vw + 20), np.float32)
    zrow[:, 20:] = c.z
    ab = np.zeros((rows, 2 * NV + 4), np.float32)
    ab[:, :NV], ab[:, NV:2 * NV] = c.beta, c.alpha
    p, z, a = dev(proj), dev(zrow), dev(ab)
    wide = torch.full((rows, vw + 36), float("nan"), device="cuda:0")
    return dict(q=p[:, :qk], k=p[:, qk:2 * qk], v=p[:, 2 * qk:2 * qk + vw], z=z[:, 20:],
                alpha=a[:, NV:2 * NV], beta=a[:, :NV], wide=wide, out=wide[:, 4:4 + vw])


def _pads_untouched(wide, st, NV, D):
    w = host(wide)
    assert np.isnan(w[:, :4]).all() and np.isnan(w[:, 4 + NV * D:]).all()
    assert np.isnan(host(st)[:, NV * D * D:]).all()


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("norm", [False, True])
def test_sequence_packed_rows(g, seq, D, norm):
    """T = 37 tokens (two full 16-token chunks and a ragged one) on packed rows;
    D = 128 runs the chunked matrix-core kernel, D = 64 the token loop."""
    B, NK, NV, T = 3, 2, 6, 37
    c = inputs.make_case(1700 + D, B=B, NK=NK, NV=NV, D=D, T=T, pitch=NV * D * D + 40)
    say("sequence packed rows", D, "norm" if norm else "raw")
    d = _packed(c, B * T)
    st = dev(c.state)
    seq(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
        d["z"] if norm else None, dev(c.gn) if norm else None, c.eps,
        out=d["out"], seq_len=T, num_k_heads=NK, num_v_heads=NV, head_dim=D)
    ref_st = c.state.copy()
    kw = dict(z=c.z, gn=c.gn, eps=c.eps) if norm else {}
    ref = orc.seq(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D, Dv=D, **kw)
    assert out_err(host(d["out"]), ref, NV, D) < TOL_CHAIN
    assert tile_err(host(st), ref_st, NV, D) < TOL_CHAIN
    _pads_untouched(d["wide"], st, NV, D)


@pytest.mark.parametrize("D", [64, 128])
def test_verify_packed_rows(g, D):
    """Five draft tokens on packed rows with the fused norm: outputs, the final
    state and every rollback slot (itself in a padded pool)."""
    import torch
    B, NK, NV, T = 3, 2, 6, 5
    pitch = NV * D * D + 40
    c = inputs.make_case(1800 + D, B=B, NK=NK, NV=NV, D=D, T=T, pitch=pitch)
    say("verify packed rows", D)
    d = _packed(c, B * T)
    st = dev(c.state)
    inter = torch.full((B * (T - 1), pitch), float("nan"), device="cuda:0")
    g.gdn_decode_verify(st, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"], dev(c.gn), c.eps,
                        out=d["out"], inter_state=inter, num_tokens=T, num_k_heads=NK,
                        num_v_heads=NV, head_dim=D)
    ref_st = c.state.copy()
    ref = orc.seq(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D, Dv=D,
                  z=c.z, gn=c.gn, eps=c.eps)
    assert out_err(host(d["out"]), ref, NV, D) < TOL_CHAIN
    assert tile_err(host(st), ref_st, NV, D) < TOL_CHAIN
    _pads_untouched(d["wide"], st, NV, D)
    got = host(inter).reshape(B, T - 1, pitch)
    assert np.isnan(got[:, :, NV * D * D:]).all()
    for t in range(T - 1):
        n = t + 1
        pre = lambda a: np.ascontiguousarray(a.reshape(B, T, -1)[:, :n].reshape(B * n, -1))
        st_t = c.state.copy()
        orc.seq(st_t, pre(c.q), pre(c.k), pre(c.v), pre(c.alpha), pre(c.beta), B=B, T=n, NK=NK,
                NV=NV, Dk=D, Dv=D)
        assert tile_err(got[:, t], st_t, NV, D) < TOL_CHAIN, t


def _seq_ws_raw(g, st, q, k, qk_stride, v, v_stride, al, be, ab_stride, out, out_stride, B, T,
                NK, NV, D):
    """gdn_recurrence_seq_ws straight through ctypes, strides exactly as given."""
    import torch
    lib = g.lib()
    need = lib.gdn_seq_workspace_bytes(B, T, NV, D, D)
    ws = torch.empty(max(need, 16) // 4, dtype=torch.float32, device="cuda:0")
    s = lib.gdn_recurrence_seq_ws(st.data_ptr(), NV * D * D, q.data_ptr(), k.data_ptr(), qk_stride,
                                  v.data_ptr(), v_stride, al.data_ptr(), be.data_ptr(), ab_stride,
                                  None, 0, None, 0.0, out.data_ptr(), out_stride, B, T, NK, NV, D,
                                  D, ws.data_ptr(), need,
                                  torch.cuda.current_stream().cuda_stream)
    assert s == 0, g.STATUS_NAMES.get(s, s)


@pytest.mark.parametrize("qk_stride", [0, 2 * 16 * 128])
def test_seq_ws_single_row_small_strides(g, qk_stride):
    """One sequence of one token takes no stride check (there is no second
    row), so strides of 0 are legal; the workspace path must still read every
    input of that row and write its output (regression: its buffer ranges were
    once sized from the stride, so everything read as 0)."""
    import torch
    B, T, NK, NV, D = 1, 1, 16, 48, 128
    c = inputs.make_case(1900 + qk_stride, B=B, NK=NK, NV=NV, D=D, T=T)
    say("seq_ws single row, qk stride", qk_stride)
    st = dev(c.state)
    if qk_stride:   # q | k of one row side by side: k read at q + NK * D
        qk = dev(np.concatenate([c.q, c.k], axis=1))
        q, k = qk[:, :NK * D], qk[:, NK * D:]
    else:
        q, k = dev(c.q), dev(c.k)
    out = torch.full((1, NV * D), float("nan"), device="cuda:0")
    _seq_ws_raw(g, st, q, k, qk_stride, dev(c.v), 0, dev(c.alpha), dev(c.beta), 0, out, 0,
                B, T, NK, NV, D)
    ref_st = c.state.copy()
    ref = orc.seq(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D, Dv=D)
    assert out_err(host(out), ref, NV, D) < 1e-5
    assert tile_err(host(st), ref_st, NV, D) < 1e-5


@pytest.mark.parametrize("T,out_stride", [(1, (1 << 28) + 64), (2, 40_000_000), (5, 36_000_000)])
def test_seq_ws_wide_output_stride_short_sequence(g, T, out_stride):
    """Output rows so far apart that the offsets of a whole 16-token chunk pass
    2^31 bytes although T rows do not: the call must still be exact, and
    nothing between the rows may be written (regression: the 32-bit lane
    offsets of the padding tokens once wrapped into the valid range)."""
    import torch
    B, NK, NV, D = 1, 16, 48, 128
    vw = NV * D
    c = inputs.make_case(1950 + T, B=B, NK=NK, NV=NV, D=D, T=T)
    say("seq_ws wide output stride", T, out_stride)
    st = dev(c.state)
    buf = torch.full(((T - 1) * out_stride + vw,), float("nan"), device="cuda:0")
    _seq_ws_raw(g, st, dev(c.q), dev(c.k), NK * D, dev(c.v), vw, dev(c.alpha), dev(c.beta), NV,
                buf, out_stride, B, T, NK, NV, D)
    torch.cuda.synchronize()
    rows = torch.stack([buf[t * out_stride:t * out_stride + vw] for t in range(T)])
    ref_st = c.state.copy()
    ref = orc.seq(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=T, NK=NK, NV=NV, Dk=D, Dv=D)
    assert out_err(host(rows), ref, NV, D) < TOL_CHAIN
    assert tile_err(host(st), ref_st, NV, D) < TOL_CHAIN
    for t in range(T - 1):
        gap = buf[t * out_stride + vw:(t + 1) * out_stride]
        assert bool(torch.isnan(gap).all()), t
