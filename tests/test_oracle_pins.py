"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compare the oracle with itself or with a retyped copy of its
formula: each checks a special case with a known answer (a closed form, an
invariant, a hand-derived example, brute force with library matrix products,
or a library conversion routine).  A dropped term, a wrong sign, a transposed
state, the h/(NV/NK) pairing, a missing 1/sqrt(D) or a norm in the wrong order
each fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

from gated_deltanet_decode_delta_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "d4_worked_example.json")


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def unit(r, d):
    x = r.standard_normal(d)
    return x / np.linalg.norm(x)


# ---------------------------------------------------------------- P1 -------
def test_p1_identity_step_leaves_state_and_reads_it(orc):
    """alpha = 1, beta = 0: no forgetting and no write; o = S q / sqrt(D)."""
    r = rng(11)
    for D in (4, 16, 128):
        S = r.standard_normal((D, D))
        q, k, v = unit(r, D), unit(r, D), r.standard_normal(D)
        S1, o = orc.head_step(S, q, k, v, 1.0, 0.0)
        assert np.array_equal(S1, S)
        np.testing.assert_allclose(o, (S @ q) / math.sqrt(D), rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- P2 -------
def test_p2_full_write_stores_value_at_key(orc):
    """alpha = beta = 1 and unit k: the delta rule makes S' k = v."""
    r = rng(12)
    for D in (4, 32, 128):
        S = r.standard_normal((D, D))            # not symmetric: a transposed S fails
        k = unit(r, D)
        v = r.standard_normal(D)
        S1, _ = orc.head_step(S, unit(r, D), k, v, 1.0, 1.0)
        np.testing.assert_allclose(S1 @ k, v, rtol=0, atol=1e-12 * np.linalg.norm(v))
        # one-hot key: column j becomes exactly v, the other columns are untouched
        j = D // 3
        e = np.zeros(D); e[j] = 1.0
        S2, _ = orc.head_step(S, e, e, v, 1.0, 1.0)
        assert np.array_equal(S2[:, j], v)
        keep = [c for c in range(D) if c != j]
        assert np.array_equal(S2[:, keep], S[:, keep])


# ---------------------------------------------------------------- P3 -------
def test_p3_full_forget_is_outer_product(orc):
    """alpha = 0: S' = beta v k^T and o = beta v (k.q) / sqrt(D)."""
    r = rng(13)
    for D in (4, 64):
        S = r.standard_normal((D, D))
        q, k, v = unit(r, D), unit(r, D), r.standard_normal(D)
        S1, o = orc.head_step(S, q, k, v, 0.0, 1.0)
        assert np.array_equal(S1, np.outer(v, k))
        S1, o = orc.head_step(S, q, k, v, 0.0, 0.375)
        np.testing.assert_allclose(S1, 0.375 * np.outer(v, k), rtol=1e-15, atol=0)
        np.testing.assert_allclose(o, 0.375 * v * float(k @ q) / math.sqrt(D),
                                   rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- P4 -------
@pytest.mark.parametrize("NV,NK", [(4, 2), (48, 16), (6, 3)])
def test_p4_tiled_key_head_pairing(orc, NV, NK):
    """Value head h reads key head h mod NK (tiled), not h // (NV/NK).

    With S = 0, alpha = beta = 1, k_g = e_g and v_h = (h+1) 1, head h must fill
    column (h mod NK) with h+1 and leave every other column zero."""
    D = max(4, NK)
    state = np.zeros((1, NV * D * D), np.float32)
    q = np.zeros((1, NK * D), np.float32)
    k = np.zeros((1, NK * D), np.float32)
    for g in range(NK):
        k[0, g * D + g] = 1.0
        q[0, g * D + g] = 1.0
    v = np.repeat(np.arange(1, NV + 1, dtype=np.float32), D)[None, :]
    ones = np.ones((1, NV), np.float32)
    out = orc.decode(state, q, k, v, ones, ones, B=1, NK=NK, NV=NV, Dk=D, Dv=D)
    tiles = state.reshape(NV, D, D)
    for h in range(NV):
        want = np.zeros((D, D), np.float32)
        want[:, h % NK] = h + 1
        assert np.array_equal(tiles[h], want), f"head {h}"
        # reading with q_g = e_g returns column g: (h+1)/sqrt(D)
        np.testing.assert_allclose(out[0, h * D:(h + 1) * D], (h + 1) / math.sqrt(D), rtol=1e-15)
    if NV // NK > 1:
        # the repeat-interleave pairing would have put head 1 in column 0
        assert tiles[1][:, 0].max() == 0.0


# ---------------------------------------------------------------- P5 -------
def test_p5_hand_derived_d4_example(orc):
    g = json.load(open(GOLDEN))
    a = g["step_a"]
    S1, o = orc.head_step(np.zeros((4, 4)), a["q"], a["k"], a["v"], a["alpha"], a["beta"])
    assert np.array_equal(S1[:, 0], a["S1_column0"]) and not S1[:, 1:].any()
    assert np.array_equal(o, a["o"])
    n = a["norm"]
    y = orc.gated_rmsnorm(o, n["z"], n["gn"], n["eps"])
    np.testing.assert_allclose(y, n["y"], rtol=1e-14, atol=0)
    for key in ("step_b_readback", "step_b_correction"):
        s = g[key]
        S2, o2 = orc.head_step(S1, s["q"], s["k"], s["v"], s["alpha"], s["beta"])
        assert np.array_equal(S2[:, 0], s["S2_column0"]) and not S2[:, 1:].any(), key
        assert np.array_equal(o2, s["o"]), key
    s = g["step_b_erase"]
    S2, o2 = orc.head_step(np.ones((4, 4)), s["q"], s["k"], s["v"], s["alpha"], s["beta"])
    nz = s["S1_nonzero"]
    want = np.zeros((4, 4)); want[nz["row"], nz["col"]] = nz["value"]
    assert np.array_equal(S2, want)
    assert np.array_equal(o2, s["o"])


def test_p5_storage_driver_matches_hand_example(orc):
    """The same worked example through the fp32-storage batch driver, 2 tokens."""
    g = json.load(open(GOLDEN))
    a, s = g["step_a"], g["step_b_correction"]
    state = np.zeros((1, 16), np.float32)
    q = np.array([a["q"], s["q"]], np.float32)
    k = np.array([a["k"], s["k"]], np.float32)
    v = np.array([a["v"], s["v"]], np.float32)
    al = np.array([[a["alpha"]], [s["alpha"]]], np.float32)
    be = np.array([[a["beta"]], [s["beta"]]], np.float32)
    out = orc.seq(state, q, k, v, al, be, B=1, T=2, NK=1, NV=1, Dk=4, Dv=4)
    assert np.array_equal(out[0], a["o"]) and np.array_equal(out[1], s["o"])
    assert np.array_equal(state.reshape(4, 4)[:, 0], s["S2_column0"])


# ---------------------------------------------------------------- P6 -------
def test_p6_brute_force_matrix_form(orc):
    """Small D: the literal products alpha S (I - beta k k^T) + beta v k^T and
    S' q / sqrt(D) with numpy matmul agree with the oracle's O(D^2) loops."""
    r = rng(16)
    for D in (1, 2, 3, 4, 5, 8):
        for _ in range(20):
            S = r.standard_normal((D, D))
            q, k, v = r.standard_normal(D), r.standard_normal(D), r.standard_normal(D)
            al, be = r.random(), 2 * r.random()
            want = al * S @ (np.eye(D) - be * np.outer(k, k)) + be * np.outer(v, k)
            S1, o = orc.head_step(S, q, k, v, al, be)
            np.testing.assert_allclose(S1, want, rtol=0, atol=1e-13 * (1 + np.abs(want).max()))
            np.testing.assert_allclose(o, want @ q / math.sqrt(D), rtol=0,
                                       atol=1e-13 * (1 + np.abs(want).max()))


def test_p6_factored_form_agrees(orc):
    """The equal factoring o = (alpha S q + coef (k.q)) / sqrt(D) with
    coef = beta (v - alpha S k), evaluated with numpy, matches to 1e-12."""
    r = rng(17)
    D = 128
    S = 0.02 * r.standard_normal((D, D))
    q, k, v = unit(r, D), unit(r, D), r.standard_normal(D)
    al, be = 0.95, 0.6
    coef = be * (v - al * (S @ k))
    want_o = (al * (S @ q) + coef * float(k @ q)) / math.sqrt(D)
    S1, o = orc.head_step(S, q, k, v, al, be)
    np.testing.assert_allclose(o, want_o, rtol=0, atol=1e-12 * np.abs(want_o).max())
    np.testing.assert_allclose(S1, al * S + np.outer(coef, k), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- P7 -------
@pytest.mark.parametrize("D", [4, 128])
def test_p7_associative_memory_sequence(orc, D):
    """S0 = 0, alpha = beta = 1, keys e_(t mod D), T <= D tokens: column t holds
    v_t exactly, and a query e_t reads back v_t / sqrt(D)."""
    T = min(D, 16)
    r = rng(18)
    q = np.zeros((T, D), np.float32); k = np.zeros((T, D), np.float32)
    for t in range(T):
        q[t, t % D] = 1.0
        k[t, t % D] = 1.0
    v = r.standard_normal((T, D)).astype(np.float32)
    ones = np.ones((T, 1), np.float32)
    state = np.zeros((1, D * D), np.float32)
    out = orc.seq(state, q, k, v, ones, ones, B=1, T=T, NK=1, NV=1, Dk=D, Dv=D)
    S = state.reshape(D, D)
    for t in range(T):
        assert np.array_equal(S[:, t], v[t])
        np.testing.assert_allclose(out[t], v[t].astype(np.float64) / math.sqrt(D), rtol=1e-15)
    assert not S[:, T:].any()


# ---------------------------------------------------------------- P8 -------
def test_p8_pure_decay_closed_form(orc):
    """beta = 0 with constant alpha: S_T = alpha^T S_0 and o_t = alpha^(t+1) S_0 q_t / sqrt(D)."""
    r = rng(19)
    D, T, al = 16, 12, 0.8125            # alpha exact in binary
    S0 = (0.02 * r.standard_normal((D, D))).astype(np.float32)
    state = S0.reshape(1, -1).copy()
    q = np.stack([unit(r, D) for _ in range(T)]).astype(np.float32)
    k = np.stack([unit(r, D) for _ in range(T)]).astype(np.float32)
    v = r.standard_normal((T, D)).astype(np.float32)
    out = orc.seq(state, q, k, v, np.full((T, 1), al, np.float32), np.zeros((T, 1), np.float32),
                  B=1, T=T, NK=1, NV=1, Dk=D, Dv=D)
    S0d = S0.astype(np.float64)
    np.testing.assert_allclose(state.reshape(D, D), al ** T * S0d, rtol=1e-6, atol=0)
    for t in range(T):
        np.testing.assert_allclose(out[t], al ** (t + 1) * (S0d @ q[t]) / math.sqrt(D),
                                   rtol=1e-6, atol=1e-9)


# ---------------------------------------------------------------- P9 -------
def test_p9_norm_closed_forms(orc):
    r = rng(20)
    D = 128
    o = r.standard_normal(D) * 1e-2
    gn = 1 + 0.1 * r.standard_normal(D)
    z = r.standard_normal(D)
    # z = 0 gates everything off
    assert not orc.gated_rmsnorm(o, np.zeros(D), gn, 1e-6).any()
    # eps = 0: invariant to o -> c o for c > 0
    y1 = orc.gated_rmsnorm(o, z, gn, 0.0)
    y2 = orc.gated_rmsnorm(3.7 * o, z, gn, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)
    silu = z / (1 + np.exp(-z))
    # constant o = c 1: y = gn sign(c) silu(z) at eps = 0, and
    # y = gn c / sqrt(c^2 + eps) silu(z) in general (eps inside the root, weight before the gate)
    for c, eps in ((-0.3, 0.0), (2.0, 0.0), (0.01, 1e-4), (0.5, 1.0)):
        y = orc.gated_rmsnorm(np.full(D, c), z, gn, eps)
        np.testing.assert_allclose(y, gn * c / math.sqrt(c * c + eps) * silu, rtol=1e-13)


# --------------------------------------------------------------- P10 -------
def test_p10_output_scale_is_one_over_sqrt_dk(orc):
    """o is S' q / sqrt(D) for the state the step returns; dropping the scale
    would change the real-head norm output far beyond any tolerance."""
    c = inputs.make_case(21, B=1, NK=16, NV=48, D=128)
    st = c.state.copy()
    out = orc.decode(st, c.q, c.k, c.v, c.alpha, c.beta, B=1, NK=16, NV=48, Dk=128, Dv=128)
    S1 = st.reshape(48, 128, 128).astype(np.float64)
    for h in (0, 17, 47):
        g = h % 16
        qg = c.q[0, g * 128:(g + 1) * 128].astype(np.float64)
        np.testing.assert_allclose(out[0, h * 128:(h + 1) * 128] * math.sqrt(128), S1[h] @ qg,
                                   rtol=0, atol=1e-6 * np.abs(S1[h] @ qg).max())
    y = orc.decode(c.state.copy(), c.q, c.k, c.v, c.alpha, c.beta, B=1, NK=16, NV=48, Dk=128,
                   Dv=128, z=c.z, gn=c.gn)
    y_unscaled = np.concatenate([
        orc.gated_rmsnorm(out[0, h * 128:(h + 1) * 128] * math.sqrt(128),
                          c.z[0, h * 128:(h + 1) * 128], c.gn, 1e-6) for h in range(48)])
    rel = np.abs(y_unscaled - y[0]).max() / np.abs(y[0]).max()
    assert rel > 1e-3


# --------------------------------------------------------------- P11 -------
def _f16_sample():
    r = rng(22)
    pats = [r.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)]
    h = np.arange(1 << 16, dtype=np.uint32)
    f = h.astype(np.uint16).view(np.float16).astype(np.float32).view(np.uint32)
    # every binary16 value, its midpoints to the next value, and +-1 ulp around them
    with np.errstate(over="ignore", invalid="ignore"):
        nxt = np.nextafter(h.astype(np.uint16).view(np.float16), np.float16(np.inf))
        mid = (h.astype(np.uint16).view(np.float16).astype(np.float64)
               + nxt.astype(np.float64)) / 2
    mid = mid[np.isfinite(mid)].astype(np.float32).view(np.uint32)
    for base in (f, mid):
        for d in (-2, -1, 0, 1, 2):
            pats.append((base.astype(np.int64) + d).astype(np.uint32))
    # all exponents near the binary16 range edges, every 16th mantissa
    e = np.arange(100, 150, dtype=np.uint32)
    m = np.arange(0, 1 << 23, 16, dtype=np.uint32)
    edge = (e[:, None] << 23 | m[None, :]).ravel()
    pats += [edge, edge | 0x80000000]
    return np.concatenate(pats).view(np.float32)


def test_p11_f32_to_f16_matches_numpy_rne(orc):
    x = _f16_sample()
    got = orc.f32_to_f16_bits(x)
    with np.errstate(over="ignore", invalid="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7c00) == 0x7c00) and np.all(got[nan] & 0x03ff)


def test_p11_f16_to_f32_exhaustive(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_bits_to_f32(h)
    want = h.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    assert np.isnan(got[nan]).all()


def test_p11_bf16_matches_torch_rne(orc):
    torch = pytest.importorskip("torch")
    r = rng(23)
    bits = np.concatenate([r.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32),
                           np.arange(0, 1 << 20, dtype=np.uint32),                 # subnormals
                           (np.arange(0x3f800000, 0x3f800000 + (1 << 18), dtype=np.uint32))])
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    got = orc.f64_to_bf16_bits(x.astype(np.float64))
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


# --------------------------------------------------------------- P12 -------
def test_p12_sequence_equals_chained_steps(orc):
    c = inputs.make_case(24, B=2, NK=2, NV=4, D=16, T=6)
    st_seq = c.state.copy()
    out = orc.seq(st_seq, c.q, c.k, c.v, c.alpha, c.beta, B=2, T=6, NK=2, NV=4, Dk=16, Dv=16,
                  z=c.z, gn=c.gn)
    st = c.state.copy()
    for t in range(6):
        rows = [b * 6 + t for b in range(2)]
        o = orc.decode(st, c.q[rows], c.k[rows], c.v[rows], c.alpha[rows], c.beta[rows], B=2,
                       NK=2, NV=4, Dk=16, Dv=16, z=c.z[rows], gn=c.gn)
        assert np.array_equal(o, out[rows])
    assert np.array_equal(st.view(np.uint32), st_seq.view(np.uint32))


# --------------------------------------------------------------- P13 -------
def test_p13_pitch_pads_and_batch_permutation(orc):
    D, NV, NK, B = 8, 4, 2, 3
    c = inputs.make_case(25, B=B, NK=NK, NV=NV, D=D, pitch=NV * D * D + 40)
    st = c.state.copy()
    out = orc.decode(st, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D)
    assert np.isnan(st[:, NV * D * D:]).all()
    perm = [2, 0, 1]
    st_p = c.state[perm].copy()
    out_p = orc.decode(st_p, c.q[perm], c.k[perm], c.v[perm], c.alpha[perm], c.beta[perm], B=B,
                       NK=NK, NV=NV, Dk=D, Dv=D)
    assert np.array_equal(out_p, out[perm])
    assert np.array_equal(st_p[:, :NV * D * D], st[perm][:, :NV * D * D])


def test_p13_strided_rows_equal_dense_rows(orc):
    """q|k|v packed in one wide projection row (element strides) gives the same result."""
    D, NV, NK, B = 8, 4, 2, 2
    c = inputs.make_case(26, B=B, NK=NK, NV=NV, D=D)
    W = 2 * NK * D + NV * D + 8
    packed = np.zeros((B, W), np.float32)
    packed[:, :NK * D] = c.q
    packed[:, NK * D:2 * NK * D] = c.k
    packed[:, 2 * NK * D:2 * NK * D + NV * D] = c.v
    st1, st2 = c.state.copy(), c.state.copy()
    o1 = orc.decode(st1, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D)
    o2 = orc.decode(st2, packed[:, :NK * D], packed[:, NK * D:2 * NK * D],
                    packed[:, 2 * NK * D:2 * NK * D + NV * D], c.alpha, c.beta,
                    B=B, NK=NK, NV=NV, Dk=D, Dv=D)
    assert np.array_equal(o1, o2) and np.array_equal(st1, st2)


# --------------------------------------------------------------- P14 -------
def test_p14_contraction_bound_and_long_run_stability(orc):
    """With alpha <= 1, beta in [0, 1] and |k| = 1: |S'|_F <= alpha |S|_F + beta |v|
    (|I - beta k k^T|_2 = 1), and 4096 steps stay finite."""
    r = rng(27)
    D = 32
    S = 0.02 * r.standard_normal((D, D))
    for _ in range(200):
        k, q, v = unit(r, D), unit(r, D), r.standard_normal(D)
        al, be = 0.9 + 0.099 * r.random(), r.random()
        S1, _ = orc.head_step(S, q, k, v, al, be)
        assert np.linalg.norm(S1) <= al * np.linalg.norm(S) + be * np.linalg.norm(v) + 1e-12
        S = S1
    c = inputs.make_case(28, B=1, NK=1, NV=1, D=16, T=4096)
    st = c.state.copy()
    out = orc.seq(st, c.q, c.k, c.v, c.alpha, c.beta, B=1, T=4096, NK=1, NV=1, Dk=16, Dv=16,
                  z=c.z, gn=c.gn)
    assert np.isfinite(out).all() and np.isfinite(st).all()


# ---------------------------------------------------------- f16 driver -----
def test_f16_storage_rounds_every_step(orc):
    """The binary16 state driver equals the double step followed by RNE to binary16."""
    c = inputs.make_case(29, B=1, NK=1, NV=1, D=8, T=1)
    s16 = orc.f32_to_f16_bits(c.state)
    s_before = orc.f16_bits_to_f32(s16).astype(np.float64).reshape(8, 8)
    out = orc.decode(s16, c.q, c.k, c.v, c.alpha, c.beta, B=1, NK=1, NV=1, Dk=8, Dv=8,
                     state_kind=orc.STATE_F16)
    S1, o = orc.head_step(s_before, c.q[0], c.k[0], c.v[0], float(c.alpha[0, 0]),
                          float(c.beta[0, 0]))
    want = S1.astype(np.float16).view(np.uint16).reshape(1, -1)   # numpy: RNE from double
    assert np.array_equal(s16, want)
    assert np.array_equal(out[0], o)


# ------------------------------------------------ P15: the front end ------
def _silu(x):
    from scipy.special import expit
    return np.asarray(x, dtype=np.float64) * expit(np.asarray(x, dtype=np.float64))


def _gates_zero(NV):
    z = np.zeros(NV, dtype=np.float32)
    return z, z.copy(), z.copy(), z.copy()


@pytest.mark.parametrize("tap", [0, 1, 3])
def test_p15_conv_ring_is_a_delay_line(orc, tap):
    """A one-hot tap weight turns the depthwise causal conv into a delay line:
    with weight 1 on tap j of a 4-deep ring, token n sees the input of token
    n - (3 - j) (zero before the first), then silu.  The ring always holds the
    last four inputs, oldest first.  v is neither mixed nor normalised."""
    NK, NV, D, taps = 1, 2, 4, 4
    C = (2 * NK + NV) * D
    r = rng(150 + tap)
    ring = np.zeros((taps, C), dtype=np.float32)
    w = np.zeros((taps, C), dtype=np.float32)
    w[tap] = 1.0
    xs = r.standard_normal((9, C)).astype(np.float32)
    br, ar, dt, rate = _gates_zero(NV)
    delay = taps - 1 - tap
    for n in range(9):
        q, k, v, al, be = orc.frontend_token(ring, xs[n], w, br, ar, dt, rate, NK=NK, NV=NV, D=D)
        src = xs[n - delay].astype(np.float64) if n >= delay else np.zeros(C)
        np.testing.assert_allclose(v, _silu(src[2 * NK * D:]), rtol=1e-15, atol=1e-300)
        hist = np.zeros((taps, C), dtype=np.float32)
        for t in range(taps):
            m = n - (taps - 1 - t)
            if m >= 0:
                hist[t] = xs[m]
        assert np.array_equal(ring, hist), n
        if n >= delay:   # q and k blocks point along silu of the delayed input
            for blk, got in ((0, q), (1, k)):
                ref = _silu(src[blk * D:(blk + 1) * D])
                cos = got @ ref / (np.linalg.norm(got) * np.linalg.norm(ref))
                assert cos == pytest.approx(1.0, abs=1e-14)


def test_p15_conv_sums_every_tap(orc):
    """All-ones weights over a ring filled with one constant c give the
    pre-activation taps * c in every channel."""
    NK, NV, D, taps = 1, 1, 4, 4
    C = (2 * NK + NV) * D
    ring = np.zeros((taps, C), dtype=np.float32)
    w = np.ones((taps, C), dtype=np.float32)
    br, ar, dt, rate = _gates_zero(NV)
    c = np.float32(0.375)
    for _ in range(taps):
        q, k, v, _, _ = orc.frontend_token(ring, np.full(C, c, np.float32), w, br, ar, dt, rate,
                                           NK=NK, NV=NV, D=D)
    np.testing.assert_allclose(v, _silu(np.full(D, taps * 0.375)), rtol=1e-15)


def test_p15_l2_normalises_q_and_k_heads(orc):
    """Each q and each k head block is scaled to norm sqrt(s / (s + eps)), where s
    is its squared norm before scaling (eps inside the root); with eps = 0 the
    blocks are unit vectors.  Blocks are per head, not over all of q."""
    NK, NV, D, taps = 3, 3, 8, 2
    C = (2 * NK + NV) * D
    r = rng(152)
    w = np.zeros((taps, C), dtype=np.float32)
    w[taps - 1] = 1.0
    x = r.standard_normal(C).astype(np.float32)
    x[:D] *= 10.0                            # head blocks of very different sizes
    br, ar, dt, rate = _gates_zero(NV)
    for eps in (0.0, 0.25):
        ring = np.zeros((taps, C), dtype=np.float32)
        q, k, _, _, _ = orc.frontend_token(ring, x, w, br, ar, dt, rate, NK=NK, NV=NV, D=D,
                                           l2_eps=eps)
        pre = _silu(x)
        for blk in range(2 * NK):
            s = float(pre[blk * D:(blk + 1) * D] @ pre[blk * D:(blk + 1) * D])
            got = (q if blk < NK else k)[(blk % NK) * D:(blk % NK + 1) * D]
            assert np.linalg.norm(got) == pytest.approx(math.sqrt(s / (s + eps)), rel=1e-14)


def test_p15_gate_closed_forms(orc):
    """beta = sigmoid(br): 1/2 at 0 and beta(-x) = 1 - beta(x).  The decay
    (1 + e^(ar+dt))^rate: 1 at rate 0, 2^rate at ar + dt = 0, e^rate at
    ar + dt = ln(e - 1), and exp(rate * softplus(ar + dt)) in general."""
    NK, NV, D, taps = 1, 8, 4, 1
    C = (2 * NK + NV) * D
    r = rng(153)
    w = np.ones((taps, C), dtype=np.float32)
    x = np.zeros(C, dtype=np.float32)
    br = np.array([0, 1.5, -1.5, 4, -4, 0.25, 9, -9], dtype=np.float32)
    ar = r.uniform(-3, 3, NV).astype(np.float32)
    dt = r.uniform(-3, 3, NV).astype(np.float32)
    rate = -r.uniform(0.001, 0.08, NV).astype(np.float32)
    ar[1], dt[1] = 0.0, 0.0
    ar[2], dt[2] = np.float32(math.log(math.e - 1)), 0.0
    rate[3] = 0.0
    ring = np.zeros((taps, C), dtype=np.float32)
    _, _, _, al, be = orc.frontend_token(ring, x, w, br, ar, dt, rate, NK=NK, NV=NV, D=D)
    assert be[0] == 0.5
    assert be[1] + be[2] == pytest.approx(1.0, abs=1e-15)
    assert be[3] + be[4] == pytest.approx(1.0, abs=1e-15)
    from scipy.special import expit
    np.testing.assert_allclose(be, expit(br.astype(np.float64)), rtol=1e-15)
    assert be[6] > 0.9998 and be[7] < 2e-4       # a large positive logit writes fully
    assert al[3] == 1.0
    assert al[1] == pytest.approx(2.0 ** float(rate[1]), rel=1e-15)
    u2 = float(ar[2]) + float(dt[2])
    assert al[2] == pytest.approx(math.exp(float(rate[2]) * math.log1p(math.exp(u2))), rel=1e-14)
    assert al[2] == pytest.approx(math.exp(float(rate[2])), rel=1e-7)
    u = ar.astype(np.float64) + dt.astype(np.float64)
    np.testing.assert_allclose(al, np.exp(rate.astype(np.float64) * np.logaddexp(0.0, u)),
                               rtol=1e-13)
    assert ((al > 0) & (al <= 1)).all()


def test_p15_fused_decode_composes_front_end_and_step(orc):
    """The fused decode of a batch equals, sequence by sequence, the front end
    followed by the pinned head step with key head g = h mod NK and the gated
    norm; the conv ring of each sequence sits at its own (padded) stride and
    the state pads stay untouched."""
    B, NK, NV, D, taps = 3, 2, 6, 8, 4
    C = (2 * NK + NV) * D
    r = rng(154)
    pitch = NV * D * D + 16
    state = np.full((B, pitch), np.nan, dtype=np.float32)
    state[:, :NV * D * D] = 0.02 * r.standard_normal((B, NV * D * D))
    ring = np.zeros((B, taps * C + 8), dtype=np.float32)
    ring[:, :taps * C] = r.standard_normal((B, taps * C))
    x = r.standard_normal((B, C + 4)).astype(np.float32)
    w = (0.5 * r.standard_normal((taps, C))).astype(np.float32)
    gates = r.standard_normal((B, 2 * NV)).astype(np.float32)
    br, ar = gates[:, :NV], gates[:, NV:]
    dt = r.standard_normal(NV).astype(np.float32)
    rate = -r.uniform(0.001, 0.08, NV).astype(np.float32)
    z = r.standard_normal((B, NV * D)).astype(np.float32)
    gn = (1 + 0.1 * r.standard_normal(D)).astype(np.float32)
    st0, ring0 = state.copy(), ring.copy()
    y = orc.fused_decode(state, ring, x, w, br, ar, dt, rate, B=B, NK=NK, NV=NV, D=D, taps=taps,
                         z=z, gn=gn)
    assert np.isnan(state[:, NV * D * D:]).all()
    assert np.array_equal(ring[:, taps * C:], ring0[:, taps * C:])
    for b in range(B):
        rb = ring0[b, :taps * C].reshape(taps, C).copy()
        q, k, v, al, be = orc.frontend_token(rb, x[b, :C], w, br[b], ar[b], dt, rate,
                                             NK=NK, NV=NV, D=D)
        assert np.array_equal(ring[b, :taps * C].reshape(taps, C), rb)
        for h in range(NV):
            g = h % NK
            S = st0[b, h * D * D:(h + 1) * D * D].reshape(D, D).astype(np.float64)
            S1, o = orc.head_step(S, q[g * D:(g + 1) * D], k[g * D:(g + 1) * D],
                                  v[h * D:(h + 1) * D], al[h], be[h])
            yr = orc.gated_rmsnorm(o, z[b, h * D:(h + 1) * D], gn, 1e-6)
            np.testing.assert_allclose(y[b, h * D:(h + 1) * D], yr, rtol=1e-12, atol=1e-15)
            assert np.array_equal(state[b, h * D * D:(h + 1) * D * D],
                                  S1.astype(np.float32).reshape(-1))


# ------------------------------------------- P16: int8 group quantisation --
def test_p16_quant_exact_cases(orc):
    """Scale = amax/127 per 32 values; ties round to even; a zero group has
    scale 1 and zero codes; groups are 32 consecutive values."""
    y = np.zeros(96, dtype=np.float32)
    y[0] = 127.0                      # scale exactly 1
    y[1:8] = [2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5]
    y[32] = -12.7                     # second group: amax 12.7
    y[33] = 6.35
    codes, scales = orc.quant_groups32(y)
    assert scales[0] == np.float32(1.0)
    assert list(codes[:8]) == [127, 2, 4, -2, -4, 0, 2, 0]
    assert scales[1] == np.float32(np.float32(12.7) / np.float32(127.0))
    assert codes[32] == -127
    assert scales[2] == 1.0 and not codes[64:].any()


def test_p16_quant_round_trip_bound(orc):
    """|y - code*scale| <= scale/2 (plus the rounding of y/scale), the group's
    largest magnitude maps to +-127 and every code is in [-127, 127]."""
    r = rng(160)
    y = (r.standard_normal(32 * 64) * np.exp(r.uniform(-8, 8, 32 * 64))).astype(np.float32)
    codes, scales = orc.quant_groups32(y)
    ys = y.reshape(-1, 32).astype(np.float64)
    cs = codes.reshape(-1, 32).astype(np.float64)
    sc = scales.astype(np.float64)[:, None]
    assert (np.abs(ys - cs * sc) <= sc * (0.5 + 1e-6)).all()
    assert (np.abs(codes.astype(int)) <= 127).all()
    top = np.abs(ys).argmax(axis=1)
    assert (np.abs(cs[np.arange(cs.shape[0]), top]) == 127).all()
    np.testing.assert_allclose(sc[:, 0], np.abs(ys).max(axis=1) / 127, rtol=1e-7)


def test_threaded_driver_equals_serial(orc):
    """The multi-threaded timing driver runs the same per-head code: outputs and
    states equal the serial call bit for bit, for any split of the heads."""
    c = inputs.make_case(91, B=3, NK=2, NV=4, D=8, T=5)
    st0 = c.state.copy()
    ref = orc.seq(st0, c.q, c.k, c.v, c.alpha, c.beta, B=3, T=5, NK=2, NV=4, Dk=8, Dv=8,
                  z=c.z, gn=c.gn, eps=1e-6)
    heads = [(b, h) for b in range(3) for h in range(4)]
    for threads in (1, 3, 5, 12):
        st = c.state.copy()
        got = orc.seq_head_threaded(st, c.q, c.k, c.v, c.alpha, c.beta, B=3, T=5, NK=2, NV=4,
                                    Dk=8, Dv=8, heads=heads, threads=threads, z=c.z, gn=c.gn,
                                    eps=1e-6)
        assert np.array_equal(got, ref), threads
        assert np.array_equal(st, st0), threads
