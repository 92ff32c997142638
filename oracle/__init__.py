"""CPU oracle of the gated delta rule recurrence (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never does, and this package never imports the product.

The arithmetic lives in ``gdn_oracle.c`` (plain C, IEEE double); this module
builds it with gcc and marshals numpy arrays through ctypes.  Array layout
conventions match the C file's header:

* ``state``: 2-D ``[B, pitch]`` (float32, or uint16 binary16 bits); head ``h``'s
  ``Dv x Dk`` tile starts at column ``h*Dv*Dk``, row-major, key index contiguous.
* ``q``/``k``: 2-D ``[B*T, >= NK*Dk]``; ``v``/``z``: ``[B*T, >= NV*Dv]``;
  ``alpha``/``beta``: ``[B*T, >= NV]``; ``gn``: ``[Dv]``.  Row ``r = b*T + t``.
  Rows may be strided (a view into a wider buffer); the inner dim is contiguous.
* outputs are float64 ``[B*T, NV*Dv]`` (raw o, or the gated-norm y when ``z``
  is given), before any rounding to an output dtype.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

STATE_F32 = 0
STATE_F16 = 1

_lib = None


def build() -> str:
    """Compile ``gdn_oracle.c`` into ``liboracle.so`` with gcc (always rebuilds)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    for name in ("orc_f32_to_f16_array", "orc_f16_to_f32_array", "orc_f64_to_bf16_array"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [vp, vp, i64]
    lib.orc_head_step.restype = None
    lib.orc_head_step.argtypes = [vp, vp, vp, vp, dbl, dbl, i32, i32, vp]
    lib.orc_gated_rmsnorm.restype = None
    lib.orc_gated_rmsnorm.argtypes = [vp, vp, vp, dbl, i32, vp]
    common = [vp, i64, vp, vp, i64, vp, i64, vp, vp, i64, vp, i64, vp, dbl, vp, i64,
              i32, i32, i32, i32]
    lib.orc_seq_head.restype = i32
    lib.orc_seq_head.argtypes = [i32, i32, i32, i32] + common
    lib.orc_seq.restype = i32
    lib.orc_seq.argtypes = [i32, i32, i32] + common
    lib.orc_seq_head_list.restype = i32
    lib.orc_seq_head_list.argtypes = [i32, vp, vp, i32, i32] + common
    f32p = vp
    lib.orc_frontend_token.restype = i32
    lib.orc_frontend_token.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, dbl,
                                       vp, vp, vp, vp, vp]
    lib.orc_fused_decode.restype = i32
    lib.orc_fused_decode.argtypes = [i32, i32, i32, i32, i32, f32p, i64, f32p, i64, vp, i64, vp,
                                     vp, vp, i64, vp, vp, dbl, vp, i64, vp, dbl, vp, i64,
                                     vp, vp, vp, vp, vp]
    lib.orc_quant_groups32.restype = i32
    lib.orc_quant_groups32.argtypes = [vp, i64, vp, vp]
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _row_stride(a: np.ndarray) -> int:
    if a.ndim != 2 or a.strides[1] != a.itemsize:
        raise ValueError("expected a 2-D array with a contiguous inner dimension")
    return a.strides[0] // a.itemsize


# --------------------------------------------------------------------------
# conversions
# --------------------------------------------------------------------------

def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 -> binary16 bit patterns, round to nearest even (uint16)."""
    src = np.ascontiguousarray(x, dtype=np.float32)
    dst = np.empty(src.shape, dtype=np.uint16)
    _load().orc_f32_to_f16_array(_ptr(src), _ptr(dst), src.size)
    return dst


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """binary16 bit patterns -> binary32 (exact)."""
    src = np.ascontiguousarray(h, dtype=np.uint16)
    dst = np.empty(src.shape, dtype=np.float32)
    _load().orc_f16_to_f32_array(_ptr(src), _ptr(dst), src.size)
    return dst


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """double -> bfloat16 bit patterns, round to nearest even (uint16)."""
    src = np.ascontiguousarray(x, dtype=np.float64)
    dst = np.empty(src.shape, dtype=np.uint16)
    _load().orc_f64_to_bf16_array(_ptr(src), _ptr(dst), src.size)
    return dst


# --------------------------------------------------------------------------
# the recurrence
# --------------------------------------------------------------------------

def head_step(S: np.ndarray, q, k, v, alpha: float, beta: float):
    """One step of one value head in double: returns (S', o).

    ``S`` is ``Dv x Dk`` (row = value index); it is not modified."""
    S2 = np.array(S, dtype=np.float64, order="C", copy=True)
    Dv, Dk = S2.shape
    qd = np.ascontiguousarray(q, dtype=np.float64)
    kd = np.ascontiguousarray(k, dtype=np.float64)
    vd = np.ascontiguousarray(v, dtype=np.float64)
    if qd.shape != (Dk,) or kd.shape != (Dk,) or vd.shape != (Dv,):
        raise ValueError("shape mismatch")
    o = np.empty(Dv, dtype=np.float64)
    _load().orc_head_step(_ptr(S2), _ptr(qd), _ptr(kd), _ptr(vd), float(alpha), float(beta),
                          Dk, Dv, _ptr(o))
    return S2, o


def gated_rmsnorm(o, z, gn, eps: float) -> np.ndarray:
    od = np.ascontiguousarray(o, dtype=np.float64)
    zd = np.ascontiguousarray(z, dtype=np.float64)
    gd = np.ascontiguousarray(gn, dtype=np.float64)
    y = np.empty_like(od)
    _load().orc_gated_rmsnorm(_ptr(od), _ptr(zd), _ptr(gd), float(eps), od.shape[0], _ptr(y))
    return y


def _check_inputs(state, q, k, v, alpha, beta, z, gn, state_kind):
    want = np.float32 if state_kind == STATE_F32 else np.uint16
    if state.dtype != want or state.ndim != 2 or not state.flags.c_contiguous:
        raise ValueError(f"state must be a C-contiguous 2-D {np.dtype(want).name} array")
    for name, a in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta)):
        if a.dtype != np.float32:
            raise ValueError(f"{name} must be float32")
    if z is not None and (z.dtype != np.float32 or gn is None or gn.dtype != np.float32):
        raise ValueError("z and gn must be float32")


def seq(state: np.ndarray, q, k, v, alpha, beta, *, B: int, T: int, NK: int, NV: int,
        Dk: int, Dv: int, z=None, gn=None, eps: float = 1e-6,
        state_kind: int = STATE_F32, heads=None) -> np.ndarray:
    """T tokens of the recurrence for every (b, h) (or only ``heads``, a list of
    (b, h) pairs).  ``state`` is updated in place.  Returns float64
    ``[B*T, NV*Dv]``; rows of heads not computed are NaN."""
    _check_inputs(state, q, k, v, alpha, beta, z, gn, state_kind)
    out = np.full((B * T, NV * Dv), np.nan, dtype=np.float64)
    lib = _load()
    args = [_ptr(state), state.shape[1],
            _ptr(q), _ptr(k), _row_stride(q),
            _ptr(v), _row_stride(v),
            _ptr(alpha), _ptr(beta), _row_stride(alpha),
            _ptr(z), _row_stride(z) if z is not None else 0, _ptr(gn), float(eps),
            _ptr(out), _row_stride(out), NK, NV, Dk, Dv]
    if _row_stride(q) != _row_stride(k):
        raise ValueError("q and k must share one row stride")
    if heads is None:
        rc = lib.orc_seq(B, T, state_kind, *args)
        if rc:
            raise RuntimeError("oracle failed")
    else:
        for (b, h) in heads:
            rc = lib.orc_seq_head(int(b), int(h), T, state_kind, *args)
            if rc:
                raise RuntimeError("oracle failed")
    return out


def decode(state: np.ndarray, q, k, v, alpha, beta, *, B: int, NK: int, NV: int, Dk: int,
           Dv: int, z=None, gn=None, eps: float = 1e-6, state_kind: int = STATE_F32,
           heads=None) -> np.ndarray:
    """One token for every sequence of the batch (the T = 1 case of ``seq``)."""
    return seq(state, q, k, v, alpha, beta, B=B, T=1, NK=NK, NV=NV, Dk=Dk, Dv=Dv, z=z, gn=gn,
               eps=eps, state_kind=state_kind, heads=heads)


def seq_head_threaded(state, q, k, v, alpha, beta, *, B, T, NK, NV, Dk, Dv, heads, threads,
                      z=None, gn=None, eps=1e-6, state_kind=STATE_F32):
    """``seq`` over ``heads`` fanned out over ``threads`` host threads.

    The C call releases the GIL, and distinct heads touch disjoint state and
    output, so this is the same oracle run concurrently (used for timing)."""
    from concurrent.futures import ThreadPoolExecutor
    _check_inputs(state, q, k, v, alpha, beta, z, gn, state_kind)
    out = np.full((B * T, NV * Dv), np.nan, dtype=np.float64)
    lib = _load()
    args = [_ptr(state), state.shape[1], _ptr(q), _ptr(k), _row_stride(q), _ptr(v),
            _row_stride(v), _ptr(alpha), _ptr(beta), _row_stride(alpha), _ptr(z),
            _row_stride(z) if z is not None else 0, _ptr(gn), float(eps), _ptr(out),
            _row_stride(out), NK, NV, Dk, Dv]

    # each thread runs a contiguous share of the heads in one C call
    hl = np.asarray(heads, dtype=np.int32).reshape(-1, 2)
    shares = [np.ascontiguousarray(part) for part in np.array_split(hl, max(1, threads)) if len(part)]

    def run(part):
        bs = np.ascontiguousarray(part[:, 0])
        hs = np.ascontiguousarray(part[:, 1])
        return lib.orc_seq_head_list(len(part), _ptr(bs), _ptr(hs), T, state_kind, *args)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        rcs = list(ex.map(run, shares))
    if any(rcs):
        raise RuntimeError("oracle failed")
    return out


# --------------------------------------------------------------------------
# front end (conv ring, silu, L2 of q and k, gates) and the fused decode
# --------------------------------------------------------------------------

def _f32(a, name):
    if a.dtype != np.float32:
        raise ValueError(f"{name} must be float32")
    return a


def frontend_token(ring: np.ndarray, x, w, br, ar, dt, rate, *, NK: int, NV: int, D: int,
                   l2_eps: float = 1e-6):
    """One token of one sequence through the input stage.  ``ring`` (float32,
    C-contiguous ``[taps, C]`` with ``C = (2*NK + NV)*D``) is updated in place.
    Returns float64 ``(q [NK*D], k [NK*D], v [NV*D], alpha [NV], beta [NV])``."""
    taps, C = ring.shape
    if C != (2 * NK + NV) * D or not ring.flags.c_contiguous:
        raise ValueError("ring must be C-contiguous [taps, (2*NK+NV)*D]")
    _f32(ring, "ring")
    xs = np.ascontiguousarray(_f32(x, "x")).reshape(-1)
    ws = np.ascontiguousarray(_f32(w, "w"))
    if xs.size < C or ws.shape != (taps, C):
        raise ValueError("x or w has the wrong shape")
    g = [np.ascontiguousarray(_f32(a, n)).reshape(-1) for a, n in
         ((br, "br"), (ar, "ar"), (dt, "dt"), (rate, "rate"))]
    q = np.empty(NK * D); k = np.empty(NK * D); v = np.empty(NV * D)
    al = np.empty(NV); be = np.empty(NV)
    rc = _load().orc_frontend_token(NK, NV, D, taps, _ptr(ring), _ptr(xs), _ptr(ws), _ptr(g[0]),
                                    _ptr(g[1]), _ptr(g[2]), _ptr(g[3]), float(l2_eps), _ptr(q),
                                    _ptr(k), _ptr(v), _ptr(al), _ptr(be))
    if rc:
        raise RuntimeError("oracle failed")
    return q, k, v, al, be


def fused_decode(state: np.ndarray, ring: np.ndarray, x, w, br, ar, dt, rate, *, B: int,
                 NK: int, NV: int, D: int, taps: int, l2_eps: float = 1e-6, z=None, gn=None,
                 eps: float = 1e-6, return_inputs: bool = False):
    """Front end plus one decode step for B sequences.  ``state`` (float32
    ``[B, pitch]``) and ``ring`` (float32 ``[B, >= taps*C]``) are updated in
    place; ``x`` is ``[B, >= C]``, ``w`` ``[taps, C]``, ``br``/``ar`` ``[B, >= NV]``,
    ``dt``/``rate`` ``[NV]``.  Returns float64 ``[B, NV*D]`` (raw o, or y with
    ``z``), and with ``return_inputs`` also the derived q, k, v, alpha, beta."""
    C = (2 * NK + NV) * D
    for a, n in ((state, "state"), (ring, "ring"), (x, "x"), (w, "w"), (br, "br"), (ar, "ar"),
                 (dt, "dt"), (rate, "rate")):
        _f32(a, n)
    if ring.shape[1] < taps * C or w.shape != (taps, C) or not w.flags.c_contiguous:
        raise ValueError("ring or w has the wrong shape")
    if _row_stride(br) != _row_stride(ar):
        raise ValueError("br and ar must share one row stride")
    if z is not None:
        _f32(z, "z"); _f32(gn, "gn")
    out = np.empty((B, NV * D))
    ins = [np.empty((B, NK * D)), np.empty((B, NK * D)), np.empty((B, NV * D)),
           np.empty((B, NV)), np.empty((B, NV))] if return_inputs else [None] * 5
    rc = _load().orc_fused_decode(B, NK, NV, D, taps, _ptr(state), state.shape[1], _ptr(ring),
                                  _row_stride(ring), _ptr(x), _row_stride(x), _ptr(w), _ptr(br),
                                  _ptr(ar), _row_stride(br), _ptr(np.ascontiguousarray(dt)),
                                  _ptr(np.ascontiguousarray(rate)), float(l2_eps), _ptr(z),
                                  _row_stride(z) if z is not None else 0, _ptr(gn), float(eps),
                                  _ptr(out), _row_stride(out), *[_ptr(a) for a in ins])
    if rc:
        raise RuntimeError("oracle failed")
    return (out, *ins) if return_inputs else out


def quant_groups32(y) -> tuple:
    """int8 codes and fp32 scales of a float32 vector in groups of 32 (decisions
    in binary32).  Returns ``(codes int8 [n], scales float32 [n/32])``."""
    ys = np.ascontiguousarray(_f32(np.asarray(y), "y")).reshape(-1)
    codes = np.empty(ys.size, dtype=np.int8)
    scales = np.empty(ys.size // 32, dtype=np.float32)
    if _load().orc_quant_groups32(_ptr(ys), ys.size, _ptr(codes), _ptr(scales)):
        raise ValueError("length must be a multiple of 32")
    return codes, scales
