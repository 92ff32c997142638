"""Seeded synthetic inputs for the gated delta rule path.

This module only draws random numbers (numpy, no torch, no HIP); it holds none
of the recurrence's arithmetic, so both the HIP path and the CPU oracle can be
fed from it.  The distributions follow the workloads the pages' model shape
implies (Qwen3.8-27B GDN layer: 48 value heads, 16 key heads, head dim 128):

* q, k: standard normal per key head, then scaled to unit L2 norm (in double,
  rounded once to fp32) -- the recurrence expects L2-normalised keys/queries;
* v, z: standard normal; gn = 1 + 0.1 N(0,1);
* alpha ~ U(0.9, 0.999) (a linear decay multiplier), beta ~ U(0, 1);
* state: 0.02 N(0,1) (standard deviation 0.02), or zeros.

Draw order from one ``numpy.random.Generator(PCG64(seed))``: gn, state
(sequence-major, then head, row, column), q, k, v, z, alpha, beta, each over
its whole ``[rows, width]`` array with row ``r = b*T + t``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass
class Case:
    B: int
    T: int
    NK: int
    NV: int
    D: int
    pitch: int
    state: np.ndarray          # float32 [B, pitch]; pads (if any) hold NaN
    q: np.ndarray              # float32 [B*T, NK*D]
    k: np.ndarray              # float32 [B*T, NK*D]
    v: np.ndarray              # float32 [B*T, NV*D]
    z: np.ndarray              # float32 [B*T, NV*D]
    alpha: np.ndarray          # float32 [B*T, NV]
    beta: np.ndarray           # float32 [B*T, NV]
    gn: np.ndarray             # float32 [D]
    eps: float = 1e-6


def _unit_rows(rng: np.random.Generator, rows: int, heads: int, d: int) -> np.ndarray:
    x = rng.standard_normal((rows, heads, d))                  # float64
    x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x.astype(np.float32).reshape(rows, heads * d)


def make_case(seed: int, *, B: int, NK: int, NV: int, D: int, T: int = 1,
              state_init: str = "normal", pitch: Optional[int] = None,
              pad_value: float = float("nan")) -> Case:
    """Draw one workload.  ``pitch`` (elements per sequence slot) defaults to the
    dense ``NV*D*D``; a larger pitch leaves ``pad_value`` in the pad."""
    dense = NV * D * D
    pitch = dense if pitch is None else int(pitch)
    if pitch < dense:
        raise ValueError("pitch smaller than a dense slot")
    rng = np.random.Generator(np.random.PCG64(seed))
    gn = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    state = np.full((B, pitch), pad_value, dtype=np.float32)
    if state_init == "normal":
        state[:, :dense] = 0.02 * rng.standard_normal((B, dense), dtype=np.float32)
    elif state_init == "zero":
        state[:, :dense] = 0.0
    else:
        raise ValueError(state_init)
    rows = B * T
    q = _unit_rows(rng, rows, NK, D)
    k = _unit_rows(rng, rows, NK, D)
    v = rng.standard_normal((rows, NV * D), dtype=np.float32)
    z = rng.standard_normal((rows, NV * D), dtype=np.float32)
    alpha = (0.9 + 0.099 * rng.random((rows, NV))).astype(np.float32)
    beta = rng.random((rows, NV)).astype(np.float32)
    return Case(B=B, T=T, NK=NK, NV=NV, D=D, pitch=pitch, state=state, q=q, k=k, v=v, z=z,
                alpha=alpha, beta=beta, gn=gn)


# The five workloads: shapes of one Qwen3.8-27B GDN layer (48 value heads over 16
# key heads, head dim 128) at several batch sizes, plus a structurally faithful
# miniature (2 value heads over 1 key head, head dim 4).
CONFIGS = {
    "tiny": dict(seed=1, B=1, NK=1, NV=2, D=4, T=8, state_init="zero"),
    "real_head": dict(seed=2, B=1, NK=16, NV=48, D=128, T=1, layers=48),
    "batched": dict(seed=3, B=64, NK=16, NV=48, D=128, T=1, pitch=983040, calls=100),
    "fp16_state": dict(seed=4, B=256, NK=16, NV=48, D=128, T=1, calls=100),
    "sequence": dict(seed=5, B=4, NK=16, NV=48, D=128, T=4096, state_init="zero"),
}


def config_case(name: str, **overrides) -> Case:
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    for extra in ("layers", "calls"):
        cfg.pop(extra, None)
    seed = cfg.pop("seed")
    return make_case(seed, **cfg)


def real_head_layer(layer: int) -> Case:
    """One of the real-head workload's 48 GDN layers, each with its own state
    and inputs: layer ``l`` draws from seed 1000 * (the config's seed) + l."""
    cfg = dict(CONFIGS["real_head"])
    if not 0 <= layer < cfg.pop("layers"):
        raise ValueError("layer out of range")
    seed = cfg.pop("seed")
    return make_case(1000 * seed + layer, **cfg)


@dataclass
class FrontCase:
    """Inputs of the decode with the fused input stage (conv ring, L2, gates)."""
    B: int
    NK: int
    NV: int
    D: int
    taps: int
    pitch: int
    state: np.ndarray          # float32 [B, pitch]; pads hold NaN
    ring: np.ndarray           # float32 [B, ring_pitch]: taps rows of C channels, pads NaN
    x: np.ndarray              # float32 [B, C]: projection rows, channels q | k | v
    w: np.ndarray              # float32 [taps, C]
    br: np.ndarray             # float32 [B, NV]
    ar: np.ndarray             # float32 [B, NV]
    dt: np.ndarray             # float32 [NV]
    rate: np.ndarray           # float32 [NV], negative
    z: np.ndarray              # float32 [B, NV*D]
    gn: np.ndarray             # float32 [D]
    eps: float = 1e-6
    l2_eps: float = 1e-6

    @property
    def C(self) -> int:
        return (2 * self.NK + self.NV) * self.D


def make_frontend_case(seed: int, *, B: int, NK: int, NV: int, D: int, taps: int = 4,
                       pitch: Optional[int] = None, ring_pitch: Optional[int] = None) -> FrontCase:
    """Draw one fused-input-stage workload from one PCG64 stream, in this order:
    gn = 1 + 0.1 N; state 0.02 N; ring N(0,1) (earlier projection rows); x N(0,1);
    conv weights 0.5 N; br, ar N(0,1); dt 0.5 N; rate = -U(0.001, 0.08) (all
    negative and small, the decay exponents the model stores); z N(0,1)."""
    C = (2 * NK + NV) * D
    dense = NV * D * D
    pitch = dense if pitch is None else int(pitch)
    ring_pitch = taps * C if ring_pitch is None else int(ring_pitch)
    if pitch < dense or ring_pitch < taps * C:
        raise ValueError("pitch smaller than a slot")
    rng = np.random.Generator(np.random.PCG64(seed))
    gn = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    state = np.full((B, pitch), np.nan, dtype=np.float32)
    state[:, :dense] = 0.02 * rng.standard_normal((B, dense), dtype=np.float32)
    ring = np.full((B, ring_pitch), np.nan, dtype=np.float32)
    ring[:, :taps * C] = rng.standard_normal((B, taps * C), dtype=np.float32)
    x = rng.standard_normal((B, C), dtype=np.float32)
    w = (0.5 * rng.standard_normal((taps, C))).astype(np.float32)
    br = rng.standard_normal((B, NV), dtype=np.float32)
    ar = rng.standard_normal((B, NV), dtype=np.float32)
    dt = (0.5 * rng.standard_normal(NV)).astype(np.float32)
    rate = (-rng.uniform(0.001, 0.08, NV)).astype(np.float32)
    z = rng.standard_normal((B, NV * D), dtype=np.float32)
    return FrontCase(B=B, NK=NK, NV=NV, D=D, taps=taps, pitch=pitch, state=state, ring=ring, x=x,
                     w=w, br=br, ar=ar, dt=dt, rate=rate, z=z, gn=gn)
