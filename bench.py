"""Benchmark of the gated delta rule decode path on one MI355X.

One step = one ``gdn_decode_norm`` call over a batch of 64 sequences at the real
head shape (NV=48 value heads over NK=16 key heads, D=128, fp32 state with a
1.25x padded slot pitch, fused gated RMS norm, fp32 output): index and pair,
stage the per-head inputs, read the state tile once, reduce, update and write it
back once, normalise and gate.  Consecutive steps cycle through ``--pools``
distinct state pools (default 48, one per GDN layer of the model), so the state
streams from HBM as it does in a real decode token rather than staying in the
256 MB Infinity Cache.  Inputs are resident in HBM before timing starts.

Prints ONE JSON line.  ``value`` is state GB/s (2*B*NV*D*D*4 bytes per step /
step time); ``roofline`` covers the decode kernel with its full algorithmic
bytes (state + inputs + outputs) against the 8 TB/s HBM peak; ``cpu_baseline``
times the CPU oracle on a bounded sample of the same workload.  ``extra`` holds
the other workloads (binary16 state at B=256, the 4096-token sequence
recurrence, the B=1 real-head token over 48 layers, the cache-resident B=64
case); ``--extras batches`` adds the fused-norm decode at other batch sizes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32: dense matrix cores, and vector with packed FMA
PMC_FILE = os.path.join(ROOT, "profiles", "decode_norm_b64_pmc.json")
KERNEL_SOURCES = ("gdn_decode.hip", "gdn_tile.h", "gdn_device.h", "gdn_launch.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_text(raw: bytes) -> bytes:
    """A source file without its comments and blank-line runs, so that the hashes
    below change with the code and not with its documentation."""
    import re
    text = raw.decode("utf-8")
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    lines = [ln.rstrip() for ln in text.splitlines()]
    return "\n".join(ln for ln in lines if ln).encode()


def kernel_hash() -> str:
    """Hash of the decode kernel's sources (code only): the committed traffic
    record of that kernel is reported while it matches."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_deltanet_decode_delta_amd", "csrc", name), "rb") as f:
            h.update(code_text(f.read()))
    return h.hexdigest()[:16]


def head_bytes(D: int, NV: int, NK: int, state_bytes: int, out_bytes: int, norm: bool) -> float:
    """Algorithmic HBM bytes of one (sequence, value head) step: the state tile
    read and written once, q and k of the key head (shared by NV/NK value
    heads), v, alpha, beta, and (with the norm) z, plus the output vector."""
    b = 2.0 * D * D * state_bytes
    b += 2.0 * D * 4 * NK / NV
    b += D * 4 + 8 + D * out_bytes
    if norm:
        b += D * 4
    return b


def _timed(fn, steps: int, warmup: int):
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps          # ms per call


def run_main(g, steps: int, warmup: int, pools: int):
    import torch
    from gated_deltanet_decode_delta_amd import inputs

    cfg = inputs.CONFIGS["batched"]
    B, NK, NV, D, pitch = cfg["B"], cfg["NK"], cfg["NV"], cfg["D"], cfg["pitch"]
    c = inputs.config_case("batched")
    dev = "cuda:0"
    log(f"[bench] main: B={B} NV={NV} NK={NK} D={D} pitch={pitch} pools={pools}")
    st0 = torch.from_numpy(c.state).to(dev)
    states = [st0.clone() for _ in range(pools)]
    del st0
    base = {n: torch.from_numpy(getattr(c, n)).to(dev) for n in ("q", "k", "v", "z", "alpha", "beta")}
    # every pool gets its own input buffers (the base rows rotated by the pool
    # index), so no layer re-reads another layer's inputs from cache
    sets = [{n: torch.roll(t, p, dims=0).contiguous() for n, t in base.items()} for p in range(pools)]
    del base
    gn = torch.from_numpy(c.gn).to(dev)
    outs = [torch.empty((B, NV * D), dtype=torch.float32, device=dev) for _ in range(pools)]

    def step(i):
        p = i % pools
        s = sets[p]
        g.gdn_decode_norm(states[p], s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["z"], gn,
                          c.eps, out=outs[p], num_k_heads=NK, num_v_heads=NV)

    ms = _timed(step, steps, warmup)
    ms_hot = _timed(lambda i: step(0), steps, warmup)
    # five further trials of 200 rotated calls each (median and minimum reported
    # beside the main figure, which stays the one timed region above)
    trials = sorted(_timed(step, 200, 5) for _ in range(5))
    state_bytes = 2.0 * B * NV * D * D * 4
    algo_bytes = B * NV * head_bytes(D, NV, NK, 4, 4, True)
    torch.cuda.synchronize()
    bad = any(not bool(torch.isfinite(o).all()) for o in outs[:2])
    del states, sets, outs
    torch.cuda.empty_cache()
    return dict(B=B, NV=NV, NK=NK, D=D, pitch=pitch, pools=pools, ms=ms, ms_hot=ms_hot,
                trials=trials,
                state_bytes=state_bytes, algo_bytes=algo_bytes, nonfinite=bad)


def run_fp16(g, calls: int):
    import torch
    from gated_deltanet_decode_delta_amd import inputs

    c = inputs.config_case("fp16_state")
    B, NK, NV, D = c.B, c.NK, c.NV, c.D
    dev = "cuda:0"
    log(f"[bench] fp16 state: B={B}")
    st32 = torch.from_numpy(c.state).to(dev)
    st16 = g.gdn_state_f32_to_f16(st32)
    del st32
    # consecutive calls rotate over three 403 MB pools (1.2 GB), so the state
    # streams from HBM and not from the 256 MB Infinity Cache
    pools = [st16] + [st16.clone() for _ in range(2)]
    t = {n: torch.from_numpy(getattr(c, n)).to(dev) for n in ("q", "k", "v", "z", "alpha", "beta", "gn")}
    out = torch.empty((B, NV * D), dtype=torch.bfloat16, device=dev)

    def step(i):
        g.gdn_decode_f16state(pools[i % 3], t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["z"],
                              t["gn"], c.eps, out=out, num_k_heads=NK, num_v_heads=NV)

    # 5 trials of `calls` calls each after a warmup; the median trial is the figure
    trials = sorted(_timed(step, calls, 5) for _ in range(5))
    ms = trials[2]
    state_bytes = 2.0 * B * NV * D * D * 2
    algo = B * NV * head_bytes(D, NV, NK, 2, 2, True)
    del st16, pools, t, out
    torch.cuda.empty_cache()
    return {"workload": "fp16 state decode, B=256, NV=48, NK=16, D=128, fused norm, bf16 out, "
                        "3 state pools in rotation",
            "ms_per_call": round(ms, 5), "trials": f"median of 5 trials x {calls} calls",
            "min_ms_per_call": round(trials[0], 5),
            "state_GBps": round(state_bytes / ms / 1e6, 1),
            "hbm_frac_algorithmic": round(algo / ms / 1e6 / HBM_PEAK_GBS, 4),
            "tokens_per_s_batch": round(B / ms * 1e3, 1),
            "model_tokens_per_s_48_layers": round(B / (48 * ms) * 1e3, 1)}


def _cold_calls(fn, trials: int, pause_s: float):
    """Single synchronised calls, each after the GPU has idled ``pause_s``
    seconds: ms of each call, sorted."""
    import torch
    out = []
    for i in range(trials):
        torch.cuda.synchronize()
        time.sleep(pause_s)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        fn(i)
        end.record()
        torch.cuda.synchronize()
        out.append(start.elapsed_time(end))
    return sorted(out)


def run_seq(g, calls: int):
    import torch
    from gated_deltanet_decode_delta_amd import inputs

    c = inputs.config_case("sequence")
    B, T, NK, NV, D = c.B, c.T, c.NK, c.NV, c.D
    dev = "cuda:0"
    log(f"[bench] sequence: B={B} T={T}")
    t = {n: torch.from_numpy(getattr(c, n)).to(dev) for n in ("q", "k", "v", "z", "alpha", "beta", "gn")}
    st = torch.from_numpy(c.state).to(dev)
    out = torch.empty((B * T, NV * D), dtype=torch.float32, device=dev)

    ws = torch.empty(g.gdn_seq_workspace_bytes(B, T, NV, D), dtype=torch.uint8, device=dev)

    def step(i):   # the workspace entry: chunk pre-pass, then four workgroups per head
        g.gdn_recurrence_seq_ws(st, t["q"], t["k"], t["v"], t["alpha"], t["beta"], out=out,
                                workspace=ws, seq_len=T, num_k_heads=NK, num_v_heads=NV,
                                head_dim=D)

    def step_plain(i):   # no workspace: one workgroup per head
        g.gdn_recurrence_seq(st, t["q"], t["k"], t["v"], t["alpha"], t["beta"], out=out, seq_len=T,
                             num_k_heads=NK, num_v_heads=NV, head_dim=D)

    # after the chip has idled both paths run slower for their first tens of
    # calls, so each gets 40 warmup calls and is timed over 100 (sustained
    # use); single calls after an idle pause are reported beside that
    def step_norm(i):   # with z: the raw pass, then the gated-norm pass over the output rows
        g.gdn_recurrence_seq_ws(st, t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["z"],
                                t["gn"], c.eps, out=out, workspace=ws, seq_len=T,
                                num_k_heads=NK, num_v_heads=NV)

    def step_norm_plain(i):
        g.gdn_recurrence_seq(st, t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["z"], t["gn"],
                             c.eps, out=out, seq_len=T, num_k_heads=NK, num_v_heads=NV)

    cold = _cold_calls(step, 5, 1.0)
    cold_plain = _cold_calls(step_plain, 5, 1.0)
    ms = _timed(step, calls, 40)
    ms_plain = _timed(step_plain, calls, 40)
    ms_norm = _timed(step_norm, calls, 40)
    ms_norm_plain = _timed(step_norm_plain, calls, 40)
    flops = 7.0 * D * D * B * NV * T
    byts = B * T * (2 * NK * D * 4 + NV * (D * 4 + 8 + D * 4)) + 2.0 * B * NV * D * D * 4
    del t, st, out, ws
    torch.cuda.empty_cache()
    return {"workload": "sequence recurrence, B=4, T=4096, NV=48, NK=16, D=128, raw o "
                        "(gdn_recurrence_seq_ws)",
            "ms_per_call": round(ms, 4), "tflops": round(flops / ms / 1e9, 2),
            "fp32_matrix_frac": round(flops / ms / 1e9 / FP32_VALU_PEAK_TFLOPS, 4),
            "GBps": round(byts / ms / 1e6, 1), "tokens_per_s": round(B * T / ms * 1e3, 1),
            "timing": f"sustained: {calls} calls after 40 warmup; cold: 1 call x 5 trials, "
                      "each after 1 s idle",
            "cold_single_call_ms": {"median": round(cold[2], 4), "min": round(cold[0], 4)},
            "no_workspace_ms_per_call": round(ms_plain, 4),
            "no_workspace_tflops": round(flops / ms_plain / 1e9, 2),
            "no_workspace_fp32_matrix_frac": round(flops / ms_plain / 1e9 / FP32_VALU_PEAK_TFLOPS, 4),
            "no_workspace_cold_single_call_ms": {"median": round(cold_plain[2], 4),
                                                 "min": round(cold_plain[0], 4)},
            "z_raw_then_norm_pass_ms_per_call": round(ms_norm, 4),
            "z_raw_then_norm_pass_no_workspace_ms_per_call": round(ms_norm_plain, 4)}


def run_verify(g, calls: int, pools: int = 16):
    """Draft verification on the decode shapes: T tokens per sequence in one
    launch (state read once, T-1 rollback tiles and the final state written),
    against T chained single-token calls on the same pools."""
    import torch
    from gated_deltanet_decode_delta_amd import inputs

    B, NK, NV, D, pitch = 64, 16, 48, 128, 983040
    dev = "cuda:0"
    res = {"workload": "draft verify, B=64, NV=48, NK=16, D=128, fused norm fp32, padded pool"}
    for T in (2, 4):
        log(f"[bench] verify: B={B} T={T} pools={pools}")
        c = inputs.make_case(3100 + T, B=B, NK=NK, NV=NV, D=D, T=T, pitch=pitch)
        st0 = torch.from_numpy(c.state).to(dev)
        states = [st0.clone() for _ in range(pools)]
        del st0
        t = {n: torch.from_numpy(getattr(c, n)).to(dev) for n in ("q", "k", "v", "z", "alpha", "beta", "gn")}
        inters = [torch.empty((B * (T - 1), NV * D * D), device=dev) for _ in range(pools)]
        out = torch.empty((B * T, NV * D), device=dev)
        rows = [torch.arange(B, device=dev) * T + j for j in range(T)]
        per_tok = [{n: t[n][r].contiguous() for n in ("q", "k", "v", "z", "alpha", "beta")} for r in rows]
        out1 = torch.empty((B, NV * D), device=dev)

        def step(i):
            p = i % pools
            g.gdn_decode_verify(states[p], t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["z"],
                                t["gn"], 1e-6, out=out, inter_state=inters[p], num_tokens=T,
                                num_k_heads=NK, num_v_heads=NV)

        def chained(i):
            p = i % pools
            for j in range(T):
                x = per_tok[j]
                g.gdn_decode_norm(states[p], x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["z"],
                                  t["gn"], 1e-6, out=out1, num_k_heads=NK, num_v_heads=NV)

        ms = _timed(step, calls, 5)
        ms_chain = _timed(chained, calls, 5)
        tile = NV * D * D * 4.0
        algo = B * (T + 1) * tile + B * T * NV * (head_bytes(D, NV, NK, 4, 4, True) - 2 * D * D * 4)
        res[f"T{T}"] = {"ms_per_call": round(ms, 5), "hbm_GBps_algorithmic": round(algo / ms / 1e6, 1),
                        "hbm_frac_algorithmic": round(algo / ms / 1e6 / HBM_PEAK_GBS, 4),
                        "chained_decode_ms": round(ms_chain, 5),
                        "speedup_vs_chained": round(ms_chain / ms, 3)}
        del states, inters, t, out, per_tok, out1
        torch.cuda.empty_cache()
    return res


def run_norm_q(g, calls: int, pools: int = 16):
    """The decode workload with the int8 quantised output (codes + one scale per
    32 values) in place of the fp32 y, rotated over state pools."""
    import torch
    from gated_deltanet_decode_delta_amd import inputs

    c = inputs.config_case("batched")
    B, NK, NV, D = c.B, c.NK, c.NV, c.D
    dev = "cuda:0"
    log(f"[bench] norm_q: B={B} pools={pools}")
    st0 = torch.from_numpy(c.state).to(dev)
    states = [st0.clone() for _ in range(pools)]
    del st0
    t = {n: torch.from_numpy(getattr(c, n)).to(dev) for n in ("q", "k", "v", "z", "alpha", "beta", "gn")}
    codes = torch.empty((B, NV * D), dtype=torch.int8, device=dev)
    scales = torch.empty((B, NV * D // 32), dtype=torch.float32, device=dev)

    def step(i):
        g.gdn_decode_norm_q(states[i % pools], t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["z"],
                            t["gn"], c.eps, codes=codes, scales=scales, write_y=False,
                            num_k_heads=NK, num_v_heads=NV)

    ms = _timed(step, calls, 5)
    algo = B * NV * (head_bytes(D, NV, NK, 4, 0, True) + D + D / 32 * 4)
    del states, t, codes, scales
    torch.cuda.empty_cache()
    return {"workload": "decode + gated norm + int8 group quantisation (no fp32 y), B=64, NV=48, "
                        "NK=16, D=128, padded pool",
            "ms_per_call": round(ms, 5),
            "state_GBps": round(2.0 * B * NV * D * D * 4 / ms / 1e6, 1),
            "hbm_frac_algorithmic": round(algo / ms / 1e6 / HBM_PEAK_GBS, 4)}


def run_batches(g, batches=(16, 32, 48, 96, 128)):
    """The fused-norm decode at other batch sizes, fp32 state (fp32 y) and
    binary16 state (bf16 y), each on its own seeded case of the batched
    workload's shape (padded pitch), rotated over enough pools to stream from
    HBM: median of 5 trials of 200 calls per point."""
    import torch
    from gated_deltanet_decode_delta_amd import inputs

    dev = "cuda:0"
    rows = []
    for B in batches:
        c = inputs.config_case("batched", B=B)
        NK, NV, D = c.NK, c.NV, c.D
        pools = max(4, min(48, -(-(3 << 29) // c.state.nbytes)))   # >= 1.5 GB in rotation
        log(f"[bench] batch sweep: B={B} pools={pools}")
        st0 = torch.from_numpy(c.state).to(dev)
        states = [st0.clone() for _ in range(pools)]
        st16 = [g.gdn_state_f32_to_f16(s) for s in states]
        del st0
        base = {n: torch.from_numpy(getattr(c, n)).to(dev) for n in ("q", "k", "v", "z", "alpha", "beta")}
        sets = [{n: torch.roll(t, p, dims=0).contiguous() for n, t in base.items()} for p in range(pools)]
        del base
        gn = torch.from_numpy(c.gn).to(dev)
        out = torch.empty((B, NV * D), dtype=torch.float32, device=dev)
        ob = torch.empty((B, NV * D), dtype=torch.bfloat16, device=dev)

        def f32(i):
            p = i % pools
            s = sets[p]
            g.gdn_decode_norm(states[p], s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["z"], gn,
                              c.eps, out=out, num_k_heads=NK, num_v_heads=NV)

        def f16(i):
            p = i % pools
            s = sets[p]
            g.gdn_decode_f16state(st16[p], s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["z"], gn,
                                  c.eps, out=ob, num_k_heads=NK, num_v_heads=NV)

        row = {"B": B, "pools": pools}
        for name, fn, sb in (("f32", f32, 4), ("f16_state", f16, 2)):
            ms = sorted(_timed(fn, 200, 10) for _ in range(5))[2]
            algo = B * NV * head_bytes(D, NV, NK, sb, 4 if sb == 4 else 2, True)
            row[name + "_us_per_call"] = round(ms * 1e3, 2)
            row[name + "_hbm_frac_algorithmic"] = round(algo / ms / 1e6 / HBM_PEAK_GBS, 4)
        rows.append(row)
        del states, st16, sets, out, ob
        torch.cuda.empty_cache()
    return {"workload": "fused-norm decode by batch size: NV=48, NK=16, D=128, padded pool; fp32 "
                        "state with fp32 y, and binary16 state with bf16 y",
            "trials": "median of 5 trials x 200 calls per point", "points": rows}


def run_raw(g, pools: int = 48):
    """gdn_decode (raw o, no norm) on the B=64 workload, rotated over state
    pools as the main workload is: median and minimum of 5 trials of 200 calls."""
    import torch
    from gated_deltanet_decode_delta_amd import inputs

    c = inputs.config_case("batched")
    B, NK, NV, D = c.B, c.NK, c.NV, c.D
    dev = "cuda:0"
    log(f"[bench] raw decode: B={B} pools={pools}")
    st0 = torch.from_numpy(c.state).to(dev)
    states = [st0.clone() for _ in range(pools)]
    del st0
    base = {n: torch.from_numpy(getattr(c, n)).to(dev) for n in ("q", "k", "v", "alpha", "beta")}
    sets = [{n: torch.roll(t, p, dims=0).contiguous() for n, t in base.items()} for p in range(pools)]
    del base
    outs = [torch.empty((B, NV * D), dtype=torch.float32, device=dev) for _ in range(pools)]

    def step(i):
        p = i % pools
        s = sets[p]
        g.gdn_decode(states[p], s["q"], s["k"], s["v"], s["alpha"], s["beta"], out=outs[p],
                     num_k_heads=NK, num_v_heads=NV, head_dim=D)

    trials = sorted(_timed(step, 200, 10) for _ in range(5))
    ms = trials[2]
    algo = B * NV * head_bytes(D, NV, NK, 4, 4, False)
    del states, sets, outs
    torch.cuda.empty_cache()
    return {"workload": "raw decode (gdn_decode, no norm), B=64, NV=48, NK=16, D=128, padded "
                        f"pool, {pools} state pools in rotation",
            "ms_per_call": round(ms, 5), "min_ms_per_call": round(trials[0], 5),
            "trials": "median of 5 trials x 200 calls",
            "state_GBps": round(2.0 * B * NV * D * D * 4 / ms / 1e6, 1),
            "hbm_frac_algorithmic": round(algo / ms / 1e6 / HBM_PEAK_GBS, 4)}


def run_strided(g, calls: int, pools: int = 16):
    """The decode workload on packed projection rows: q | k | v read as column
    slices of one [B, 10240] row (2048 + 2048 + 6144 floats), z at an offset in a
    [B, 16384] row, alpha and beta interleaved in one [B, 96] row, rotated over
    state pools.  The kernel is the same; only the strides differ."""
    import torch
    from gated_deltanet_decode_delta_amd import inputs

    c = inputs.config_case("batched")
    B, NK, NV, D = c.B, c.NK, c.NV, c.D
    dev = "cuda:0"
    log(f"[bench] strided rows: B={B} pools={pools}")
    st0 = torch.from_numpy(c.state).to(dev)
    states = [st0.clone() for _ in range(pools)]
    del st0
    qkv = torch.empty((B, 10240), dtype=torch.float32, device=dev)
    qkv[:, :NK * D] = torch.from_numpy(c.q).to(dev)
    qkv[:, NK * D:2 * NK * D] = torch.from_numpy(c.k).to(dev)
    qkv[:, 2 * NK * D:] = torch.from_numpy(c.v).to(dev)
    zrow = torch.zeros((B, 16384), dtype=torch.float32, device=dev)
    zrow[:, 8192:8192 + NV * D] = torch.from_numpy(c.z).to(dev)
    ab = torch.empty((B, 2 * NV), dtype=torch.float32, device=dev)
    ab[:, :NV] = torch.from_numpy(c.alpha).to(dev)
    ab[:, NV:] = torch.from_numpy(c.beta).to(dev)
    gn = torch.from_numpy(c.gn).to(dev)
    out = torch.empty((B, NV * D), dtype=torch.float32, device=dev)
    q, k, v = qkv[:, :NK * D], qkv[:, NK * D:2 * NK * D], qkv[:, 2 * NK * D:]
    z, al, be = zrow[:, 8192:8192 + NV * D], ab[:, :NV], ab[:, NV:]

    def step(i):
        g.gdn_decode_norm(states[i % pools], q, k, v, al, be, z, gn, c.eps, out=out,
                          num_k_heads=NK, num_v_heads=NV)

    ms = _timed(step, calls, 5)
    algo = B * NV * head_bytes(D, NV, NK, 4, 4, True)
    del states, qkv, zrow, ab, out
    torch.cuda.empty_cache()
    return {"workload": "batched decode with fused norm on packed rows (q|k|v in [64,10240], z in "
                        "[64,16384]), B=64, NV=48, NK=16, D=128, padded pool",
            "ms_per_call": round(ms, 5),
            "state_GBps": round(2.0 * B * NV * D * D * 4 / ms / 1e6, 1),
            "hbm_frac_algorithmic": round(algo / ms / 1e6 / HBM_PEAK_GBS, 4)}


def run_fused(g, calls: int, pools: int = 16):
    """The decode workload with the input stage fused in front (4-tap conv ring,
    silu, L2 of q/k, gates): one launch per layer from the projection row, with
    the ring updated in place and with two alternating ring buffers."""
    import torch
    from gated_deltanet_decode_delta_amd import inputs

    B, NK, NV, D, taps = 64, 16, 48, 128, 4
    c = inputs.make_frontend_case(3200, B=B, NK=NK, NV=NV, D=D, taps=taps, pitch=983040)
    dev = "cuda:0"
    st0 = torch.from_numpy(c.state).to(dev)
    states = [st0.clone() for _ in range(pools)]
    del st0
    r0 = torch.from_numpy(c.ring).to(dev)
    rings = [[r0.clone(), r0.clone()] for _ in range(pools)]
    del r0
    t = {n: torch.from_numpy(getattr(c, n)).to(dev) for n in ("x", "w", "br", "ar", "dt", "rate", "z", "gn")}
    out = torch.empty((B, NV * D), device=dev)
    C = c.C
    algo = (2.0 * B * NV * D * D * 4                      # state read + write
            + B * (2 * taps - 1) * C * 4.0                # ring: taps-1 rows read, taps rows written
            + B * C * 4.0 + taps * C * 4.0                # x, conv weights
            + B * NV * (2 * 4 + 2 * D * 4) + NV * 8.0)    # br, ar, z, y; dt, rate
    res = {"workload": "decode with fused input stage (4-tap conv ring, silu, L2 q/k, gates) and "
                       "gated norm, B=64, NV=48, NK=16, D=128, padded pool",
           "algorithmic_bytes_per_launch": int(algo)}
    for mode in ("in_place", "two_buffers"):
        log(f"[bench] fused input stage ({mode}): B={B} pools={pools}")

        def step(i):
            p = i % pools
            pair = rings[p]
            src, dst = (pair[0], None) if mode == "in_place" else (pair[(i // pools) % 2],
                                                                    pair[(i // pools + 1) % 2])
            g.gdn_decode_fused(states[p], src, t["x"], t["w"], t["br"], t["ar"], t["dt"], t["rate"],
                               t["z"], t["gn"], 1e-6, 1e-6, out=out, conv_state_out=dst,
                               num_k_heads=NK, num_v_heads=NV)

        ms = _timed(step, calls, 5)
        res[mode] = {"ms_per_call": round(ms, 5),
                     "state_GBps": round(2.0 * B * NV * D * D * 4 / ms / 1e6, 1),
                     "hbm_frac_algorithmic": round(algo / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del states, rings, t, out
    torch.cuda.empty_cache()
    return res


def run_real_head(g, tokens: int):
    import torch
    from gated_deltanet_decode_delta_amd import inputs

    cfg = inputs.CONFIGS["real_head"]
    NK, NV, D, L = cfg["NK"], cfg["NV"], cfg["D"], cfg["layers"]
    dev = "cuda:0"
    log("[bench] real head: B=1, 48 layers")
    layers = []
    for l in range(L):
        c = inputs.real_head_layer(l)
        d = {n: torch.from_numpy(getattr(c, n)).to(dev) for n in ("q", "k", "v", "z", "alpha", "beta", "gn")}
        d["state"] = torch.from_numpy(c.state).to(dev)
        d["out"] = torch.empty((1, NV * D), device=dev)
        layers.append(d)

    def token(i):
        for d in layers:
            g.gdn_decode_norm(d["state"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["z"],
                              d["gn"], 1e-6, out=d["out"], num_k_heads=NK, num_v_heads=NV)

    # each figure: median of 5 trials of `tokens` tokens (48 calls each), warmup 10
    def median5(fn):
        return sorted(_timed(fn, tokens, 10) for _ in range(5))[2]

    ms = median5(token)
    # the same 48 calls marshalled once (static buffers, as in a serving loop)
    calls = [g.prepare(g.gdn_decode_norm, d["state"], d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                       d["z"], d["gn"], 1e-6, out=d["out"], num_k_heads=NK, num_v_heads=NV)
             for d in layers]

    def token_prepared(i):
        for call in calls:
            call()

    ms_prepared = median5(token_prepared)
    del calls
    graph_ms = None
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            token(0)
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            token(0)
        graph_ms = median5(lambda i: graph.replay())
    except Exception as e:  # capture is an optional measurement
        log(f"[bench] graph capture skipped: {e}")
    state_bytes = 2.0 * L * NV * D * D * 4
    del layers
    torch.cuda.empty_cache()
    res = {"workload": "real head B=1, 48 layer states per token, fused norm fp32",
           "trials": f"median of 5 trials x {tokens} tokens ({tokens * L} calls), warmup 10",
           "us_per_token": round(ms * 1e3, 2), "tokens_per_s": round(1e3 / ms, 1),
           "state_GBps": round(state_bytes / ms / 1e6, 1),
           "prepared_us_per_token": round(ms_prepared * 1e3, 2)}
    if graph_ms is not None:
        res.update({"graph_us_per_token": round(graph_ms * 1e3, 2),
                    "graph_state_GBps": round(state_bytes / graph_ms / 1e6, 1)})
    return res


def cpu_model() -> str:
    """The host CPU's model name, as /proc/cpuinfo gives it (empty if unknown)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(seconds: float):
    """The oracle on a bounded sample of the main workload: whole B=64 calls,
    (sequence, head) pairs fanned out over the host's threads (capped at 16)."""
    import oracle
    from gated_deltanet_decode_delta_amd import inputs

    c = inputs.config_case("batched")
    B, NK, NV, D = c.B, c.NK, c.NV, c.D
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    heads = [(b, h) for b in range(B) for h in range(NV)]
    st = c.state.copy()
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.seq_head_threaded(st, c.q, c.k, c.v, c.alpha, c.beta, B=B, T=1, NK=NK, NV=NV, Dk=D,
                                 Dv=D, z=c.z, gn=c.gn, eps=c.eps, heads=heads, threads=threads)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds or calls >= 200:
            break
    state_bytes = 2.0 * B * NV * D * D * 4 * calls
    # the same oracle on one thread, one whole call
    t1 = time.perf_counter()
    oracle.decode(st, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D, z=c.z,
                  gn=c.gn, eps=c.eps)
    el1 = time.perf_counter() - t1
    return {"value": round(state_bytes / el / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{calls} full B=64 gdn_decode_norm calls (3072 heads each) in {el:.1f} s "
                      f"on {threads} host threads; state GB/s by the same formula",
            "tokens_per_s_batch": round(B * calls / el, 1),
            "single_thread_GBps": round(2.0 * B * NV * D * D * 4 / el1 / 1e9, 3)}


def cpu_extras(seconds: float):
    """The oracle beside each extra workload, each on a bounded sample (about
    ``seconds`` of host time): binary16-state decode, the 4096-token sequence,
    the fused input stage and the two-token verify.  Rates use the same
    formulas as the GPU figures."""
    import oracle
    from gated_deltanet_decode_delta_amd import inputs

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    res = {}

    def repeat(fn):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds or n >= 100:
                return n, el

    # binary16 state: 16 of the 256 sequences (768 heads) per repetition
    c = inputs.config_case("fp16_state", B=16)
    st16 = oracle.f32_to_f16_bits(c.state)
    heads = [(b, h) for b in range(c.B) for h in range(c.NV)]
    n, el = repeat(lambda: oracle.seq_head_threaded(
        st16, c.q, c.k, c.v, c.alpha, c.beta, B=c.B, T=1, NK=c.NK, NV=c.NV, Dk=c.D, Dv=c.D, z=c.z,
        gn=c.gn, eps=c.eps, heads=heads, threads=threads, state_kind=oracle.STATE_F16))
    res["fp16_state"] = {"state_GBps": round(2.0 * len(heads) * c.D * c.D * 2 * n / el / 1e9, 3),
                         "cores": threads, "sample": f"{n} x 768 heads in {el:.1f} s"}
    # sequence: 2 x threads heads over all 4096 tokens
    c = inputs.config_case("sequence")
    heads = [(b, h) for b in range(c.B) for h in range(c.NV)][:2 * threads]
    st = c.state.copy()
    t0 = time.perf_counter()
    oracle.seq_head_threaded(st, c.q, c.k, c.v, c.alpha, c.beta, B=c.B, T=c.T, NK=c.NK, NV=c.NV,
                             Dk=c.D, Dv=c.D, heads=heads, threads=threads)
    el = time.perf_counter() - t0
    res["sequence"] = {"gflops": round(7.0 * c.D * c.D * c.T * len(heads) / el / 1e9, 3),
                       "cores": threads,
                       "sample": f"{len(heads)} heads x {c.T} tokens in {el:.1f} s"}
    # fused input stage: 2 sequences of the B=64 workload, one thread
    c = inputs.make_frontend_case(3200, B=2, NK=16, NV=48, D=128, taps=4)
    st, ring = c.state.copy(), c.ring.copy()
    n, el = repeat(lambda: oracle.fused_decode(st, ring, c.x, c.w, c.br, c.ar, c.dt, c.rate, B=2,
                                               NK=16, NV=48, D=128, taps=4, z=c.z, gn=c.gn))
    res["fused"] = {"state_GBps": round(2.0 * 2 * 48 * 128 * 128 * 4 * n / el / 1e9, 3), "cores": 1,
                    "sample": f"{n} x 2 sequences in {el:.1f} s"}
    # two-token verify: 4 sequences x 48 heads, threaded
    c = inputs.make_case(3102, B=4, NK=16, NV=48, D=128, T=2)
    heads = [(b, h) for b in range(c.B) for h in range(c.NV)]
    st = c.state.copy()
    n, el = repeat(lambda: oracle.seq_head_threaded(
        st, c.q, c.k, c.v, c.alpha, c.beta, B=c.B, T=2, NK=c.NK, NV=c.NV, Dk=c.D, Dv=c.D, z=c.z,
        gn=c.gn, eps=c.eps, heads=heads, threads=threads))
    res["verify"] = {"ms_per_call_B64_T2": round(el / n * 16 * 1e3, 2), "cores": threads,
                     "sample": f"{n} x 4 sequences (T=2) in {el:.1f} s, scaled to B=64"}
    return res


def pmc_traffic(algo_bytes: float):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel sources."""
    try:
        with open(PMC_FILE) as f:
            pmc = json.load(f)
    except (OSError, ValueError):
        return None
    if pmc.get("kernel_hash") != kernel_hash():
        return None
    return pmc.get("bytes_per_launch")


# rocprofv3 --pmc passes over one `--pmc-run` program (one pass per counter
# set: a pass holds few counters of each hardware block, and the derived
# counters need their own inputs)
PMC_PASSES = (
    ("fetch", "FETCH_SIZE"),
    ("write", "WRITE_SIZE"),
    ("insts", "SQ_INSTS_VALU SQ_WAVES SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT"),
    ("busy", "VALUBusy OccupancyPercent MfmaUtil"),
    ("l2", "TCC_HIT_sum TCC_MISS_sum"),
)
PMC_DETAIL_FILE = os.path.join(ROOT, "profiles", "kernel_counters.json")
PMC_TABLE_FILE = os.path.join(ROOT, "profiles", "kernel_counters.md")


def sources_hash() -> str:
    """Hash of every library source (the counters of any kernel are void once
    any of them changes)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_deltanet_decode_delta_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(code_text(f.read()))
    return h.hexdigest()[:16]


def calibrate_and_profile(g, steps: int):
    """The program the counter passes run: a plain device copy of a known size
    (to scale FETCH_SIZE / WRITE_SIZE), then `steps` calls of each profiled
    workload, in this order: the B=64 fused-norm decode (8 rotated pools), the
    B=64 raw decode (the same pools), the B=256 binary16 decode, draft verify at T=2 then T=4 (B=64), the decode with
    the fused input stage (two ring buffers, B=64) and the B=4, T=4096 sequence
    through both entry points (raw o)."""
    import torch
    from gated_deltanet_decode_delta_amd import inputs
    dev = "cuda:0"
    n = 1 << 28
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[pmc] copy kernel: {n * 4} bytes read, {n * 4} bytes written per dispatch")
    del a, b

    def load(c, names):
        return {x: torch.from_numpy(getattr(c, x)).to(dev) for x in names}

    c = inputs.config_case("batched")
    t = load(c, ("q", "k", "v", "z", "alpha", "beta", "gn"))
    st = [torch.from_numpy(c.state).to(dev) for _ in range(8)]
    out = torch.empty((c.B, c.NV * c.D), device=dev)
    log("[pmc] decode B=64")
    for i in range(steps):
        g.gdn_decode_norm(st[i % 8], t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["z"], t["gn"],
                          c.eps, out=out, num_k_heads=c.NK, num_v_heads=c.NV)
    torch.cuda.synchronize()
    log("[pmc] raw decode B=64")
    for i in range(steps):
        g.gdn_decode(st[i % 8], t["q"], t["k"], t["v"], t["alpha"], t["beta"], out=out,
                     num_k_heads=c.NK, num_v_heads=c.NV, head_dim=c.D)
    torch.cuda.synchronize()
    del st, t, out

    c = inputs.config_case("fp16_state")
    t = load(c, ("q", "k", "v", "z", "alpha", "beta", "gn"))
    st16 = g.gdn_state_f32_to_f16(torch.from_numpy(c.state).to(dev))
    out = torch.empty((c.B, c.NV * c.D), dtype=torch.bfloat16, device=dev)
    log("[pmc] binary16 decode B=256")
    for i in range(steps):
        g.gdn_decode_f16state(st16, t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["z"], t["gn"],
                              c.eps, out=out, num_k_heads=c.NK, num_v_heads=c.NV)
    torch.cuda.synchronize()
    del st16, t, out

    for T in (2, 4):
        c = inputs.make_case(3100 + T, B=64, NK=16, NV=48, D=128, T=T, pitch=983040)
        t = load(c, ("q", "k", "v", "z", "alpha", "beta", "gn"))
        st = [torch.from_numpy(c.state).to(dev) for _ in range(4)]
        inter = torch.empty((64 * (T - 1), 48 * 128 * 128), device=dev)
        out = torch.empty((64 * T, 48 * 128), device=dev)
        log(f"[pmc] verify B=64 T={T}")
        for i in range(steps):
            g.gdn_decode_verify(st[i % 4], t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["z"],
                                t["gn"], c.eps, out=out, inter_state=inter, num_tokens=T,
                                num_k_heads=16, num_v_heads=48)
        torch.cuda.synchronize()
        del st, t, inter, out

    c = inputs.make_frontend_case(3200, B=64, NK=16, NV=48, D=128, taps=4, pitch=983040)
    t = load(c, ("x", "w", "br", "ar", "dt", "rate", "z", "gn"))
    st = [torch.from_numpy(c.state).to(dev) for _ in range(4)]
    rings = [torch.from_numpy(c.ring).to(dev) for _ in range(2)]
    out = torch.empty((64, 48 * 128), device=dev)
    log("[pmc] fused input stage B=64, two ring buffers")
    for i in range(steps):
        g.gdn_decode_fused(st[i % 4], rings[i % 2], t["x"], t["w"], t["br"], t["ar"], t["dt"],
                           t["rate"], t["z"], t["gn"], 1e-6, 1e-6, out=out,
                           conv_state_out=rings[(i + 1) % 2], num_k_heads=16, num_v_heads=48)
    torch.cuda.synchronize()
    del st, rings, t, out

    c = inputs.config_case("sequence")
    t = load(c, ("q", "k", "v", "alpha", "beta"))
    st = torch.from_numpy(c.state).to(dev)
    out = torch.empty((c.B * c.T, c.NV * c.D), device=dev)
    ws = torch.empty(g.gdn_seq_workspace_bytes(c.B, c.T, c.NV, c.D), dtype=torch.uint8, device=dev)
    log("[pmc] sequence B=4 T=4096, with and without a workspace")
    for i in range(max(1, steps // 4)):
        g.gdn_recurrence_seq_ws(st, t["q"], t["k"], t["v"], t["alpha"], t["beta"], out=out,
                                workspace=ws, seq_len=c.T, num_k_heads=c.NK, num_v_heads=c.NV,
                                head_dim=c.D)
        g.gdn_recurrence_seq(st, t["q"], t["k"], t["v"], t["alpha"], t["beta"], out=out,
                             seq_len=c.T, num_k_heads=c.NK, num_v_heads=c.NV, head_dim=c.D)
    torch.cuda.synchronize()
    log("[pmc] done")


def _pmc_rows(root: str):
    """Every row of every rocprofv3 counter-collection csv under `root`."""
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _algorithmic(kernel: str, n_dispatch: int):
    """(label, algorithmic bytes per launch by dispatch index) of the profiled
    decode-shaped kernels, from the figures the bench uses; None otherwise."""
    hb = head_bytes
    if "decode_kernel<128, float, 1, 16, 1>" in kernel:
        return "fused-norm decode, B=64", lambda i: 64 * 48 * hb(128, 48, 16, 4, 4, True)
    if "decode_kernel<128, float, 0, 8, 2>" in kernel:
        return "raw decode, B=64, two workgroups per head", lambda i: 64 * 48 * hb(128, 48, 16, 4, 4, False)
    if "decode_kernelILi128EDF16_Li2ELi32" in kernel or "decode_kernel<128, _Float16, 2, 32>" in kernel:
        return "binary16 state, bf16 y, B=256", lambda i: 256 * 48 * hb(128, 48, 16, 2, 2, True)
    if "verify_kernel<128, true>" in kernel:
        T = 4 if kernel.endswith("[T=4]") else 2
        algo = 64 * (T + 1) * 48 * 128 * 128 * 4.0 + 64 * T * 48 * (hb(128, 48, 16, 4, 4, True)
                                                                  - 2 * 128 * 128 * 4)
        return f"draft verify, B=64, T={T}", lambda i: algo
    if "fused_split_kernel<128, true>" in kernel:
        C, taps = (2 * 16 + 48) * 128, 4
        algo = (2.0 * 64 * 48 * 128 * 128 * 4 + 64 * (2 * taps - 1) * C * 4.0 + 64 * C * 4.0
                + taps * C * 4.0 + 64 * 48 * (2 * 4 + 2 * 128 * 4) + 48 * 8.0)
        return "fused input stage, two ring buffers, B=64", lambda i: algo
    return None


def pmc_summarize(root: str):
    """Turn the counter passes of a --pmc-run (csv files under `root`, one
    subdirectory per pass) into the committed records: per kernel the mean of
    every counter per dispatch, HBM bytes scaled by what the counters read for
    the 1 GiB device copy, and for the decode-shaped kernels the ratio of those
    bytes to the algorithmic bytes.  Writes profiles/kernel_counters.json and
    .md, and the main decode's traffic record (profiles/decode_norm_b64_pmc.json)."""
    import statistics
    rows = _pmc_rows(root)
    per = {}   # kernel -> counter -> [values in dispatch order]
    for r in sorted(rows, key=lambda r: int(r.get("Dispatch_Id") or 0)):
        per.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
            float(r["Counter_Value"]))
    copy = "__amd_rocclr_copyBuffer"
    nbytes = float(1 << 30)
    ff = nbytes / (max(per[copy]["FETCH_SIZE"]) * 1024)
    wf = nbytes / (max(per[copy]["WRITE_SIZE"]) * 1024)
    out = {"sources_hash": sources_hash(), "kernel_hash": kernel_hash(),
           "calibration": {"kernel": copy + " (torch copy_ of a 1 GiB fp32 buffer)",
                           "fetch_factor": round(ff, 5), "write_factor": round(wf, 5)},
           "passes": [p for p in PMC_PASSES], "kernels": {}}
    entries = []
    for name, cs in per.items():
        if "gdn::" not in name and not name.startswith("_ZN3gdn"):
            continue
        if "verify_kernel<128, true>" in name:
            # the program ran T = 2 first, then as many calls at T = 4
            for tag, first in (("T=2", True), ("T=4", False)):
                entries.append((f"{name} [{tag}]", {c: (v[:len(v) // 2] if first else v[len(v) // 2:])
                                                    for c, v in cs.items()}))
        else:
            entries.append((name, cs))
    for name, cs in entries:
        rec = {c: statistics.mean(v) for c, v in cs.items()}
        rec["dispatches"] = max(len(v) for v in cs.values())
        if "FETCH_SIZE" in cs and "WRITE_SIZE" in cs:
            rec["hbm_bytes_per_launch"] = (rec["FETCH_SIZE"] * ff + rec["WRITE_SIZE"] * wf) * 1024
        if "SQ_INSTS_VALU" in cs and "SQ_WAVES" in cs:
            rec["valu_insts_per_wave"] = rec["SQ_INSTS_VALU"] / rec["SQ_WAVES"]
        if "TCC_HIT_sum" in cs and "TCC_MISS_sum" in cs:
            rec["l2_hit_pct"] = 100.0 * rec["TCC_HIT_sum"] / max(1.0, rec["TCC_HIT_sum"] + rec["TCC_MISS_sum"])
        alg = _algorithmic(name, len(cs.get("FETCH_SIZE", [])))
        if alg and "FETCH_SIZE" in cs and "WRITE_SIZE" in cs:
            label, fn = alg
            fe, wr = cs["FETCH_SIZE"], cs["WRITE_SIZE"]
            ratios = [((fe[i] * ff + wr[i] * wf) * 1024) / fn(i) for i in range(min(len(fe), len(wr)))]
            rec["workload"] = label
            rec["traffic_over_algorithmic"] = statistics.mean(ratios)
            rec["algorithmic_bytes_per_launch"] = [int(fn(0)), int(fn(len(fe) - 1))]
        out["kernels"][name] = rec
    with open(PMC_DETAIL_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")

    main = next(k for k in out["kernels"] if "decode_kernel<128, float, 1, 16, 1>" in k)
    m = out["kernels"][main]
    cfg = inputs_batched_algo()
    rec = {
        "kernel": main,
        "workload": "gdn_decode_norm, B=64, NV=48, NK=16, D=128, fp32 state, pitch 983040, fp32 out",
        "kernel_hash": kernel_hash(),
        "kernel_sources": list(KERNEL_SOURCES),
        "dispatches": m["dispatches"],
        "fetch_size_kib_per_dispatch": round(m["FETCH_SIZE"], 1),
        "write_size_kib_per_dispatch": round(m["WRITE_SIZE"], 1),
        "calibration": out["calibration"],
        "fetch_bytes_per_launch": int(m["FETCH_SIZE"] * 1024 * ff),
        "write_bytes_per_launch": int(m["WRITE_SIZE"] * 1024 * wf),
        "bytes_per_launch": int(m["hbm_bytes_per_launch"]),
        "algorithmic_bytes_per_launch": int(cfg),
        "commands": pmc_commands(),
    }
    with open(PMC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")

    def fmt(x, nd=1):
        return "" if x is None else (f"{x:,.{nd}f}" if isinstance(x, float) else f"{x:,}")

    lines = ["# Counters per kernel -- decode-shaped kernels and the sequence passes", "",
             "Every figure is the mean per dispatch of a rocprofv3 `--pmc` pass over "
             "`bench.py --pmc-run` (the workloads and their order are in `calibrate_and_profile`); "
             "HBM bytes are FETCH_SIZE and WRITE_SIZE scaled by what the same counters read for a "
             f"1 GiB device copy (factors {ff:.5f} and {wf:.5f}).", "",
             f"Library sources hash `{out['sources_hash']}`.", "", "Commands (repo at `<repo>`, "
             "output under `<out>`):", "", "```"] + pmc_commands() + ["```", "",
             "| Kernel | Workload | Dispatches | HBM bytes / launch | / algorithmic | VALU insts / wave "
             "| VALUBusy % | Occupancy % | MfmaUtil % | L2 hit % | LDS bank conflicts / LDS insts |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for name, r in sorted(out["kernels"].items()):
        conf = (r["SQ_LDS_BANK_CONFLICT"] / r["SQ_INSTS_LDS"]) if r.get("SQ_INSTS_LDS") else None
        lines.append("| `{}` | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} |".format(
            name.replace("void ", "").replace("(gdn::StepArgs)", ""), r.get("workload", ""),
            r["dispatches"], fmt(r.get("hbm_bytes_per_launch"), 0),
            fmt(r.get("traffic_over_algorithmic"), 4), fmt(r.get("valu_insts_per_wave")),
            fmt(r.get("VALUBusy")), fmt(r.get("OccupancyPercent")), fmt(r.get("MfmaUtil")),
            fmt(r.get("l2_hit_pct")), fmt(conf, 3)))
    with open(PMC_TABLE_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"kernels": len(out["kernels"]), "main_bytes_per_launch": rec["bytes_per_launch"],
                      "main_algorithmic": rec["algorithmic_bytes_per_launch"]}))


def inputs_batched_algo() -> float:
    from gated_deltanet_decode_delta_amd import inputs
    cfg = inputs.CONFIGS["batched"]
    return cfg["B"] * cfg["NV"] * head_bytes(cfg["D"], cfg["NV"], cfg["NK"], 4, 4, True)


def pmc_commands():
    cmds = [f"cd /tmp && TMPDIR=/tmp timeout -s KILL 300 rocprofv3 --pmc {ctr} -d <out>/{name} -o {name} "
            f"--output-format csv -- python3 <repo>/bench.py --pmc-run --steps 12"
            for name, ctr in PMC_PASSES]
    return cmds + ["python3 <repo>/bench.py --pmc-summarize <out>"]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--pools", type=int, default=48)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-extra", action="store_true", help="main workload only")
    ap.add_argument("--extras", default="raw,fp16_state,sequence,verify,norm_q,strided,fused,real_head",
                    help="comma list of extra workloads: raw, fp16_state, sequence, verify, norm_q, "
                         "strided, fused, real_head; also batches (the fused-norm decode at other "
                         "batch sizes, not in the default run, so that a kernel trace of the default "
                         "run keeps one shape per decode kernel)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--seq-only", action="store_true", help="time the sequence workload alone")
    ap.add_argument("--pmc-summarize", metavar="DIR",
                    help="write the counter records from the rocprofv3 --pmc passes under DIR (no GPU)")
    ap.add_argument("--pmc-run", action="store_true",
                    help="copy-kernel calibration + the profiled workloads (for rocprofv3 --pmc)")
    args = ap.parse_args()

    if args.pmc_summarize:
        pmc_summarize(args.pmc_summarize)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_decode_delta_amd as g

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    g.lib()
    if args.pmc_run:
        calibrate_and_profile(g, args.steps)
        return
    if args.seq_only:
        print(json.dumps(run_seq(g, 100)), flush=True)
        return

    m = run_main(g, args.steps, args.warmup, args.pools)
    ms = m["ms"]
    B = m["B"]
    value = m["state_bytes"] / ms / 1e6
    achieved = m["algo_bytes"] / ms / 1e6
    extra = {"cache_resident_single_pool": {
        "ms_per_call": round(m["ms_hot"], 5),
        "state_GBps": round(m["state_bytes"] / m["ms_hot"] / 1e6, 1),
        "note": "same pool every call: the 201 MB state can stay in the 256 MB Infinity Cache"},
        "trials_5x200": {"median_ms": round(m["trials"][2], 5), "min_ms": round(m["trials"][0], 5),
                         "median_hbm_frac_algorithmic": round(
                             m["algo_bytes"] / m["trials"][2] / 1e6 / HBM_PEAK_GBS, 4)}}
    wanted = [] if args.no_extra else [w for w in args.extras.split(",") if w]
    runners = {"raw": lambda: run_raw(g), "fp16_state": lambda: run_fp16(g, 100),
               "batches": lambda: run_batches(g), "sequence": lambda: run_seq(g, 100),
               "verify": lambda: run_verify(g, 100), "norm_q": lambda: run_norm_q(g, 200),
               "strided": lambda: run_strided(g, 200), "fused": lambda: run_fused(g, 200),
               "real_head": lambda: run_real_head(g, 100)}
    for w in wanted:
        extra[w] = runners[w]()
    cpu = None if args.no_cpu else cpu_baseline(args.cpu_seconds)
    if not args.no_cpu and wanted:
        for name, rate in cpu_extras(args.cpu_seconds / 5).items():
            if name in extra:
                extra[name]["cpu_oracle"] = rate
    line = {
        "metric": "GDN decode state GB/s and % HBM roofline; tokens/s·batch at HV=48,D=128",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "batched decode with fused gated RMSNorm: B=64, NV=48, NK=16, "
                               "D=128, fp32 state pitch 1.25x slot, fp32 out, "
                               f"{m['pools']} state pools in rotation",
                   "global_batch": B, "seq_len": 1, "parallelism": "single GPU"},
        "tokens_per_s_batch": round(B / ms * 1e3, 1),
        # the same rate per model token: one token of each sequence steps all 48
        # GDN layer states of the model, one call per layer
        "model_tokens_per_s_48_layers": round(B / (48 * ms) * 1e3, 1),
        "hbm_frac_state": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": pmc_traffic(m["algo_bytes"]),
                     "kernel": "gdn::decode_kernel<128, float, kOutNormF32, 16, 1>",
                     "algorithmic_bytes_per_launch": int(m["algo_bytes"])},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    if m["nonfinite"]:
        line["warning"] = "non-finite outputs"
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
