"""The C ABI without a GPU: libgdn.so loads, exports every function that
include/gdn.h declares, and its host-side validation returns the documented
status codes.  Only calls that validation rejects are made here (they return
before any HIP call), plus empty calls, which the contract makes no-ops; the
pointers are fake addresses that are never dereferenced."""
import ctypes
import json
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def lib():
    import gated_deltanet_decode_delta_amd as gdn
    if not os.path.exists(gdn.LIB_PATH):
        from gated_deltanet_decode_delta_amd import _build
        _build.build()
    return gdn.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(gdn_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def test_header_declarations_found():
    names = _declared()
    assert "gdn_decode" in names and "gdn_decode_verify" in names
    assert len(names) == 14, names


def test_every_declared_symbol_is_exported(lib):
    import gated_deltanet_decode_delta_amd as gdn
    names = _declared()
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n), n
    assert sorted(gdn.EXPORTS) == names       # the binding wraps exactly these


def test_status_strings(lib):
    for code in range(10):
        assert lib.gdn_status_string(code)
        assert b"unknown" not in lib.gdn_status_string(code).lower()
    assert b"unknown" in lib.gdn_status_string(99).lower()


# fake, suitably aligned device addresses (never dereferenced)
A = 1 << 32
NK, NV, D, B = 2, 4, 16, 2
SLOT = NV * D * D


def _bases():
    step = 1 << 24
    names = ["state", "q", "k", "v", "alpha", "beta", "z", "gn", "out", "inter"]
    return {n: A + i * step for i, n in enumerate(names)}


def decode(lib, **kw):
    p = _bases()
    a = dict(state=p["state"], pitch=SLOT, q=p["q"], k=p["k"], qk=NK * D, v=p["v"], vs=NV * D,
             al=p["alpha"], be=p["beta"], ab=NV, out=p["out"], os=NV * D, B=B, nk=NK, nv=NV,
             dk=D, dv=D)
    a.update(kw)
    return lib.gdn_decode(a["state"], a["pitch"], a["q"], a["k"], a["qk"], a["v"], a["vs"],
                          a["al"], a["be"], a["ab"], a["out"], a["os"], a["B"], a["nk"], a["nv"],
                          a["dk"], a["dv"], None)


def norm(lib, **kw):
    p = _bases()
    a = dict(state=p["state"], pitch=SLOT, q=p["q"], k=p["k"], qk=NK * D, v=p["v"], vs=NV * D,
             al=p["alpha"], be=p["beta"], ab=NV, z=p["z"], zs=NV * D, gn=p["gn"], eps=1e-6,
             out=p["out"], dt=0, os=NV * D, B=B, nk=NK, nv=NV, dk=D, dv=D)
    a.update(kw)
    return lib.gdn_decode_norm(a["state"], a["pitch"], a["q"], a["k"], a["qk"], a["v"], a["vs"],
                               a["al"], a["be"], a["ab"], a["z"], a["zs"], a["gn"], a["eps"],
                               a["out"], a["dt"], a["os"], a["B"], a["nk"], a["nv"], a["dk"],
                               a["dv"], None)


def seq(lib, **kw):
    p = _bases()
    a = dict(state=p["state"], pitch=SLOT, q=p["q"], k=p["k"], qk=NK * D, v=p["v"], vs=NV * D,
             al=p["alpha"], be=p["beta"], ab=NV, z=None, zs=0, gn=None, eps=1e-6,
             out=p["out"], os=NV * D, B=B, T=5, nk=NK, nv=NV, dk=D, dv=D)
    a.update(kw)
    return lib.gdn_recurrence_seq(a["state"], a["pitch"], a["q"], a["k"], a["qk"], a["v"],
                                  a["vs"], a["al"], a["be"], a["ab"], a["z"], a["zs"], a["gn"],
                                  a["eps"], a["out"], a["os"], a["B"], a["T"], a["nk"], a["nv"],
                                  a["dk"], a["dv"], None)


def verify(lib, **kw):
    p = _bases()
    a = dict(state=p["state"], pitch=SLOT, inter=p["inter"], ip=SLOT, q=p["q"], k=p["k"],
             qk=NK * D, v=p["v"], vs=NV * D, al=p["alpha"], be=p["beta"], ab=NV, z=None, zs=0,
             gn=None, eps=1e-6, out=p["out"], os=NV * D, B=B, T=3, nk=NK, nv=NV, dk=D, dv=D)
    a.update(kw)
    return lib.gdn_decode_verify(a["state"], a["pitch"], a["inter"], a["ip"], a["q"], a["k"],
                                 a["qk"], a["v"], a["vs"], a["al"], a["be"], a["ab"], a["z"],
                                 a["zs"], a["gn"], a["eps"], a["out"], a["os"], a["B"], a["T"],
                                 a["nk"], a["nv"], a["dk"], a["dv"], None)


def test_decode_validation(lib):
    p = _bases()
    assert decode(lib, dk=12, dv=12) == 4          # not a power of two
    assert decode(lib, dk=512, dv=512) == 4        # above 256
    assert decode(lib, dk=16, dv=32) == 4          # Dk != Dv
    assert decode(lib, nv=3) == 2                  # NV % NK
    assert decode(lib, nk=0) == 2
    assert decode(lib, B=-1) == 2
    assert decode(lib, q=None) == 1
    assert decode(lib, state=None) == 1
    assert decode(lib, pitch=SLOT - 4) == 3        # slot pitch shorter than a slot
    assert decode(lib, qk=NK * D - 4) == 3
    assert decode(lib, q=p["q"] + 4) == 3          # 16-byte alignment
    assert decode(lib, qk=NK * D + 2) == 3         # row stride not a multiple of 4
    assert decode(lib, al=p["alpha"] + 2) == 3
    assert decode(lib, out=p["state"] + 64) == 5   # output inside the state
    assert decode(lib, out=p["v"]) == 5            # output over an input
    assert decode(lib, q=p["state"] + 4096) == 5   # state over an input
    assert decode(lib, B=0) == 0                   # empty: no launch, OK
    assert decode(lib, B=0, q=None) == 0


def test_norm_validation(lib):
    assert norm(lib, eps=-1.0) == 8
    assert norm(lib, eps=float("nan")) == 8
    assert norm(lib, eps=float("inf")) == 8
    assert norm(lib, dt=7) == 6
    assert norm(lib, z=None) == 1
    assert norm(lib, gn=None) == 1
    assert norm(lib, zs=NV * D - 4) == 3
    p = _bases()
    assert norm(lib, out=p["z"]) == 5
    assert norm(lib, B=0) == 0


def test_seq_validation(lib):
    assert seq(lib, T=-1) == 2
    assert seq(lib, T=0) == 0
    assert seq(lib, vs=NV * D - 4) == 3
    p = _bases()
    assert seq(lib, out=p["q"]) == 5


def seq_ws(lib, **kw):
    """gdn_recurrence_seq_ws at D = 128 (the shape that uses the workspace)."""
    p = _bases()
    d, slot = 128, NV * 128 * 128
    need = B * NV * 1 * 2304
    a = dict(state=p["state"], pitch=slot, q=p["q"], k=p["k"], qk=NK * d, v=p["v"], vs=NV * d,
             al=p["alpha"], be=p["beta"], ab=NV, z=None, zs=0, gn=None, eps=1e-6,
             out=p["out"], os=NV * d, B=B, T=5, nk=NK, nv=NV, dk=d, dv=d,
             ws=A + 10 * (1 << 24), wsb=need)
    a.update(kw)
    return lib.gdn_recurrence_seq_ws(a["state"], a["pitch"], a["q"], a["k"], a["qk"], a["v"],
                                     a["vs"], a["al"], a["be"], a["ab"], a["z"], a["zs"],
                                     a["gn"], a["eps"], a["out"], a["os"], a["B"], a["T"],
                                     a["nk"], a["nv"], a["dk"], a["dv"], a["ws"], a["wsb"], None)


def test_seq_workspace_bytes(lib):
    assert lib.gdn_seq_workspace_bytes(4, 4096, 48, 128, 128) == 4 * 48 * 256 * 2304
    assert lib.gdn_seq_workspace_bytes(2, 16, 4, 128, 128) == 2 * 4 * 1 * 2304
    assert lib.gdn_seq_workspace_bytes(2, 17, 4, 128, 128) == 2 * 4 * 2 * 2304
    assert lib.gdn_seq_workspace_bytes(2, 0, 4, 128, 128) == 0
    assert lib.gdn_seq_workspace_bytes(2, 17, 4, 64, 64) == 0      # no workspace used
    assert lib.gdn_seq_workspace_bytes(-1, 5, 4, 128, 128) == -1


def test_seq_ws_validation(lib):
    p = _bases()
    need = B * NV * 2304
    assert seq_ws(lib, ws=None) == 1                      # needed at D = 128, raw output
    assert seq_ws(lib, wsb=need - 4) == 8                 # smaller than gdn_seq_workspace_bytes
    assert seq_ws(lib, ws=A + 10 * (1 << 24) + 4) == 3    # not 16-byte aligned
    assert seq_ws(lib, ws=p["state"] + 64) == 5           # inside the state
    assert seq_ws(lib, ws=p["q"]) == 5                    # over an input
    assert seq_ws(lib, ws=p["out"] + 16) == 5             # over the output
    assert seq_ws(lib, T=-1) == 2
    assert seq_ws(lib, T=0, ws=None) == 0                 # empty: no launch, OK
    assert seq_ws(lib, vs=NV * 128 - 4) == 3              # the plain call's checks come first
    assert seq_ws(lib, out=p["q"], ws=None) == 5


def noalloc(lib, **kw):
    """gdn_recurrence_seq_noalloc at D = 128 on fake bases 64 GiB apart, so that
    long sequences fit between them."""
    step, base = 1 << 36, 1 << 40
    p = {n: base + i * step for i, n in enumerate(["state", "q", "k", "v", "alpha", "beta", "out"])}
    d = 128
    a = dict(state=p["state"], pitch=NV * d * d, q=p["q"], k=p["k"], qk=NK * d, v=p["v"],
             vs=NV * d, al=p["alpha"], be=p["beta"], ab=NV, z=None, zs=0, gn=None, eps=1e-6,
             out=p["out"], os=NV * d, B=1, T=5, nk=NK, nv=NV, dk=d, dv=d)
    a.update(kw)
    return lib.gdn_recurrence_seq_noalloc(a["state"], a["pitch"], a["q"], a["k"], a["qk"], a["v"],
                                          a["vs"], a["al"], a["be"], a["ab"], a["z"], a["zs"],
                                          a["gn"], a["eps"], a["out"], a["os"], a["B"], a["T"],
                                          a["nk"], a["nv"], a["dk"], a["dv"], None)


def test_noalloc_validation(lib):
    import gated_deltanet_decode_delta_amd as gdn
    limit = gdn.SEQ_NOALLOC_MAX_BYTES
    assert limit == 64 << 20
    # the largest length whose records fit, and the first that does not
    chunks = limit // (NV * 2304)
    assert lib.gdn_seq_workspace_bytes(1, 16 * chunks, NV, 128, 128) <= limit
    assert lib.gdn_seq_workspace_bytes(1, 16 * chunks + 1, NV, 128, 128) > limit
    assert noalloc(lib, T=16 * chunks + 1) == 9          # GDN_ERR_SCRATCH, nothing launched
    assert noalloc(lib, B=3, T=16 * chunks) == 9
    assert noalloc(lib, T=-1) == 2                       # the plain call's checks come first
    assert noalloc(lib, T=0) == 0                        # empty: no launch, OK
    assert noalloc(lib, vs=NV * 128 - 4, T=100) == 3
    assert noalloc(lib, q=None) == 1
    assert noalloc(lib, out=(1 << 40) + (1 << 36) + 64) == 5   # output over q
    assert noalloc(lib, dk=96, dv=96) == 4


def test_verify_validation(lib):
    p = _bases()
    assert verify(lib, T=0) == 2
    assert verify(lib, T=9) == 2
    assert verify(lib, inter=None) == 1             # needed when T > 1
    assert verify(lib, ip=SLOT - 4) == 3            # rollback slots overlap
    assert verify(lib, ip=SLOT + 2) == 3            # pitch not a multiple of 4
    assert verify(lib, inter=p["inter"] + 8) == 3   # misaligned
    assert verify(lib, inter=p["state"]) == 5       # over the state
    assert verify(lib, inter=p["out"] - 4 * SLOT) == 5   # tail runs into the output
    assert verify(lib, inter=p["v"]) == 5           # over an input
    assert verify(lib, z=p["z"], gn=None) == 1
    assert verify(lib, B=0) == 0
    assert verify(lib, B=0, T=9) == 2               # the token bound comes first


def normq(lib, **kw):
    p = _bases()
    a = dict(state=p["state"], pitch=SLOT, q=p["q"], k=p["k"], qk=NK * D, v=p["v"], vs=NV * D,
             al=p["alpha"], be=p["beta"], ab=NV, z=p["z"], zs=NV * D, gn=p["gn"], eps=1e-6,
             out=p["out"], os=NV * D, codes=p["inter"], cs=NV * D, scales=p["inter"] + (1 << 20),
             ss=NV * D // 32, B=B, nk=NK, nv=NV, dk=D, dv=D)
    a.update(kw)
    return lib.gdn_decode_norm_q(a["state"], a["pitch"], a["q"], a["k"], a["qk"], a["v"], a["vs"],
                                 a["al"], a["be"], a["ab"], a["z"], a["zs"], a["gn"], a["eps"],
                                 a["out"], a["os"], a["codes"], a["cs"], a["scales"], a["ss"],
                                 a["B"], a["nk"], a["nv"], a["dk"], a["dv"], None)


def test_norm_q_validation(lib):
    p = _bases()
    assert normq(lib) == 4                               # D = 16: not a multiple of 32
    big = dict(dk=32, dv=32, pitch=NV * 32 * 32, vs=NV * 32, zs=NV * 32, os=NV * 32,
               cs=NV * 32, ss=NV, qk=NK * 32)
    assert normq(lib, codes=None, **big) == 1
    assert normq(lib, scales=None, **big) == 1
    assert normq(lib, **dict(big, cs=NV * 32 - 1)) == 3  # codes rows too short
    assert normq(lib, **dict(big, ss=NV - 1)) == 3
    assert normq(lib, scales=p["inter"] + (1 << 20) + 2, **big) == 3   # scales misaligned
    assert normq(lib, scales=p["inter"] + 64, **big) == 5              # scales inside codes
    assert normq(lib, codes=p["state"] + 16, **big) == 5               # codes over the state
    assert normq(lib, codes=p["out"], **big) == 5                      # codes over y
    assert normq(lib, scales=p["q"], **big) == 5                       # scales over an input
    assert normq(lib, out=None, z=None, **big) == 1                    # z is required
    assert normq(lib, B=0, **big) == 0


def fused(lib, **kw):
    p = _bases()
    C = (2 * NK + NV) * D
    a = dict(state=p["state"], pitch=SLOT, ring=p["inter"], rs=4 * C, x=p["q"], xs=C, w=p["k"],
             taps=4, br=p["alpha"], ar=p["beta"], gs=NV, dt=p["gn"], rate=p["gn"] + 4096,
             l2=1e-6, z=None, zs=0, gn=None, eps=1e-6, out=p["out"], os=NV * D, B=B, nk=NK, nv=NV,
             dk=D, dv=D)
    a.update(kw)
    return lib.gdn_decode_fused(a["state"], a["pitch"], a["ring"], a["rs"], a.get("rout"), a["x"],
                                a["xs"], a["w"],
                                a["taps"], a["br"], a["ar"], a["gs"], a["dt"], a["rate"], a["l2"],
                                a["z"], a["zs"], a["gn"], a["eps"], a["out"], a["os"], a["B"],
                                a["nk"], a["nv"], a["dk"], a["dv"], None)


def test_fused_validation(lib):
    p = _bases()
    C = (2 * NK + NV) * D
    assert fused(lib, taps=0) == 2
    assert fused(lib, taps=9) == 2
    assert fused(lib, nv=3) == 2
    assert fused(lib, dk=12, dv=12) == 4
    assert fused(lib, nk=1, nv=64, dk=256, dv=256) == 4     # LDS features above 64 KiB
    assert fused(lib, l2=-1.0) == 8
    assert fused(lib, l2=float("nan")) == 8
    assert fused(lib, ring=None) == 1
    assert fused(lib, rate=None) == 1
    assert fused(lib, z=p["z"]) == 1                         # z without norm weight
    assert fused(lib, rs=4 * C - 4) == 3                     # ring slots overlap
    assert fused(lib, xs=C - 4) == 3
    assert fused(lib, ring=p["inter"] + 8) == 3              # misaligned ring
    assert fused(lib, w=p["k"] + 4) == 3
    assert fused(lib, ring=p["state"] + 64) == 5             # ring inside the state
    assert fused(lib, out=p["q"] + 16) == 5                  # output over x
    assert fused(lib, ring=p["k"] - 16) == 5                 # ring runs into the weights
    assert fused(lib, rout=p["inter"] + 64) == 5             # new ring over the old one
    assert fused(lib, rout=p["out"]) == 5                    # new ring over the output
    assert fused(lib, rout=p["inter"] + (1 << 20) + 4) == 3  # misaligned new ring
    assert fused(lib, nk=1, nv=64, dk=256, dv=256, rout=p["inter"] + (1 << 20)) != 4
    assert fused(lib, B=0) == 0
    # 2^26 sequences x 64 value heads is past a 32-bit grid, though x 1 key head is not
    assert fused(lib, B=1 << 26, nk=1, nv=64, rout=p["inter"] + (1 << 20)) == 2


def test_converter_validation(lib):
    p = _bases()
    assert lib.gdn_state_f32_to_f16(p["state"], p["state"] + 16, 64, None) == 5
    assert lib.gdn_state_f32_to_f16(None, p["out"], 64, None) == 1
    assert lib.gdn_state_f16_to_f32(p["state"], p["out"], -1, None) == 2
    assert lib.gdn_state_f16_to_f32(p["state"], p["out"], 0, None) == 0


_ONE_RUNTIME = r"""
import json, sys
sys.path.insert(0, {root!r})
import gated_deltanet_decode_delta_amd as gdn
gdn.lib()                      # the library first, torch only afterwards
import torch
maps = open("/proc/self/maps").read().split("\n")
print(json.dumps(sorted({{ln.split()[-1] for ln in maps if "libamdhip64" in ln}})))
"""


def test_one_hip_runtime_whatever_the_import_order(lib):
    """torch ships its own HIP runtime under ROCm's soname.  Loading libgdn.so
    through the binding before torch must still leave a single runtime mapped
    (regression: the library bound to ROCm's copy, torch then loaded its own,
    and every launch of the library failed with hipErrorNoDevice)."""
    res = subprocess.run(["python3", "-c", _ONE_RUNTIME.format(root=ROOT)],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr
    paths = json.loads(res.stdout.strip().splitlines()[-1])
    assert len(paths) == 1, paths
