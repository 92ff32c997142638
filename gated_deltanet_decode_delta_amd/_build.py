"""Build ``libgdn.so`` in-tree with hipcc for gfx950.

Each ``csrc/*.hip`` file compiles to an object in ``_build/`` in parallel, then
one link makes ``libgdn.so`` next to this file.  Packed FP32 instructions are
disabled for every device pass (``-packed-fp32-ops``); hipcc's host pass warns
that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgdn.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]


# Per-source extra flags.  The split and grouped sequence kernels keep their matrix-core
# accumulators in ordinary VGPRs: left to itself the compiler puts them in
# AGPRs and copies every one back for the vector-ALU work on it.
EXTRA = {"gdn_seq_split.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "gdn_seq_group.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in res.stderr.splitlines()
                     if "packed-fp32-ops" not in line and line.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    if errs:
        sys.stderr.write(errs + "\n")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link ``libgdn.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


DEMO_SRC = os.path.join(os.path.dirname(HERE), "tests", "c", "gdn_c_demo.c")
DEMO = DEMO_SRC[:-2]


def build_c_demo() -> str:
    """Compile the plain-C program that drives ``libgdn.so`` through ``gdn.h``
    alone (hipMalloc buffers, no Python); it finds the library next to this
    file and the HIP runtime under /opt/rocm by its run path."""
    cc = os.environ.get("CC", "gcc")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE,
           "-I", "/opt/rocm/include", DEMO_SRC, "-o", DEMO + ".tmp", "-L", HERE, "-lgdn",
           "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../gated_deltanet_decode_delta_amd", "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"{cc} failed on {DEMO_SRC}:\n{res.stderr}")
    os.replace(DEMO + ".tmp", DEMO)
    return DEMO


if __name__ == "__main__":
    print(build(verbose=True))
