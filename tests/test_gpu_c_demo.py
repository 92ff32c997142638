"""The C ABI from a plain C program (``tests/c/gdn_c_demo.c``): hipMalloc
buffers, ``gdn_decode`` and ``gdn_decode_norm`` through ``gdn.h``, no Python or
torch in the process.  Its printed results must match the hand-derived D = 4
worked example (``tests/golden/d4_worked_example.json``, step a, with its
citation): o and the state's key column 0 exactly (every value is a small
binary fraction), y to fp32 rounding; and the two malformed calls must come
back as the right validation codes.
"""
import json
import os
import subprocess

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "tests", "c", "gdn_c_demo")
GOLDEN = os.path.join(ROOT, "tests", "golden", "d4_worked_example.json")


def test_c_program_reproduces_the_worked_example():
    if not os.path.exists(DEMO):
        raise RuntimeError(f"{DEMO} is not built; run __graft_entry__.build() first")
    a = json.load(open(GOLDEN))["step_a"]
    n = a["norm"]
    args = [*a["k"], *a["q"], *a["v"], a["alpha"], a["beta"], *n["gn"], *n["z"], n["eps"]]
    print("[case] C program, D=4 worked example step a", flush=True)
    res = subprocess.run([DEMO, *(repr(float(x)) for x in args)], capture_output=True, text=True,
                         timeout=60)
    assert res.returncode == 0, res.stderr
    got = {}
    for line in res.stdout.splitlines():
        key, _, rest = line.partition(":")
        got[key] = rest.split()
    o = np.array(got["o"], np.float64)
    col0 = np.array(got["state_col0"], np.float64)
    y = np.array(got["y"], np.float64)
    assert np.array_equal(o, np.array(a["o"])), o
    assert np.array_equal(col0, np.array(a["S1_column0"])), col0
    ref_y = np.array(n["y"])
    assert np.all(np.abs(y - ref_y) <= 1e-6 * np.abs(ref_y).max()), y
    assert got["status_shape"][0] == "GDN_ERR_SHAPE:"
    assert got["status_align"][0] == "GDN_ERR_STRIDE:"
