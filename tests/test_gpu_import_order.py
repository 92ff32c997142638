"""The library loaded before torch on a GPU: one decode step in a fresh process
whose first import is the binding, checked against the oracle.  torch carries
its own HIP runtime under ROCm's soname; the binding loads torch first so that
libgdn.so binds to that runtime (regression: loaded the other way round the
process held two runtimes and the step failed with hipErrorNoDevice)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import gated_deltanet_decode_delta_amd as gdn
gdn.lib()
import numpy as np
import torch
import oracle as orc
from gated_deltanet_decode_delta_amd import inputs
B, NK, NV, D = 2, 2, 6, 128
c = inputs.make_case(2100, B=B, NK=NK, NV=NV, D=D, T=1)
st = torch.from_numpy(c.state).to("cuda:0")
t = {{n: torch.from_numpy(getattr(c, n)).to("cuda:0") for n in ("q", "k", "v", "alpha", "beta")}}
out = gdn.gdn_decode(st, t["q"], t["k"], t["v"], t["alpha"], t["beta"], num_k_heads=NK,
                     num_v_heads=NV, head_dim=D)
torch.cuda.synchronize()
ref_st = c.state.copy()
ref = orc.decode(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D)
g = out.cpu().numpy().astype(np.float64).reshape(-1, D)
r = np.asarray(ref, np.float64).reshape(-1, D)
err = float((np.abs(g - r).max(axis=1) / np.abs(r).max(axis=1)).max())
gs = st.cpu().numpy().astype(np.float64).reshape(-1, D * D)
rs = np.asarray(ref_st, np.float64).reshape(-1, D * D)
serr = float((np.abs(gs - rs).max(axis=1) / np.abs(rs).max(axis=1)).max())
print("ERR", err, serr, flush=True)
"""


def test_decode_with_library_loaded_before_torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[case] decode in a child process, library loaded before torch", file=sys.stderr,
          flush=True)
    code = _CHILD.format(root=ROOT)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=240)
    assert res.returncode == 0, res.stderr[-2000:]
    line = [ln for ln in res.stdout.splitlines() if ln.startswith("ERR")][-1]
    err, serr = map(float, line.split()[1:])
    assert err < 1e-5 and serr < 1e-5, (err, serr)


def test_launch_status_ignores_an_earlier_failed_call():
    """A failed HIP call of the caller stays recorded in the thread until it is
    read.  The library must judge each launch by that launch's own status, not
    by the thread's last error: with a failed hipSetDevice before it, a decode
    step still returns GDN_OK and the right values."""
    import ctypes

    import numpy as np
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle as orc
    import gated_deltanet_decode_delta_amd as gdn
    from gated_deltanet_decode_delta_amd import inputs
    gdn.lib()
    hip = ctypes.CDLL("libamdhip64.so.7")     # the runtime already loaded (torch's)
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    hip.hipGetLastError.restype = ctypes.c_int
    B, NK, NV, D = 2, 2, 6, 128
    c = inputs.make_case(2200, B=B, NK=NK, NV=NV, D=D, T=1)
    st = torch.from_numpy(c.state).to("cuda:0")
    t = {n: torch.from_numpy(getattr(c, n)).to("cuda:0") for n in ("q", "k", "v", "alpha", "beta")}
    torch.cuda.synchronize()
    print("[case] decode after a failed hipSetDevice", file=sys.stderr, flush=True)
    assert hip.hipSetDevice(1 << 20) != 0
    try:
        out = gdn.gdn_decode(st, t["q"], t["k"], t["v"], t["alpha"], t["beta"], num_k_heads=NK,
                             num_v_heads=NV, head_dim=D)
    finally:
        hip.hipGetLastError()                 # leave no recorded error behind
    torch.cuda.synchronize()
    ref_st = c.state.copy()
    ref = orc.decode(ref_st, c.q, c.k, c.v, c.alpha, c.beta, B=B, NK=NK, NV=NV, Dk=D, Dv=D)
    g = out.cpu().numpy().astype(np.float64).reshape(-1, D)
    r = np.asarray(ref, np.float64).reshape(-1, D)
    assert float((np.abs(g - r).max(axis=1) / np.abs(r).max(axis=1)).max()) < 1e-5
