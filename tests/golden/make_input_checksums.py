"""Write ``input_checksums.json``: sha256 of every array the seeded input
generator draws for the benchmark workloads.

The generator (``gated_deltanet_decode_delta_amd/inputs.py``) draws from
numpy's PCG64 stream; these digests pin that stream, so that a change in numpy's
generators or in the draw order shows up as a failing CPU test instead of as
silently different workloads.  The script calls the input generator only.

    python tests/golden/make_input_checksums.py      # rewrites the json
"""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from gated_deltanet_decode_delta_amd import inputs  # noqa: E402

OUT = os.path.join(HERE, "input_checksums.json")
CASE_FIELDS = ("state", "q", "k", "v", "z", "alpha", "beta", "gn")
FRONT_FIELDS = ("state", "ring", "x", "w", "br", "ar", "dt", "rate", "z", "gn")


def digest(a: np.ndarray) -> str:
    """sha256 of the array's bytes in C order, with its dtype and shape."""
    h = hashlib.sha256()
    h.update(f"{a.dtype.str}{a.shape}".encode())
    h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def workloads():
    """(name, case, fields) of every pinned workload, one at a time."""
    for name in inputs.CONFIGS:
        yield name, (lambda n=name: inputs.config_case(n)), CASE_FIELDS
    yield ("sequence/normal", lambda: inputs.config_case("sequence", state_init="normal"),
           CASE_FIELDS)
    for layer in (0, 47):   # first and last of the 48 real-head layer states
        yield (f"real_head/layer{layer}",
               lambda s=2000 + layer: inputs.make_case(s, B=1, NK=16, NV=48, D=128), CASE_FIELDS)
    yield ("frontend/B64",
           lambda: inputs.make_frontend_case(3200, B=64, NK=16, NV=48, D=128, taps=4, pitch=983040),
           FRONT_FIELDS)


def compute() -> dict:
    out = {}
    for name, make, fields in workloads():
        c = make()
        out[name] = {f: digest(getattr(c, f)) for f in fields}
        del c
    return out


if __name__ == "__main__":
    data = {"_what": "sha256 of dtype, shape and C-order bytes of each generated input array",
            "workloads": compute()}
    with open(OUT, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(OUT)
