"""The seeded inputs are the same arrays on every machine.

``tests/golden/input_checksums.json`` holds the sha256 of every array the input
generator draws for the benchmark workloads (written by
``tests/golden/make_input_checksums.py``).  A drift of numpy's PCG64 stream or
of the draw order would change every workload; this test catches it.
"""
import importlib.util
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = os.path.join(HERE, "golden")


def _maker():
    spec = importlib.util.spec_from_file_location("make_input_checksums",
                                                  os.path.join(GOLD, "make_input_checksums.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_generated_inputs_match_stored_checksums():
    want = json.load(open(os.path.join(GOLD, "input_checksums.json")))["workloads"]
    mk = _maker()
    seen = set()
    for name, make, fields in mk.workloads():
        c = make()
        for f in fields:
            assert mk.digest(getattr(c, f)) == want[name][f], (name, f)
        seen.add(name)
        del c
    assert seen == set(want)


def test_checksum_covers_dtype_and_shape():
    import numpy as np
    mk = _maker()
    a = np.arange(8, dtype=np.float32)
    assert mk.digest(a) != mk.digest(a.reshape(2, 4))
    assert mk.digest(a) != mk.digest(a.view(np.int32))
