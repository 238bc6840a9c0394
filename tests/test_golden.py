"""The oracle still reproduces its frozen outputs on the tiny Mamba-2 workload.

The fixture was written by tests/golden/make_golden.py from the oracle alone;
it guards against unintended changes to the oracle's arithmetic.
"""
import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_oracle_matches_frozen_fixture():
    import importlib.util

    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(HERE, "golden", "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    outs, ses = mg.run()
    doc = json.load(open(os.path.join(HERE, "golden", "mamba2_tiny_oracle.json")))
    ref = np.array(doc["outputs"])
    np.testing.assert_allclose(outs[doc["steps"]], ref, rtol=1e-13, atol=1e-13)
    assert ses.pm.snapshot() == doc["final_pointers"]
