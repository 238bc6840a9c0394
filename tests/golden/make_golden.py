"""Writes tests/golden/mamba2_tiny_oracle.json from the oracle alone.

The pages print no worked numerical example, so this file holds no page value:
it freezes the fp64 oracle's outputs on the tiny Mamba-2 workload (B=1, H=2,
P=N=16, L=4, 64 decode steps, seed 0) so that any later change to the oracle's
arithmetic shows up as a failing comparison and has to be justified.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle.session import OracleSession, select_heads  # noqa: E402
from synth import WORKLOADS, host_initial_state, host_step  # noqa: E402


def run(seed=0):
    w = WORKLOADS["mamba2_tiny"]
    sh = w.shape
    heads = [(b, h) for b in range(sh.B) for h in range(sh.H)]
    S0 = host_initial_state(seed, w.wid, sh, w.s0_sigma).reshape(-1, sh.P, sh.N)
    ses = OracleSession("mamba2", sh.B, sh.H, sh.P, sh.N, w.L, w.T, S0, heads)
    outs = []
    for t in range(w.steps):
        x = host_step(seed, w.wid, t, sh, 1)
        ses.append(select_heads(x["alpha"], heads), select_heads(x["k"], heads), select_heads(x["v"], heads))
        o, _, _ = ses.decode(select_heads(x["q"], heads))
        outs.append(o[:, 0])
    return np.stack(outs), ses


if __name__ == "__main__":
    outs, ses = run()
    doc = {
        "what": "fp64 oracle outputs o[step][head][p], mamba2_tiny workload, seed 0, every 4th step",
        "source": "written by tests/golden/make_golden.py, which calls only oracle/ and synth/",
        "steps": list(range(0, outs.shape[0], 4)),
        "outputs": [[[float(f"{x:.17g}") for x in row] for row in outs[s]] for s in range(0, outs.shape[0], 4)],
        "final_pointers": ses.pm.snapshot(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mamba2_tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", path)
