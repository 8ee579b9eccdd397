"""Writes tests/golden/oracle_small.json: oracle outputs on one small seeded case.

Calls only the oracle and the seeded input generator.  The stored values are a
regression lock on the oracle (the pins in tests/pins.py are what tie it to
the pages); regenerate only with a change to the oracle that names its reason.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import ssd_inputs  # noqa: E402

CASE = ssd_inputs.Workload("golden_small", 2, 7, 4, 2, 3, 2, 4, "f32", init_state=True, state_out=True, seed=77)


def run_case():
    inp = ssd_inputs.generate(CASE)
    y, fin, sout, _ = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.init_state,
                                         inp.state_out_idx)
    return y, fin, sout, inp


if __name__ == "__main__":
    y, fin, sout, inp = run_case()
    out = {"case": CASE.__dict__, "sha256": inp.sha256, "y": y.ravel().tolist(),
           "final_state": fin.ravel().tolist(), "state_out": sout.ravel().tolist()}
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump(out, f, indent=0)
