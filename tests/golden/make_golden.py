"""Writes tiny_f32_oracle.json: a frozen sample of the fp64 oracle's output on the
tiny fp32 workload (1 x 256 tokens, 4 heads, P = N = 16), so that any later change
to the oracle's arithmetic shows up as a diff.  Calls only ``oracle`` (and the
seeded input generator); nothing here comes from the HIP library.

The pages ("Compiler-First State Space Duality and Portable O(1) Autoregressive
Caching for Inference") print no worked numeric SSD example, so this fixture is a
regression record of the oracle, not an independent pin; the independent pins
are in tests/test_oracle_pins.py.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import ssd_inputs as si  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_f32_oracle.json")


def compute():
    w = si.WORKLOADS["tiny_f32"]
    A, D = si.head_params(w)
    inp = si.prefill_inputs(w)
    wid = {k: si.widen(v, w.io) if k != "dt" else v.astype(np.float64) for k, v in inp.items()}
    y, hL = oracle.ssd_scan(wid["x"], wid["dt"], A, wid["B"], wid["C"], D)
    return w, y, hL


def main():
    w, y, hL = compute()
    rec = {
        "workload": w.name,
        "what": "fp64 oracle: y[0, t, h, 0:4] for t in {0, 1, 63, 64, 255}, h in 0..3; final state [0, h, 0, 0:4]",
        "tokens": [0, 1, 63, 64, 255],
        "y": [[[float(v) for v in y[0, t, h, :4]] for h in range(w.nheads)] for t in [0, 1, 63, 64, 255]],
        "final_state": [[float(v) for v in hL[0, h, 0, :4]] for h in range(w.nheads)],
    }
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
