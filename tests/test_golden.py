"""The oracle's output on the tiny fp32 workload has not drifted from the frozen
record written by tests/golden/make_golden.py (CPU only)."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


def test_oracle_matches_frozen_record():
    rec = json.load(open(make_golden.OUT))
    _, y, hL = make_golden.compute()
    got_y = np.array([[y[0, t, h, :4] for h in range(4)] for t in rec["tokens"]])
    assert np.allclose(got_y, np.array(rec["y"]), rtol=1e-13, atol=1e-15)
    assert np.allclose(hL[0, :, 0, :4], np.array(rec["final_state"]), rtol=1e-13, atol=1e-15)
