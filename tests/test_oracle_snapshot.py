"""Regression guard: the oracle still reproduces its stored c1 snapshot."""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_c1_snapshot  # noqa: E402


def test_c1_snapshot_unchanged():
    with open(os.path.join(HERE, "golden", "c1_oracle_snapshot.json")) as f:
        want = json.load(f)
    got = make_c1_snapshot.snapshot()
    assert got["idx"] == want["idx"]
    assert np.allclose(got["tau"], want["tau"], rtol=1e-13, atol=0)
    assert np.allclose(got["out"], want["out"], rtol=1e-12, atol=1e-14)
