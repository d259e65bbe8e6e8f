"""Regression pin: the oracle reproduces its stored fp64 outputs for a tiny case
(tests/golden/kda_small_case.json, written by tests/golden/make_golden.py)."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kda_small_case.json")


def test_oracle_matches_stored_small_case():
    with open(GOLDEN) as f:
        d = json.load(f)
    x = {n: np.array(a) for n, a in d["inputs"].items()}
    e = {n: np.array(a) for n, a in d["expected"].items()}
    g = oracle.gate(x["z"], x["A"])
    np.testing.assert_allclose(g, e["g"], rtol=1e-14, atol=0)
    o, ST = oracle.forward(x["q"], x["k"], x["v"], e["g"], x["beta"], x["S0"])
    np.testing.assert_allclose(o, e["o"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(ST, e["ST"], rtol=1e-13, atol=1e-15)
    o2, S2 = oracle.forward_np(x["q"], x["k"], x["v"], e["g"], x["beta"], x["S0"])
    np.testing.assert_allclose(o2, e["o"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S2, e["ST"], rtol=1e-13, atol=1e-15)
