"""Writes tests/golden/kda_small_case.json: a tiny seeded KDA problem and the
oracle's fp64 outputs for it.  Calls only the oracle (no HIP code).

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def main():
    r = np.random.default_rng(20261202)
    B, T, H, dk, dv = 1, 20, 2, 4, 3
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = unit(r.standard_normal((B, T, H, dk)))
    k = unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, H))))
    z = r.standard_normal((B, T, H, dk))
    A = r.standard_normal((H, dk)) * 0.5
    S0 = r.standard_normal((B, H, dk, dv)) * 0.1
    g = oracle.gate(z, A)
    o, ST = oracle.forward(q, k, v, g, beta, S0)
    out = {
        "_written_by": "tests/golden/make_golden.py (oracle only)",
        "shape": {"B": B, "T": T, "H": H, "dk": dk, "dv": dv},
        "inputs": {n: a.tolist() for n, a in
                   dict(q=q, k=k, v=v, beta=beta, z=z, A=A, S0=S0).items()},
        "expected": {"g": g.tolist(), "o": o.tolist(), "ST": ST.tolist()},
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "kda_small_case.json")
    with open(path, "w") as f:
        json.dump(out, f)
    print("wrote", path)


if __name__ == "__main__":
    main()
