"""Writes oracle_regression.json: oracle outputs on small fixed inputs.

Calls only ``oracle/``.  Run from the repository root:
    python tests/golden/make_golden.py
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import oracle_scan  # noqa: E402

# One channel per column; rows are tokens.  Hand-picked values covering
# ordinary gates, p = 0, phi = 0 (missing observation) and a = 1.
INPUT = {
    "a":   [[0.9, 1.0, 0.5], [0.75, 1.0, 0.001], [0.5, 0.25, 1.0], [1.0, 0.9, 0.001]],
    "p":   [[0.5, 0.0, 1.0], [0.25, 0.0, 0.0], [2.0, 1.0, 1.0], [0.125, 0.0, 0.0]],
    "phi": [[1.0, 2.0, 0.0], [0.0, 0.5, 10000.0], [3.0, 0.0, 0.0], [0.5, 1.0, 10000.0]],
    "b":   [[0.5, -1.0, 0.0], [0.0, 0.25, -10000.0], [-3.0, 0.0, 0.0], [0.25, 2.0, 10000.0]],
    "lam0": [1.0, 2.0, 0.5],
    "eta0": [0.0, -1.0, 0.25],
}


def main():
    import numpy as np
    T = len(INPUT["a"])
    D = len(INPUT["a"][0])
    g = {k: np.array(INPUT[k], dtype=np.float64).reshape(1, 1, T, D)
         for k in ("a", "p", "phi", "b")}
    lam0 = np.array(INPUT["lam0"]).reshape(1, 1, D)
    eta0 = np.array(INPUT["eta0"]).reshape(1, 1, D)
    lam, eta, eta_abs = oracle_scan(g["a"], g["p"], g["phi"], g["b"], lam0, eta0)
    out = {"input": INPUT,
           "lam": lam.reshape(T, D).tolist(),
           "eta": eta.reshape(T, D).tolist(),
           "eta_abs": eta_abs.reshape(T, D).tolist(),
           "writer": "tests/golden/make_golden.py (oracle/ only)"}
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
