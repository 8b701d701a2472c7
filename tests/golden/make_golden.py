"""Writes oracle_tiny.json: the CPU oracle's outputs on a tiny fixed input, kept
as a regression fixture (a later change to the oracle's arithmetic shows up as
a mismatch).  Calls only oracle/.  Run from the repository root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import oracle as O  # noqa: E402


def tiny_inputs():
    # small exact binary fractions, so the inputs are the same in every dtype
    T, H, d = 5, 2, 4
    n = T * H * d
    base = (np.arange(n, dtype=np.float64) % 9 - 4) / 8.0
    q = base.reshape(T, H, d)
    k = np.roll(base, 3).reshape(T, H, d)
    v = np.roll(base, 7).reshape(T, H, d)
    x = np.roll(base, 11).reshape(T, H * d)
    return q, k, v, x


def main():
    q, k, v, x = tiny_inputs()
    out, S, _ = O.forward(q, k, v, x, gated=True)
    yn, Sn, zn = O.forward(q + 1.0, k + 1.0, v, normalized=True)
    doc = {
        "note": "oracle outputs on tiny_inputs(); regression fixture written by make_golden.py",
        "gated_out": out.tolist(), "state": S.tolist(),
        "normalized_y": yn.tolist(), "normalized_z": zn.tolist(),
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
