"""Writes oracle_regression.json: a small seeded case and the fp64 oracle's outputs for it.

The stored values come only from the oracle (``oracle`` package) and the seeded generators;
the test that reads the file guards the oracle against accidental changes to its arithmetic.
Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

LENGTHS = [13, 0, 27]
H, D, SEED = 2, 4, 5
DECAY = [0.9, 1.0]


def case():
    rng = np.random.default_rng(SEED)
    T = sum(LENGTHS)
    q, k, v = (rng.standard_normal((T, H, D)) for _ in range(3))
    S0 = rng.standard_normal((len(LENGTHS), H, D, D))
    cu = np.concatenate([[0], np.cumsum(LENGTHS)]).astype(np.int32)
    return q, k, v, np.array(DECAY), cu, S0


def backward_case():
    """case() plus upstream gradients d_out [T,H,D] and d_final [S,H,D,D], drawn after it."""
    rng = np.random.default_rng(SEED)
    T = sum(LENGTHS)
    for _ in range(3):
        rng.standard_normal((T, H, D))
    rng.standard_normal((len(LENGTHS), H, D, D))
    d_out = rng.standard_normal((T, H, D))
    d_final = rng.standard_normal((len(LENGTHS), H, D, D))
    return case() + (d_out, d_final)


def main():
    q, k, v, lam, cu, S0, d_out, d_final = backward_case()
    out = oracle.quadratic(q, k, v, lam, cu, init_state=S0)
    st = oracle.final_state(k, v, lam, cu, init_state=S0)
    dq, dk, dv, d_init = oracle.backward(q, k, v, lam, d_out, cu, init_state=S0, d_final=d_final)
    doc = {
        "what": "fp64 oracle outputs for a seeded varlen case with an empty sequence and an "
                "initial state; written by tests/golden/make_golden.py from the oracle only",
        "lengths": LENGTHS, "H": H, "D": D, "seed": SEED, "decay": DECAY,
        "out": out.tolist(), "final_state": st.tolist(),
        "dq": dq.tolist(), "dk": dk.tolist(), "dv": dv.tolist(), "d_init": d_init.tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=0)
    print("wrote", path)


if __name__ == "__main__":
    main()
