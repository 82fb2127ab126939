"""Writes the frozen oracle regression fixture oracle_s8_regression.txt.

Calls only the oracle and the seeded input generator.  The fixture guards
against unintended drift of the oracle's arithmetic: regenerate it only with a
commit whose message names the passage of the pages that justifies the change.

    python tests/golden/make_golden.py
"""

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

PATH = os.path.join(HERE, "oracle_s8_regression.txt")


def problem():
    """8 tokens, 4 query heads over 2 KV heads, head dim 256, seed 2024, gate sigma 2."""
    return synth.make_problem(T=8, n_q_heads=4, n_kv_heads=2, seed=2024, gate_sigma=2.0)


def read():
    rows = []
    with open(PATH) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            rows.append([int(t, 16) for t in line.split()])
    return np.array(rows, dtype=np.uint16)


def write():
    import oracle
    p = problem()
    out = oracle.get().attention(p)
    with open(PATH, "w") as f:
        f.write("# gated output bits [row][Hq*D] of tests/golden/make_golden.py:problem(),\n")
        f.write(f"# inputs sha256 {p.digest()}\n")
        for row in out:
            f.write(" ".join(f"{x:04x}" for x in row) + "\n")


if __name__ == "__main__":
    write()
