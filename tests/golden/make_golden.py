"""Writes the stored expected values under tests/golden/ from the oracle only.

Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def p3_seed42():
    """The 5688vip example's inputs (legacy generator, seed 42, three 4 x 8
    normal draws), standard attention without a scale."""
    np.random.seed(42)
    Q = np.random.randn(4, 8)
    K = np.random.randn(4, 8)
    V = np.random.randn(4, 8)
    out = oracle.attention(Q[None, None], K[None, None], V[None, None], 1.0)[0, 0]
    np.savetxt(os.path.join(HERE, "p3_seed42_output.txt"), out, fmt="%.17e",
               header="oracle output for the 5688vip self-test inputs (seed 42, N=4, d=8, scale 1)")


if __name__ == "__main__":
    p3_seed42()
