"""Brute-force Sketch Attention for tiny inputs: pure Python loops, math.exp.

TEST INFRASTRUCTURE, used only by the oracle's own tests.  It follows the
same definition as ``sa_oracle`` (prototype logits p_j . (h_t Wk) / sqrt(d),
softmax over prototypes for each token, mass-normalised sum of values) but
spells every sum out as an explicit loop, one scalar at a time, with no numpy.
"""
from __future__ import annotations

import math


def sketch_bruteforce(H, Wk, Wv, P):
    """H: list of n rows of d floats; Wk, Wv: d x d; P: k x d.  Returns (S, m, A)."""
    n = len(H)
    k = len(P)
    d = len(Wk)
    dv = len(Wv[0])
    # keys and values, one coordinate at a time
    K = [[sum(H[t][a] * Wk[a][b] for a in range(d)) for b in range(d)] for t in range(n)]
    V = [[sum(H[t][a] * Wv[a][b] for a in range(d)) for b in range(dv)] for t in range(n)]
    A = [[0.0] * n for _ in range(k)]
    for t in range(n):
        col = [sum(P[j][b] * K[t][b] for b in range(d)) / math.sqrt(d) for j in range(k)]
        top = max(col)
        ex = [math.exp(v - top) for v in col]
        z = sum(ex)
        for j in range(k):
            A[j][t] = ex[j] / z
    m = [sum(A[j][t] for t in range(n)) for j in range(k)]
    S = [[0.0] * dv for _ in range(k)]
    for j in range(k):
        if m[j] > 0.0:
            for c in range(dv):
                S[j][c] = sum(A[j][t] * V[t][c] for t in range(n)) / m[j]
    return S, m, A
