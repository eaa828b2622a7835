"""Pins of the fp64 target-attention oracle against values fixed outside it:
scipy's softmax, a pure-Python brute force, closed forms and invariances."""
import math

import numpy as np
import pytest
import scipy.special

from oracle import target_attention_batch, target_attention_one


def _brute(Q, S):
    d = len(S[0])
    out, lse = [], []
    for q in Q:
        sc = [sum(q[e] * s[e] for e in range(d)) / math.sqrt(d) for s in S]
        top = max(sc)
        ex = [math.exp(v - top) for v in sc]
        z = sum(ex)
        out.append([sum(ex[j] / z * S[j][e] for j in range(len(S))) for e in range(d)])
        lse.append(top + math.log(z))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_and_scipy(seed):
    g = np.random.default_rng(seed)
    c, k, d = 5, 7, 4
    Q, S = g.standard_normal((c, d)) * 2, g.standard_normal((k, d))
    out, lse = target_attention_one(Q, S)
    bo, bl = _brute(Q.tolist(), S.tolist())
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-13)
    a = scipy.special.softmax(Q @ S.T / math.sqrt(d), axis=1)
    np.testing.assert_allclose(out, a @ S, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(Q @ S.T / math.sqrt(d), axis=1), rtol=1e-12)


def test_closed_forms():
    g = np.random.default_rng(1)
    d, k = 6, 9
    S = g.standard_normal((k, d))
    Q = g.standard_normal((4, d))
    # equal rows: every weighting returns that row
    row = g.standard_normal(d)
    out, _ = target_attention_one(Q, np.tile(row, (k, 1)))
    np.testing.assert_allclose(out, np.tile(row, (4, 1)), rtol=1e-13, atol=1e-14)
    # zero query: uniform weights, the mean row; lse = log k
    out, lse = target_attention_one(np.zeros((2, d)), S)
    np.testing.assert_allclose(out, np.tile(S.mean(axis=0), (2, 1)), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(k), rtol=1e-14)
    # one key: that row, lse = the single score
    out, lse = target_attention_one(Q, S[:1])
    np.testing.assert_allclose(out, np.tile(S[0], (4, 1)), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, Q @ S[0] / math.sqrt(d), rtol=1e-13)
    # a dominant key: q aligned with s_3 scaled up picks row 3
    q = 1e4 * S[3][None, :]
    out, _ = target_attention_one(q, S)
    np.testing.assert_allclose(out[0], S[3], rtol=1e-10, atol=1e-10)


def test_invariances():
    g = np.random.default_rng(2)
    d, k = 5, 11
    S = g.standard_normal((k, d))
    Q = g.standard_normal((6, d))
    out, lse = target_attention_one(Q, S)
    perm = g.permutation(k)
    o2, l2 = target_attention_one(Q, S[perm])
    np.testing.assert_allclose(o2, out, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l2, lse, rtol=1e-13)
    # translating every sketch row by b shifts each score of a candidate by
    # the same amount, so the weights stay and the output moves by b
    b = g.standard_normal(d)
    o3, _ = target_attention_one(Q, S + b)
    np.testing.assert_allclose(o3, out + b, rtol=1e-12, atol=1e-13)


def test_batch_layout_and_empty_users():
    g = np.random.default_rng(3)
    d, k = 4, 3
    S = g.standard_normal((3, k, d))
    lens = [2, 0, 3]
    off = np.concatenate([[0], np.cumsum(lens)])
    Q = g.standard_normal((5, d))
    out, lse = target_attention_batch(Q, off, S)
    np.testing.assert_allclose(out[:2], target_attention_one(Q[:2], S[0])[0], rtol=1e-14)
    np.testing.assert_allclose(out[2:], target_attention_one(Q[2:], S[2])[0], rtol=1e-14)
