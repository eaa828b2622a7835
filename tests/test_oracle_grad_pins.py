"""Pins of the fp64 gradient oracle against values fixed outside it.

The oracle differentiates the forward definition node by node.  These tests
check it against (1) central finite differences of the forward oracle, whose
own pins are in test_oracle_pins.py; (2) closed forms for two special cases
worked out by hand (one prototype; Wk = 0, where every allocation is 1/k);
(3) identities that follow from invariances of the forward map.  A dropped
term (the mass derivative), a sign error, a missing softmax centring or a
transposed operand each breaks at least the finite differences and one of
the closed forms.
"""
import math

import numpy as np
import pytest

from oracle import sketch_batch, sketch_batch_grad, sketch_one_grad


def _case(seed, lens=(5, 3, 4), k=4, d=3, masked=True):
    g = np.random.default_rng(seed)
    N = sum(lens)
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    H = g.standard_normal((N, d))
    Wk = g.standard_normal((d, d))
    Wv = g.standard_normal((d, d))
    P = g.standard_normal((k, d))
    G = g.standard_normal((len(lens), k, d))
    mask = (g.random(N) > 0.25).astype(np.uint8) if masked else None
    return H, offsets, Wk, Wv, P, G, mask


def _loss(H, offsets, Wk, Wv, P, G, mask):
    S, _ = sketch_batch(H, offsets, Wk, Wv, P, mask)
    return float((S * G).sum())


def _fd(f, X, eps=1e-6):
    out = np.zeros_like(X)
    it = np.nditer(X, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        Xp = X.copy()
        Xm = X.copy()
        Xp[i] += eps
        Xm[i] -= eps
        out[i] = (f(Xp) - f(Xm)) / (2 * eps)
    return out


@pytest.mark.parametrize("seed", range(4))
def test_finite_differences(seed):
    H, off, Wk, Wv, P, G, mask = _case(seed)
    dH, dP, dWk, dWv = sketch_batch_grad(H, off, Wk, Wv, P, G, mask)
    fH = _fd(lambda X: _loss(X, off, Wk, Wv, P, G, mask), H)
    fP = _fd(lambda X: _loss(H, off, Wk, Wv, X, G, mask), P)
    fWk = _fd(lambda X: _loss(H, off, X, Wv, P, G, mask), Wk)
    fWv = _fd(lambda X: _loss(H, off, Wk, X, P, G, mask), Wv)
    for got, want in ((dH, fH), (dP, fP), (dWk, fWk), (dWv, fWv)):
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-7)
    # masked tokens take no part: their rows are exactly zero
    assert np.all(dH[mask == 0] == 0.0)


def test_finite_differences_sharp_softmax():
    # large logits: allocations close to one-hot, where a wrong centring shows
    H, off, Wk, Wv, P, G, mask = _case(11, lens=(6,), k=5, d=4, masked=False)
    P = 3.0 * P
    dH, dP, dWk, dWv = sketch_batch_grad(H, off, Wk, Wv, P, G, mask)
    fP = _fd(lambda X: _loss(H, off, Wk, Wv, X, G, mask), P)
    fH = _fd(lambda X: _loss(X, off, Wk, Wv, P, G, mask), H)
    np.testing.assert_allclose(dP, fP, rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(dH, fH, rtol=1e-5, atol=1e-7)


def test_closed_form_one_prototype():
    # k = 1: A = 1, m = n, S = mean of the values, the logits do not matter
    g = np.random.default_rng(5)
    n, d = 7, 4
    H, Wk, Wv = g.standard_normal((n, d)), g.standard_normal((d, d)), g.standard_normal((d, d))
    P, G = g.standard_normal((1, d)), g.standard_normal((1, d))
    dH, dP, dWk, dWv = sketch_one_grad(H, Wk, Wv, P, G)
    np.testing.assert_allclose(dP, 0.0, atol=1e-14)
    np.testing.assert_allclose(dWk, 0.0, atol=1e-14)
    np.testing.assert_allclose(dH, np.tile(G @ Wv.T / n, (n, 1)), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dWv, np.outer(H.mean(axis=0), G[0]), rtol=1e-13, atol=1e-14)


def test_closed_form_one_token():
    # n = 1: A[j] = 1 for every prototype, m_j = 1, S_j = h Wv whatever P and
    # Wk are, so dP = dWk = 0, dH = (sum_j G_j) Wv^T, dWv = h^T (sum_j G_j)
    g = np.random.default_rng(7)
    k, d = 5, 4
    H, Wk, Wv = g.standard_normal((1, d)), g.standard_normal((d, d)), g.standard_normal((d, d))
    P, G = g.standard_normal((k, d)), g.standard_normal((k, d))
    dH, dP, dWk, dWv = sketch_one_grad(H, Wk, Wv, P, G)
    np.testing.assert_allclose(dP, 0.0, atol=1e-14)
    np.testing.assert_allclose(dWk, 0.0, atol=1e-14)
    np.testing.assert_allclose(dH, G.sum(axis=0)[None, :] @ Wv.T, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dWv, np.outer(H[0], G.sum(axis=0)), rtol=1e-13, atol=1e-14)


def test_closed_form_zero_key_projection():
    # Wk = 0: every logit is 0, A = 1/k, m_j = n/k, S_j = mean value row vbar.
    # Worked by hand from the definition:
    #   dA[j,t] = (k/n) G_j . (v_t - vbar)
    #   dK_t    = (1/(n sqrt d)) sum_j (G_j . (v_t - vbar)) (p_j - pbar)
    #   dWk = H^T dK,  dP = 0,  dH_t = (sum_j G_j) Wv^T / n,  dWv = hbar (sum_j G_j)^T
    g = np.random.default_rng(6)
    n, k, d = 6, 5, 3
    H, Wv = g.standard_normal((n, d)), g.standard_normal((d, d))
    Wk = np.zeros((d, d))
    P, G = g.standard_normal((k, d)), g.standard_normal((k, d))
    dH, dP, dWk, dWv = sketch_one_grad(H, Wk, Wv, P, G)
    V = H @ Wv
    vbar, pbar = V.mean(axis=0), P.mean(axis=0)
    dK = np.zeros((n, d))
    for t in range(n):
        for j in range(k):
            dK[t] += (G[j] @ (V[t] - vbar)) * (P[j] - pbar)
    dK /= n * math.sqrt(d)
    np.testing.assert_allclose(dP, 0.0, atol=1e-14)
    np.testing.assert_allclose(dWk, H.T @ dK, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dH, np.tile(G.sum(axis=0) @ Wv.T / n, (n, 1)), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dWv, np.outer(H.mean(axis=0), G.sum(axis=0)), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("seed", range(3))
def test_invariance_identities(seed):
    g = np.random.default_rng(40 + seed)
    lens = (9, 0, 6, 12)
    k, d = 6, 5
    H, off, Wk, Wv, P, G, mask = _case(40 + seed, lens=lens, k=k, d=d)
    dH, dP, dWk, dWv = sketch_batch_grad(H, off, Wk, Wv, P, G, mask)
    S, _ = sketch_batch(H, off, Wk, Wv, P, mask)
    # adding one vector to every prototype leaves every softmax unchanged
    np.testing.assert_allclose(dP.sum(axis=0), 0.0, atol=1e-12)
    # P -> a P with Wk -> Wk / a leaves the logits unchanged
    assert abs((dP * P).sum() - (dWk * Wk).sum()) < 1e-11 * (1 + abs((dP * P).sum()))
    # S is linear in Wv: <dWv, Wv> = <G, S>
    assert abs((dWv * Wv).sum() - (G * S).sum()) < 1e-11 * (1 + abs((G * S).sum()))
    # H -> a H equals (Wk, Wv) -> (a Wk, a Wv): <dH, H> = <dWk, Wk> + <dWv, Wv>
    lhs = (dH * H).sum()
    rhs = (dWk * Wk).sum() + (dWv * Wv).sum()
    assert abs(lhs - rhs) < 1e-11 * (1 + abs(lhs))
    del g


def test_mask_equals_removal_and_empty_users():
    H, off, Wk, Wv, P, G, mask = _case(21, lens=(8, 5, 0, 7), k=4, d=3)
    dH, dP, dWk, dWv = sketch_batch_grad(H, off, Wk, Wv, P, G, mask)
    keep = mask != 0
    lens2 = [int(keep[off[u]:off[u + 1]].sum()) for u in range(len(off) - 1)]
    off2 = np.concatenate([[0], np.cumsum(lens2)]).astype(np.int64)
    dH2, dP2, dWk2, dWv2 = sketch_batch_grad(H[keep], off2, Wk, Wv, P, G)
    np.testing.assert_allclose(dH[keep], dH2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dP, dP2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dWk, dWk2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dWv, dWv2, rtol=1e-13, atol=1e-15)
    # a user with no tokens has a constant (zero) sketch: its G changes nothing
    G3 = G.copy()
    G3[2] = 1e3
    out = sketch_batch_grad(H, off, Wk, Wv, P, G3, mask)
    for a, b in zip(out, (dH, dP, dWk, dWv)):
        np.testing.assert_array_equal(a, b)
