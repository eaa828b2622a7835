"""Plain fp64 oracle of the gradients of Sketch Attention (SA) compression.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run this module.  It shares no
code with the HIP library.

Why gradients: the blog "100,000 videos in your pocket" ("How it works",
item 1) notes that the compression is differentiable, so the gradients of
the final ranking loss flow back through it and train the prototypes and
projections; its "State of the art: the pattern behind the paper" item 2
and "Takeaways" say SequenceO1 trains the compressor on the ranking loss end
to end instead of freezing an offline stage.  The pages give no formula for the backward pass; it is the
chain rule applied to the forward definition of ``sa_oracle`` (the same
readings: K = H Wk, V = H Wv, logits P K^T / sqrt(d), softmax over
prototypes per token, each sketch row the mass-weighted mean of the values,
zero rows where the mass is zero, masked tokens removed).

Given dS = dLoss/dS for every user, this module returns dLoss/dH (per token),
and dLoss/dP, dLoss/dWk, dLoss/dWv summed over the users of the batch (the
prototypes and projections are shared by all users).  Every step below is
one node of the forward graph, differentiated on its own, in the order the
forward runs backwards; nothing is reassociated.

Pinned by ``tests/test_oracle_grad_pins.py``: central finite differences of
the forward oracle, closed forms for k = 1 and for Wk = 0, and the identities
that follow from the forward's invariances (prototype translation, the
P/Wk rescaling, homogeneity in Wv and in H).
"""
from __future__ import annotations

import numpy as np

__all__ = ["sketch_one_grad", "sketch_batch_grad"]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def sketch_one_grad(Hu, Wk, Wv, P, G):
    """Gradients of Loss through one user's (unmasked) sketch.

    Hu [n, d], Wk [d, d], Wv [d, d], P [k, d], G = dLoss/dS [k, d].
    Returns (dHu [n, d], dP [k, d], dWk [d, d], dWv [d, d]) in fp64.
    """
    Hu, Wk, Wv, P, G = _f64(Hu), _f64(Wk), _f64(Wv), _f64(P), _f64(G)
    n, d = Hu.shape[0], Wk.shape[1]
    k = P.shape[0]
    if n == 0:
        return np.zeros((0, Hu.shape[1])), np.zeros_like(P), np.zeros_like(Wk), np.zeros_like(Wv)
    rs = 1.0 / np.sqrt(d)
    # forward, keeping every intermediate
    K = Hu @ Wk                                   # [n, d]
    V = Hu @ Wv                                   # [n, d]
    L = (P @ K.T) * rs                            # [k, n]
    c = L.max(axis=0, keepdims=True)
    E = np.exp(L - c)
    A = E / E.sum(axis=0, keepdims=True)          # softmax over prototypes (axis 0)
    m = A.sum(axis=1)                             # [k]
    U = A @ V                                     # [k, d]
    ok = m > 0
    S = np.zeros((k, V.shape[1]))
    S[ok] = U[ok] / m[ok, None]
    # S_j = U_j / m_j (rows with m_j = 0 are the constant 0: no gradient)
    dU = np.zeros_like(U)
    dU[ok] = G[ok] / m[ok, None]
    dm = np.zeros(k)
    dm[ok] = -(G[ok] * S[ok]).sum(axis=1) / m[ok]     # d(U_j / m_j) / dm_j = -S_j / m_j
    # U = A V and m = A 1
    dA = dU @ V.T + dm[:, None]                   # [k, n]
    dV = A.T @ dU                                 # [n, d]
    # A[:, t] = softmax(L[:, t]): Jacobian diag(a) - a a^T, applied per token
    dL = A * (dA - (A * dA).sum(axis=0, keepdims=True))
    # L = P K^T / sqrt(d)
    dP = (dL @ K) * rs                            # [k, d]
    dK = (dL.T @ P) * rs                          # [n, d]
    # K = Hu Wk, V = Hu Wv
    dHu = dK @ Wk.T + dV @ Wv.T
    dWk = Hu.T @ dK
    dWv = Hu.T @ dV
    return dHu, dP, dWk, dWv


def sketch_batch_grad(H, offsets, Wk, Wv, P, G, mask=None):
    """Gradients through a packed ragged batch (the layout of ``sketch_batch``).

    G [R, k, d] = dLoss/dS.  Returns dH [N, d] (zero rows for masked tokens),
    and dP, dWk, dWv summed over the users, all fp64.
    """
    H = _f64(H)
    offsets = np.asarray(offsets, dtype=np.int64)
    R = offsets.shape[0] - 1
    dH = np.zeros_like(H)
    dP = np.zeros(np.shape(P))
    dWk = np.zeros(np.shape(Wk))
    dWv = np.zeros(np.shape(Wv))
    for u in range(R):
        lo, hi = int(offsets[u]), int(offsets[u + 1])
        rows = np.arange(lo, hi)
        if mask is not None:
            rows = rows[np.asarray(mask[lo:hi]) != 0]
        gH, gP, gWk, gWv = sketch_one_grad(H[rows], Wk, Wv, P, G[u])
        dH[rows] = gH
        dP += gP
        dWk += gWk
        dWv += gWv
    return dH, dP, dWk, dWv
