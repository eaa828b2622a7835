"""Plain fp64 oracle of Sketch Attention (SA) compression.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run this module.  It is a slow,
obviously correct restatement of the method in numpy float64 and shares no
code with the HIP library.

What SA computes, and where the pages say so (SequenceO1, arXiv 2609.08443):

* arXiv abstract (mlsanity paper page, "Abstract"): SA compresses the raw
  history into a fixed-size, target-agnostic user representation using
  learnable prototypes and prototype-wise normalisation.
* Blog "100,000 videos in your pocket", "How it works" item 1: every history
  item is softly assigned across the k prototypes; every item distributes its
  mass over the prototypes; the output is a k x d sketch.
* Review page (evolve.pub), "Summary" and the FAQ entry on how SA differs from
  standard attention: the weights are normalised across prototypes rather than
  across the sequence, so each token spreads a fixed total mass over the
  prototype slots; the output size does not depend on the history length.

Readings taken where the pages are silent (each one is listed in the design
notes of the repository):

* keys and values are linear projections of the history, K = H Wk and
  V = H Wv (row-vector convention), logits are P K^T / sqrt(d);
* the per-token normaliser is the exponential softmax over the k prototypes;
* "prototype-wise normalisation" also divides each prototype's accumulated
  value sum by that prototype's total mass over tokens, so each sketch row is
  a weighted mean of value rows (the Slot Attention form the paper lists among
  the works it builds on);
* no positions, heads, biases or iterations: one step;
* an empty history, or a prototype whose mass is exactly zero, gives a zero
  sketch row (and zero mass);
* masked tokens take no part at all: the result equals that of the history
  with those tokens removed.

Every function here is pinned by ``tests/test_oracle_*.py`` against values
fixed by hand or by the mathematics (hand-worked examples, closed forms,
library routines, brute force, invariants); none is left parity unpinned.
"""
from __future__ import annotations

import numpy as np

__all__ = ["logits", "allocations", "sketch_one", "sketch_batch", "normalised_rows_batch"]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def logits(Hu, Wk, P) -> np.ndarray:
    """Prototype-token logits L[j, t] = p_j . k_t / sqrt(d), with K = Hu Wk.

    Hu [n, d] history, Wk [d, d], P [k, d].  Returns L [k, n] (fp64).
    The 1/sqrt(d) scale uses d, the key width.
    """
    Hu, Wk, P = _f64(Hu), _f64(Wk), _f64(P)
    d = Wk.shape[1]
    K = Hu @ Wk                      # [n, d]
    return (P @ K.T) / np.sqrt(d)    # [k, n]


def allocations(L) -> np.ndarray:
    """Per-token softmax over prototypes: column t of A sums to one.

    A[j, t] = exp(L[j, t] - c_t) / sum_j' exp(L[j', t] - c_t), where c_t is the
    column maximum (subtracting it changes nothing but keeps exp finite).
    """
    L = _f64(L)
    if L.shape[1] == 0:
        return np.zeros_like(L)
    c = L.max(axis=0, keepdims=True)
    E = np.exp(L - c)
    return E / E.sum(axis=0, keepdims=True)


def sketch_one(Hu, Wk, Wv, P, return_alloc: bool = False):
    """Sketch of one user's (unmasked) history.

    Returns S [k, d] and the prototype masses m [k] (and A [k, n] on request):
        V = Hu Wv,  A = allocations(logits(Hu, Wk, P)),
        m_j = sum_t A[j, t],  S_j = (sum_t A[j, t] V_t) / m_j   (0 where m_j = 0).
    """
    Hu, Wk, Wv, P = _f64(Hu), _f64(Wk), _f64(Wv), _f64(P)
    k, d = P.shape[0], Wv.shape[1]
    n = Hu.shape[0]
    if n == 0:
        S, m, A = np.zeros((k, d)), np.zeros(k), np.zeros((k, 0))
    else:
        V = Hu @ Wv                                  # [n, d]
        A = allocations(logits(Hu, Wk, P))           # [k, n]
        m = A.sum(axis=1)                            # [k]
        U = A @ V                                    # [k, d]
        S = np.zeros((k, d))
        ok = m > 0
        S[ok] = U[ok] / m[ok, None]
    if return_alloc:
        return S, m, A
    return S, m


def sketch_batch(H, offsets, Wk, Wv, P, mask=None, users=None):
    """Sketches of a packed ragged batch.

    H [N, d] holds the users' histories back to back; user u owns rows
    offsets[u] .. offsets[u+1]-1.  ``mask`` [N] (1 = keep) drops tokens.
    ``users`` restricts the work to a subset of user indices (the other rows
    of the result stay zero).  Returns S [R, k, d] and m [R, k] (fp64).
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    R = offsets.shape[0] - 1
    k, d = np.shape(P)[0], np.shape(Wv)[1]
    S = np.zeros((R, k, d))
    m = np.zeros((R, k))
    todo = range(R) if users is None else users
    for u in todo:
        lo, hi = int(offsets[u]), int(offsets[u + 1])
        Hu = H[lo:hi]
        if mask is not None:
            Hu = Hu[np.asarray(mask[lo:hi]) != 0]
        S[u], m[u] = sketch_one(Hu, Wk, Wv, P)
    return S, m


def normalised_rows_batch(H, offsets, Wk, P, mask=None):
    """The mass-normalised history rows Sbar_u[j] = (sum_t A[j,t] h_t) / m_j
    of every user (0 where m_j = 0), so that S_u = Sbar_u Wv.  The value
    projection is linear, so averaging the h rows and then applying Wv equals
    averaging the v rows (blog "How it works" item 1: the sketch of softly
    assigned items).  Returns [R, k, d] (fp64)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    R = offsets.shape[0] - 1
    k, d = np.shape(P)[0], np.shape(H)[1]
    out = np.zeros((R, k, d))
    for u in range(R):
        lo, hi = int(offsets[u]), int(offsets[u + 1])
        Hu = _f64(H[lo:hi])
        if mask is not None:
            Hu = Hu[np.asarray(mask[lo:hi]) != 0]
        if Hu.shape[0] == 0:
            continue
        A = allocations(logits(Hu, Wk, P))
        m = A.sum(axis=1)
        ok = m > 0
        out[u][ok] = (A @ Hu)[ok] / m[ok, None]
    return out
