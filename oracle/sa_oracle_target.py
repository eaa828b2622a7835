"""Plain fp64 oracle of sketch-branch target attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run this module.  It shares no
code with the HIP library.

What it computes, and where the pages say so: after compression, each
candidate item attends over its user's fixed-size sketch (blog "100,000
videos in your pocket", "How it works" item 2, the sketch branch of STCA);
one user's many candidates share one read of that sketch (same page, item 3,
multi-request user-level batching).  The stacking of STCA is defined only in
the predecessor paper, which is not among the pages, so this is the plainest
single-layer reading: single-head scaled dot-product cross attention in which
the candidate's query vector q_c attends over the k sketch rows s_j of its
user, which serve as both keys and values:

    a[c, j] = exp(q_c . s_j / sqrt(d)) / sum_j' exp(q_c . s_j' / sqrt(d))
    out_c   = sum_j a[c, j] s_j

Any projections of the candidate or of the sketch, further layers and the
fusion with the recent-history branch are outside this operation.

Pinned by ``tests/test_oracle_target_pins.py``: scipy's softmax, a
pure-Python brute force, closed forms (equal rows, zero query, one key, a
dominant key) and invariances (key permutation, translation of the sketch).
"""
from __future__ import annotations

import numpy as np

__all__ = ["target_attention_one", "target_attention_batch"]


def target_attention_one(Qu, Su):
    """Qu [c, d] candidate queries of one user, Su [k, d] the user's sketch.

    Returns (out [c, d], lse [c]) in fp64; lse is the natural-log normaliser
    log sum_j exp(q . s_j / sqrt(d)).
    """
    Qu = np.asarray(Qu, dtype=np.float64)
    Su = np.asarray(Su, dtype=np.float64)
    d = Su.shape[1]
    if Qu.shape[0] == 0:
        return np.zeros((0, d)), np.zeros(0)
    scores = (Qu @ Su.T) / np.sqrt(d)                # [c, k]
    top = scores.max(axis=1, keepdims=True)
    e = np.exp(scores - top)
    z = e.sum(axis=1, keepdims=True)
    a = e / z                                        # softmax over the sketch rows
    return a @ Su, (top + np.log(z))[:, 0]


def target_attention_batch(Q, cand_offsets, S):
    """Q [C, d] candidates packed user by user (user u owns rows
    cand_offsets[u] .. cand_offsets[u+1]-1), S [R, k, d] sketches.
    Returns out [C, d] and lse [C] (fp64)."""
    Q = np.asarray(Q, dtype=np.float64)
    off = np.asarray(cand_offsets, dtype=np.int64)
    out = np.zeros((Q.shape[0], np.shape(S)[2]))
    lse = np.zeros(Q.shape[0])
    for u in range(off.shape[0] - 1):
        lo, hi = int(off[u]), int(off[u + 1])
        out[lo:hi], lse[lo:hi] = target_attention_one(Q[lo:hi], S[u])
    return out, lse
