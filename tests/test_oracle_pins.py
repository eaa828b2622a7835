"""Pins of the fp64 oracle against values fixed outside the oracle.

Each test compares the oracle with something it does not share code with:
hand-worked examples (tests/golden), closed forms, library routines
(scipy.special.softmax, numpy.average), a pure-Python brute force, and the
invariants the pages state (every token spreads a unit mass over the
prototypes; the sketch has a fixed k x d size; the sketch is user-only).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from oracle import allocations, logits, sketch_batch, sketch_one
from oracle.brute import sketch_bruteforce
from synth import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _frac(a):
    if isinstance(a, str):
        return float(Fraction(a))
    return [_frac(x) for x in a]


def _rand(n, k, d, seed, pscale=1.0):
    g = np.random.default_rng(seed)
    H = g.standard_normal((n, d))
    Wk = g.standard_normal((d, d)) / math.sqrt(d)
    Wv = g.standard_normal((d, d)) / math.sqrt(d)
    P = g.standard_normal((k, d)) / math.sqrt(d) * pscale
    return H, Wk, Wv, P


# ---------------------------------------------------------------- hand-worked
@pytest.mark.parametrize("name", ["hand_d1", "hand_d2", "hard_assignment"])
def test_golden_hand_examples(name):
    o = json.load(open(os.path.join(GOLDEN, name + ".json")))
    tol = o.get("tolerance", 1e-14)
    S, m, A = sketch_one(o["H"], o["Wk"], o["Wv"], o["P"], return_alloc=True)
    np.testing.assert_allclose(S, np.array(_frac(o["expected_S"])), rtol=0, atol=tol)
    np.testing.assert_allclose(m, np.array(_frac(o["expected_m"])), rtol=0, atol=tol)
    if "expected_A" in o:
        np.testing.assert_allclose(A, np.array(_frac(o["expected_A"])), rtol=0, atol=tol)


def test_rows_ratio_on_pages():
    # blog "ELI5": at k=256 the sketch holds ~390x fewer rows than a 100K history
    assert int(100_000 / 256) == 390


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed", range(12))
def test_bruteforce_tiny(seed):
    g = np.random.default_rng(100 + seed)
    n, k, d = int(g.integers(1, 7)), int(g.integers(1, 5)), int(g.integers(1, 4))
    H, Wk, Wv, P = _rand(n, k, d, seed, pscale=float(g.uniform(0.5, 6.0)))
    S, m, A = sketch_one(H, Wk, Wv, P, return_alloc=True)
    Sb, mb, Ab = sketch_bruteforce(H.tolist(), Wk.tolist(), Wv.tolist(), P.tolist())
    np.testing.assert_allclose(S, np.array(Sb), rtol=0, atol=1e-12)
    np.testing.assert_allclose(m, np.array(mb), rtol=0, atol=1e-12)
    np.testing.assert_allclose(A, np.array(Ab), rtol=0, atol=1e-12)


# ---------------------------------------------------------- library routines
def test_allocations_match_scipy_softmax_over_prototypes():
    H, Wk, Wv, P = _rand(200, 17, 8, 1, pscale=5.0)
    L = logits(H, Wk, P)
    np.testing.assert_allclose(allocations(L), scipy.special.softmax(L, axis=0),
                               rtol=1e-13, atol=1e-15)


def test_logits_match_einsum_of_keys():
    H, Wk, Wv, P = _rand(50, 9, 6, 2)
    K = np.einsum("na,ab->nb", H, Wk)
    L_ref = np.einsum("jb,nb->jn", P, K) / math.sqrt(6)
    np.testing.assert_allclose(logits(H, Wk, P), L_ref, rtol=1e-13, atol=1e-14)


def test_sketch_rows_are_np_average_of_values():
    H, Wk, Wv, P = _rand(300, 11, 7, 3, pscale=3.0)
    S, m, A = sketch_one(H, Wk, Wv, P, return_alloc=True)
    V = H @ Wv
    for j in range(11):
        np.testing.assert_allclose(S[j], np.average(V, axis=0, weights=A[j]),
                                   rtol=1e-12, atol=1e-14)


# -------------------------------------------------------------- closed forms
def test_zero_prototypes_give_uniform_allocation_and_mean():
    H, Wk, Wv, P = _rand(123, 10, 5, 4)
    S, m, A = sketch_one(H, Wk, Wv, np.zeros_like(P), return_alloc=True)
    np.testing.assert_allclose(A, np.full_like(A, 0.1), rtol=0, atol=1e-15)
    np.testing.assert_allclose(m, np.full(10, 12.3), rtol=1e-13)
    mean_v = (H @ Wv).mean(axis=0)
    np.testing.assert_allclose(S, np.tile(mean_v, (10, 1)), rtol=1e-12, atol=1e-14)


def test_zero_key_projection_gives_mean():
    H, Wk, Wv, P = _rand(77, 6, 4, 5)
    S, m = sketch_one(H, np.zeros_like(Wk), Wv, P)
    np.testing.assert_allclose(S, np.tile((H @ Wv).mean(axis=0), (6, 1)), rtol=1e-12, atol=1e-14)


def test_single_prototype_gives_mean():
    H, Wk, Wv, P = _rand(64, 1, 5, 6, pscale=10.0)
    S, m = sketch_one(H, Wk, Wv, P)
    np.testing.assert_allclose(S[0], (H @ Wv).mean(axis=0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(m, [64.0], rtol=1e-14)


def test_single_token_gives_its_value_row():
    H, Wk, Wv, P = _rand(1, 13, 6, 7, pscale=4.0)
    S, m = sketch_one(H, Wk, Wv, P)
    np.testing.assert_allclose(S, np.tile((H @ Wv)[0], (13, 1)), rtol=1e-12, atol=1e-14)
    assert abs(m.sum() - 1.0) < 1e-14


def test_identical_value_rows_give_that_row():
    H, Wk, Wv, P = _rand(90, 8, 5, 8, pscale=3.0)
    H[:, 0] = 1.0
    Wv = np.zeros_like(Wv)
    Wv[0] = np.array([0.5, -2.0, 3.25, 0.0, 1.0])   # V_t = H[t,0] * Wv[0] = Wv[0]
    S, m = sketch_one(H, Wk, Wv, P)
    np.testing.assert_allclose(S, np.tile(Wv[0], (8, 1)), rtol=1e-13, atol=1e-14)


def test_empty_history_gives_zeros():
    H, Wk, Wv, P = _rand(0, 5, 4, 9)
    S, m = sketch_one(H, Wk, Wv, P)
    assert S.shape == (5, 4) and m.shape == (5,)
    assert not S.any() and not m.any()


# ---------------------------------------------------------------- invariants
def test_unit_mass_per_token_and_total_mass():
    H, Wk, Wv, P = _rand(500, 33, 8, 10, pscale=4.0)
    S, m, A = sketch_one(H, Wk, Wv, P, return_alloc=True)
    np.testing.assert_allclose(A.sum(axis=0), 1.0, rtol=0, atol=1e-14)
    assert abs(m.sum() - 500) < 1e-10
    # normalised per-prototype weights also sum to one
    np.testing.assert_allclose((A / m[:, None]).sum(axis=1), 1.0, rtol=0, atol=1e-13)


def test_sketch_rows_in_convex_hull_of_values():
    H, Wk, Wv, P = _rand(400, 20, 6, 11, pscale=5.0)
    S, m = sketch_one(H, Wk, Wv, P)
    V = H @ Wv
    assert (S >= V.min(axis=0) - 1e-12).all() and (S <= V.max(axis=0) + 1e-12).all()


def test_token_permutation_invariance():
    H, Wk, Wv, P = _rand(257, 16, 8, 12, pscale=3.0)
    S, m = sketch_one(H, Wk, Wv, P)
    perm = np.random.default_rng(0).permutation(257)
    S2, m2 = sketch_one(H[perm], Wk, Wv, P)
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(m2, m, rtol=1e-12)


def test_history_duplication_invariance():
    H, Wk, Wv, P = _rand(100, 12, 6, 13, pscale=3.0)
    S, m = sketch_one(H, Wk, Wv, P)
    S3, m3 = sketch_one(np.concatenate([H, H, H]), Wk, Wv, P)
    np.testing.assert_allclose(S3, S, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(m3, 3 * m, rtol=1e-12)


def test_prototype_translation_invariance():
    H, Wk, Wv, P = _rand(150, 10, 7, 14, pscale=3.0)
    S, m = sketch_one(H, Wk, Wv, P)
    c = np.random.default_rng(1).standard_normal(7) * 2.0
    S2, m2 = sketch_one(H, Wk, Wv, P + c[None, :])
    np.testing.assert_allclose(S2, S, rtol=1e-11, atol=1e-13)


def test_prototype_permutation_equivariance():
    H, Wk, Wv, P = _rand(150, 10, 7, 15, pscale=3.0)
    S, m = sketch_one(H, Wk, Wv, P)
    perm = np.random.default_rng(2).permutation(10)
    S2, m2 = sketch_one(H, Wk, Wv, P[perm])
    np.testing.assert_allclose(S2, S[perm], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(m2, m[perm], rtol=1e-12)


def test_linearity_in_value_projection():
    H, Wk, Wv, P = _rand(120, 9, 5, 16, pscale=2.0)
    Wv2 = np.random.default_rng(3).standard_normal(Wv.shape)
    S1, _ = sketch_one(H, Wk, Wv, P)
    S2, _ = sketch_one(H, Wk, Wv2, P)
    S12, _ = sketch_one(H, Wk, Wv + Wv2, P)
    np.testing.assert_allclose(S12, S1 + S2, rtol=1e-12, atol=1e-13)


def test_reassociated_form_matches():
    # S = ((A H) / m) Wv with A from L = (P Wk^T / sqrt(d)) H^T: the order of the
    # two projections does not change the sketch.
    H, Wk, Wv, P = _rand(333, 14, 8, 17, pscale=3.0)
    S, m, A = sketch_one(H, Wk, Wv, P, return_alloc=True)
    Q = P @ Wk.T / math.sqrt(8)
    L2 = Q @ H.T
    A2 = scipy.special.softmax(L2, axis=0)
    S2 = ((A2 @ H) / A2.sum(axis=1)[:, None]) @ Wv
    np.testing.assert_allclose(S2, S, rtol=1e-11, atol=1e-13)


def test_fixed_output_size():
    for n in (1, 10, 1000):
        H, Wk, Wv, P = _rand(n, 7, 5, 18)
        S, m = sketch_one(H, Wk, Wv, P)
        assert S.shape == (7, 5) and m.shape == (7,)


# ------------------------------------------------------- ragged batch + mask
def test_batch_equals_single_user_calls():
    inp = make_inputs([5, 0, 31, 200, 1], d=8, k=6, seed=21, dtype="f32")
    S, m = sketch_batch(inp.H, inp.offsets, inp.Wk, inp.Wv, inp.P)
    for u in range(inp.R):
        Su, mu = sketch_one(inp.H[inp.user_slice(u)], inp.Wk, inp.Wv, inp.P)
        np.testing.assert_array_equal(S[u], Su)
        np.testing.assert_array_equal(m[u], mu)
    assert not S[1].any()


def test_mask_equals_truncation():
    inp = make_inputs([40, 77], d=8, k=5, seed=22, dtype="bf16", mask_tail_frac=0.25)
    S, m = sketch_batch(inp.H, inp.offsets, inp.Wk, inp.Wv, inp.P, mask=inp.mask)
    for u in range(inp.R):
        sl = inp.user_slice(u)
        keep = inp.H[sl][inp.mask[sl] == 1]
        n_keep = int(inp.mask[sl].sum())
        np.testing.assert_array_equal(keep, inp.H[sl][:n_keep])
        Su, mu = sketch_one(keep, inp.Wk, inp.Wv, inp.P)
        np.testing.assert_array_equal(S[u], Su)
        assert abs(m[u].sum() - n_keep) < 1e-10


def test_masked_tokens_do_not_propagate_nan():
    inp = make_inputs([30], d=4, k=3, seed=23, dtype="f32", mask_tail_frac=0.2)
    H = inp.H.copy()
    H[inp.mask == 0] = np.nan
    S, m = sketch_batch(H, inp.offsets, inp.Wk, inp.Wv, inp.P, mask=inp.mask)
    assert np.isfinite(S).all() and np.isfinite(m).all()


# ------------------------------------------------------------- a planted bug
def test_planted_transpose_is_caught_by_golden():
    # a wrong orientation of Wk must fail the hand-worked d=2 example
    o = json.load(open(os.path.join(GOLDEN, "hand_d2.json")))
    S_bad, _ = sketch_one(o["H"], np.array(o["Wk"]).T, o["Wv"], o["P"])
    assert np.abs(S_bad - np.array(_frac(o["expected_S"]))).max() > 1e-3


def test_normalised_rows_times_wv_is_the_sketch():
    """Sbar Wv = S for every user (the value projection is linear), with
    masked tokens, an empty user and a one-token user."""
    from oracle import normalised_rows_batch
    g = np.random.default_rng(77)
    lens = [9, 0, 1, 14]
    off = np.concatenate([[0], np.cumsum(lens)])
    d, k = 5, 6
    H = g.standard_normal((off[-1], d))
    Wk, Wv, P = g.standard_normal((d, d)), g.standard_normal((d, d)), g.standard_normal((k, d))
    mask = (g.random(off[-1]) > 0.3).astype(np.uint8)
    Sbar = normalised_rows_batch(H, off, Wk, P, mask)
    S, _ = sketch_batch(H, off, Wk, Wv, P, mask)
    np.testing.assert_allclose(Sbar @ Wv, S, rtol=1e-12, atol=1e-13)
    assert not Sbar[1].any()
    # one token: every prototype's weighted mean is that token's row
    i = int(off[2])
    if mask[i]:
        np.testing.assert_allclose(Sbar[2], np.tile(H[i], (k, 1)), rtol=1e-13)
