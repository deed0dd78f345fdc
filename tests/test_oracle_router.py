"""Pins of the oracle's router and top-k selection (reading R9).

The oracle ranks every group against every other one with explicit loops.  Here
the selection is checked against a stable-sort library routine (np.lexsort) and
against the seeded input generator's own top-k (separate code), on rows full of
ties; against special cases (all equal, signed zeros, k = 0, k = n); and the
logits against linearity and a closed form.
"""
import itertools

import numpy as np
import pytest

import synth
from oracle import router_topk


def _lexsort_topk(L, k):
    T, n = L.shape
    m = np.zeros((T, n), np.uint8)
    for t in range(T):
        order = np.lexsort((np.arange(n), -L[t]))  # primary: larger logit; then lower index
        m[t, order[:k]] = 1
    return m


@pytest.mark.parametrize("n,k", [(8, 4), (16, 8), (112, 56), (5, 1), (70, 69)])
def test_selection_matches_stable_sort(n, k):
    rng = np.random.default_rng(n * 131 + k)
    L = rng.integers(-3, 4, size=(40, n)).astype(np.float64)  # many ties
    out = router_topk(None, None, k, logits=L)
    np.testing.assert_array_equal(out["mask"], _lexsort_topk(L, k))
    np.testing.assert_array_equal(out["mask"], synth.topk_mask(L, k))
    assert np.all(out["mask"].sum(axis=1) == k)


def test_selection_brute_force_small():
    # every logit row over {0, 1, 2}^4 and every k: the kept set is the one whose
    # members all rank before every non-member
    n = 4
    for row in itertools.product([0.0, 1.0, 2.0], repeat=n):
        L = np.array([row])
        for k in range(n + 1):
            m = router_topk(None, None, k, logits=L)["mask"][0]
            kept = [g for g in range(n) if m[g]]
            assert len(kept) == k
            for a in kept:
                for b in range(n):
                    if b not in kept:
                        assert row[a] > row[b] or (row[a] == row[b] and a < b)


def test_special_cases():
    n = 10
    eq = np.full((3, n), 0.25)
    np.testing.assert_array_equal(router_topk(None, None, 3, logits=eq)["mask"],
                                  np.tile((np.arange(n) < 3).astype(np.uint8), (3, 1)))
    z = np.array([[-0.0, 0.0, -0.0, 0.0]])
    np.testing.assert_array_equal(router_topk(None, None, 2, logits=z)["mask"], [[1, 1, 0, 0]])
    L = np.random.default_rng(1).standard_normal((6, n))
    assert router_topk(None, None, 0, logits=L)["mask"].sum() == 0
    assert router_topk(None, None, n, logits=L)["mask"].min() == 1
    with pytest.raises(ValueError):
        router_topk(None, None, n + 1, logits=L)


def test_packed_words_follow_the_mask():
    rng = np.random.default_rng(7)
    L = rng.standard_normal((9, 130))
    out = router_topk(None, None, 65, logits=L)
    pad = np.zeros((9, 192), np.uint8)
    pad[:, :130] = out["mask"]
    ref = np.packbits(pad, axis=1, bitorder="little").view("<u8").reshape(9, 3)
    np.testing.assert_array_equal(out["packed"], ref)


def test_logits_linear_and_closed_form():
    rng = np.random.default_rng(3)
    d, n = 12, 5
    X1, X2 = rng.standard_normal((4, d)), rng.standard_normal((4, d))
    R = rng.standard_normal((n, d))
    L1, L2 = router_topk(X1, R, 2)["logits"], router_topk(X2, R, 2)["logits"]
    np.testing.assert_allclose(router_topk(X1 + X2, R, 2)["logits"], L1 + L2, rtol=1e-12, atol=1e-12)
    E = np.eye(n, d)  # group g reads input feature g
    np.testing.assert_array_equal(router_topk(X1, E, 2)["logits"], X1[:, :n])
