"""Pins of the oracle's routing (oracle/moe.py: route).

Selection is checked by brute force over all C(E, k) subsets with exact
rational sums; the weights against closed forms (k = 1, k = E softmax) and
invariants (sum to 1, relabelling, shift)."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import route


def _brute_select(l, k):
    """Max-sum k-subset of the logits, exact; among equal sums the
    lexicographically smallest sorted tuple (= lowest index wins ties)."""
    best = None
    for sub in itertools.combinations(range(len(l)), k):
        s = sum(Fraction(float(l[e])) for e in sub)
        if best is None or s > best[0] or (s == best[0] and sub < best[1]):
            best = (s, sub)
    return set(best[1])


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (6, 3), (8, 2), (10, 4), (7, 7)])
def test_selection_is_max_sum_subset(E, k):
    rng = np.random.default_rng(E * 100 + k)
    for trial in range(40):
        if trial % 2:
            l = rng.standard_normal(E).astype(np.float32)
        else:                                   # coarse grid: many exact ties
            l = (rng.integers(-3, 4, E) / 2.0).astype(np.float32)
        idx, w = route(l[None, :], k)
        assert set(idx[0].tolist()) == _brute_select(l, k)
        # slot order: logit descending, then index ascending
        keys = [(-float(l[e]), int(e)) for e in idx[0]]
        assert keys == sorted(keys)
        assert np.all(np.diff(w[0]) <= 0)


def test_hand_built_ties():
    assert route(np.array([[1, 1, 0]], np.float32), 1)[0].tolist() == [[0]]
    assert route(np.array([[0, 1, 0, 1, 0]], np.float32), 3)[0].tolist() == [[1, 3, 0]]
    # +0 and -0 compare equal: the lower index wins either way round
    assert route(np.array([[-0.0, 0.0, -1]], np.float32), 1)[0].tolist() == [[0]]
    assert route(np.array([[0.0, -0.0, -1]], np.float32), 1)[0].tolist() == [[0]]
    assert route(np.array([[-1, -0.0, 0.0]], np.float32), 2)[0].tolist() == [[1, 2]]
    # all equal: the first k indices, equal weights
    idx, w = route(np.zeros((1, 6), np.float32), 4)
    assert idx.tolist() == [[0, 1, 2, 3]] and np.all(w == 0.25)


def test_nonfinite_rejected():
    with pytest.raises(ValueError):
        route(np.array([[0, np.nan, 1]], np.float32), 1)
    with pytest.raises(ValueError):
        route(np.array([[0, np.inf, 1]], np.float32), 1)
    with pytest.raises(ValueError):
        route(np.zeros((1, 3), np.float32), 4)


def test_weights_sum_to_one_and_k1_exact():
    rng = np.random.default_rng(0)
    for k in (1, 2, 8, 10):
        l = rng.standard_normal((500, 64)).astype(np.float32) * 3
        idx, w = route(l, k)
        assert np.all(np.abs(w.sum(1) - 1.0) <= 4 * k * 2.0 ** -53)
        if k == 1:
            assert np.all(w == 1.0)


def test_k_equals_E_is_softmax_over_all_experts():
    rng = np.random.default_rng(1)
    l = rng.standard_normal((200, 16)).astype(np.float32) * 2
    idx, w = route(l, 16)
    ld = l.astype(np.float64)
    sm = np.exp(ld - ld.max(1, keepdims=True))
    sm /= sm.sum(1, keepdims=True)
    assert np.allclose(w, np.take_along_axis(sm, idx, 1), rtol=1e-14, atol=0)


def test_relabelling_invariance_bitwise():
    rng = np.random.default_rng(2)
    E, k = 32, 6
    l = rng.standard_normal((300, E)).astype(np.float32)
    perm = rng.permutation(E)             # new column c holds old expert perm[c]
    idx, w = route(l, k)
    idx2, w2 = route(l[:, perm], k)
    assert np.array_equal(perm[idx2], idx)
    assert np.array_equal(w2.view(np.uint64), w.view(np.uint64))


def test_shift_invariance_on_exact_grid():
    rng = np.random.default_rng(4)
    l = (rng.integers(-64, 64, (100, 20)) / 16.0).astype(np.float32)  # exact sums
    idx, w = route(l, 5)
    idx2, w2 = route(l + np.float32(3.0), 5)
    assert np.array_equal(idx, idx2)
    assert np.allclose(w, w2, rtol=1e-15, atol=0)
