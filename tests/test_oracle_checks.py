"""Pins of the routing checkers in oracle/checks.py (CPU only).

The GPU tests use ``check_routing`` and ``topk_is_valid`` as validity
checkers where several results are correct (top-k decisions within the
logit uncertainty of a tie).  A checker that accepted everything would let
every such test pass, so each one is pinned here two ways:
  * it accepts what the definition of routing fixes as correct: the top-k of
    a brute-force tuple sort, any order of equal keys within the tolerance,
    softmax weights over the selected logits;
  * it rejects planted mistakes, one property at a time: a non-top-k id, a
    duplicate id, an id out of range, a negative weight, weights that do not
    sum to 1.
"""

import itertools

import numpy as np
import pytest

from oracle import checks


def _brute_topk(keys, k):
    """Top-k of each row by a plain tuple sort: largest key first, lower id on ties."""
    out = []
    for row in keys:
        order = sorted(range(len(row)), key=lambda e: (-row[e], e))
        out.append(order[:k])
    return np.array(out, dtype=np.int32)


def _softmax_rows(L, ids):
    sel = np.take_along_axis(L, ids.astype(np.int64), 1)
    z = np.exp(sel - sel.max(1, keepdims=True))
    return z / z.sum(1, keepdims=True)


@pytest.fixture
def routed():
    rng = np.random.default_rng(5)
    T, E, k = 40, 16, 4
    L = rng.normal(size=(T, E))
    ids = _brute_topk(L, k)
    return L, ids, _softmax_rows(L, ids), E, k


# --- check_routing ----------------------------------------------------------
def test_check_routing_accepts_a_correct_routing(routed):
    L, ids, w, E, k = routed
    checks.check_routing(ids, w, E)
    # k == E (every expert, any order) and k == 1 (weight 1)
    full = np.argsort(-L, axis=1, kind="stable").astype(np.int32)
    checks.check_routing(full, _softmax_rows(L, full), E)
    checks.check_routing(ids[:, :1], np.ones((ids.shape[0], 1)), E)


@pytest.mark.parametrize("mutation", ["duplicate", "out_of_range_high", "out_of_range_negative",
                                      "weights_sum_1.01", "negative_weight", "weight_shape"])
def test_check_routing_rejects_planted_mistakes(routed, mutation):
    L, ids, w, E, k = routed
    ids, w = ids.copy(), w.copy()
    t = 7
    if mutation == "duplicate":
        ids[t, 2] = ids[t, 0]
    elif mutation == "out_of_range_high":
        ids[t, 1] = E
    elif mutation == "out_of_range_negative":
        ids[t, 3] = -1
    elif mutation == "weights_sum_1.01":
        w[t] *= 1.01
    elif mutation == "negative_weight":
        w[t, 0], w[t, 1] = -w[t, 0], w[t, 1] + 2 * w[t, 0]   # still sums to 1
    elif mutation == "weight_shape":
        w = w[:, :-1]
    with pytest.raises(AssertionError):
        checks.check_routing(ids, w, E)


def test_check_routing_tolerance_is_the_stated_one(routed):
    """Weights summing to 1 within 1e-6 pass; 1 + 1e-5 does not."""
    L, ids, w, E, k = routed
    w = w.copy()
    w[3] *= 1 + 5e-7
    checks.check_routing(ids, w, E)
    w[3] *= 1 + 1e-5
    with pytest.raises(AssertionError):
        checks.check_routing(ids, w, E)


# --- topk_is_valid ----------------------------------------------------------
def test_topk_is_valid_accepts_the_brute_force_top_k(routed):
    L, ids, w, E, k = routed
    assert checks.topk_is_valid(ids, L, 0.0).all()
    # the chosen set in any order is still a valid top-k
    assert checks.topk_is_valid(ids[:, ::-1].copy(), L, 0.0).all()


def test_topk_is_valid_rejects_a_non_top_k_id(routed):
    L, ids, w, E, k = routed
    bad = ids.copy()
    T = L.shape[0]
    for t in range(T):
        # swap the k-th choice for the smallest key of the row
        bad[t, k - 1] = int(np.argmin(L[t]))
    ok = checks.topk_is_valid(bad, L, 0.0)
    assert not ok.any()
    # only the mutated token is flagged when one row is changed
    one = ids.copy()
    one[11, 0] = int(np.argmin(L[11]))
    ok = checks.topk_is_valid(one, L, 0.0)
    assert not ok[11] and ok[np.arange(T) != 11].all()


def test_topk_is_valid_rejects_a_duplicate_id(routed):
    L, ids, w, E, k = routed
    bad = ids.copy()
    bad[4, 1] = bad[4, 0]
    ok = checks.topk_is_valid(bad, L, 0.0)
    assert not ok[4] and ok[np.arange(len(ok)) != 4].all()


def test_topk_is_valid_uses_the_tolerance_both_ways():
    """A near-tie (gap 1e-4 between the k-th and (k+1)-th key) may go either way
    within a tolerance of 1e-4; a gap of 1e-2 may not."""
    keys = np.array([[3.0, 2.0, 1.0, 1.0 - 1e-4, 0.0],
                     [3.0, 2.0, 1.0, 1.0 - 1e-2, 0.0]])
    swapped = np.array([[0, 1, 3], [0, 1, 3]], dtype=np.int32)
    exact = np.array([[0, 1, 2], [0, 1, 2]], dtype=np.int32)
    assert checks.topk_is_valid(exact, keys, 1e-4).all()
    ok = checks.topk_is_valid(swapped, keys, np.array([1e-4, 1e-4]))
    assert ok[0] and not ok[1]
    # with no tolerance the swap is wrong in both rows
    assert not checks.topk_is_valid(swapped, keys, 0.0).any()


def test_topk_is_valid_on_every_choice_of_a_tiny_row():
    """Brute force over all 3-subsets of 6 distinct keys: exactly one is valid at tolerance 0."""
    keys = np.array([[0.5, -1.0, 2.0, 0.0, 1.5, -0.25]])
    best = set(_brute_topk(keys, 3)[0].tolist())
    for sub in itertools.permutations(range(6), 3):
        ok = checks.topk_is_valid(np.array([sub], dtype=np.int32), keys, 0.0)[0]
        assert ok == (set(sub) == best), sub
