"""Pins of the oracle's load-balancing step for the selection bias
(oracle.layer.update_selection_bias; teardown "How Big Is Each Expert?": a
small per-expert correction bias keeps the load even, with no update formula
on the page).  The pins: hand-worked values, the cases where nothing may
change, the single float32 addition, and the property the rule exists for
(iterated on a skewed routing, it evens the load; stepped the wrong way, it
makes the load worse)."""

import numpy as np
import pytest

from oracle import layer as OL


def test_hand_worked_step():
    # loads 10, 2, 6, 6 over 4 experts: mean 6 -> above, below, at, at
    b = OL.update_selection_bias([0, 10, 12, 18, 24], 0.25, np.full(4, 0.5, np.float32))
    assert b.dtype == np.float32
    assert b.tolist() == [0.25, 0.75, 0.5, 0.5]
    # offsets need not start at 0: only the differences and the total count
    b = OL.update_selection_bias([100, 110, 112, 118, 124], 0.25, np.full(4, 0.5, np.float32))
    assert b.tolist() == [0.25, 0.75, 0.5, 0.5]


def test_mean_compared_exactly():
    # N = 10 over E = 3: mean 3.333..; loads 3, 3, 4 -> below, below, above
    b = OL.update_selection_bias([0, 3, 6, 10], 1.0, np.zeros(3, np.float32))
    assert b.tolist() == [1.0, 1.0, -1.0]
    # a load of exactly N / E keeps its bias even when N / E is not a float32-friendly value
    E = 7
    off = np.arange(E + 1) * 1_000_003
    b0 = np.linspace(-1, 1, E).astype(np.float32)
    assert np.array_equal(OL.update_selection_bias(off, 0.125, b0).view(np.uint32), b0.view(np.uint32))


def test_nothing_moves_without_a_step_or_an_imbalance():
    rng = np.random.default_rng(1)
    b0 = rng.normal(size=64).astype(np.float32)
    off = np.concatenate([[0], np.cumsum(rng.integers(0, 50, 64))])
    assert np.array_equal(OL.update_selection_bias(off, 0.0, b0).view(np.uint32), b0.view(np.uint32))
    even = np.arange(65) * 8
    assert np.array_equal(OL.update_selection_bias(even, 0.5, b0).view(np.uint32), b0.view(np.uint32))
    # no rows at all: every expert is at the mean (0)
    assert np.array_equal(OL.update_selection_bias(np.zeros(65, np.int64), 0.5, b0).view(np.uint32),
                          b0.view(np.uint32))


def test_one_float32_addition():
    # 1 + 2^-30 rounds back to 1 in float32 (a float64 update would keep it)
    b = OL.update_selection_bias([0, 0, 2], 2.0 ** -30, np.array([1.0, 1.0], np.float32))
    assert b.tolist() == [1.0, 1.0]
    b = OL.update_selection_bias([0, 0, 2], 2.0 ** -30, np.array([0.0, 0.0], np.float32))
    assert b.tolist() == [2.0 ** -30, -(2.0 ** -30)]
    # a step that is not a float32 value is used as its float32 rounding
    b = OL.update_selection_bias([0, 0, 2], 0.1, np.zeros(2, np.float32))
    assert b[0] == np.float32(0.1) and b[1] == -np.float32(0.1)


def test_rule_evens_out_a_skewed_load():
    rng = np.random.default_rng(7)
    T, E, k = 512, 16, 2
    logits = (rng.normal(size=(T, E)) + np.where(np.arange(E) < 2, 1.5, 0.0)).astype(np.float32)

    def ratio_after(steps, step):
        b = np.zeros(E, np.float32)
        for _ in range(steps):
            ids, _ = OL.select_topk(logits, k, b, score="sigmoid")
            c = np.bincount(ids.ravel(), minlength=E)
            b = OL.update_selection_bias(np.concatenate([[0], np.cumsum(c)]), step, b)
        ids, _ = OL.select_topk(logits, k, b, score="sigmoid")
        c = np.bincount(ids.ravel(), minlength=E)
        return c.max() / c.mean()

    start = ratio_after(0, 0.01)
    assert start > 3.5
    assert ratio_after(60, 0.01) < 1.2          # the rule evens the load out
    assert ratio_after(60, -0.01) > start       # the other sign concentrates it further


def test_rejects_no_experts():
    with pytest.raises(ValueError):
        OL.update_selection_bias([0], 0.1, np.zeros(0, np.float32))
