"""Invariant checkers for routing, permutation and FP8 blocks.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Each checker raises AssertionError with a message naming the first violated
property.  They state what any correct result must satisfy, so they apply
equally to the oracle's results and to results computed elsewhere.
"""

import numpy as np

from . import formats as F

__all__ = ["check_routing", "check_permutation", "check_fp8_blocks", "topk_is_valid"]


def check_routing(ids, w, num_experts, atol=1e-6):
    """Ids in range and distinct per token; weights non-negative and summing to 1."""
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    T, k = ids.shape
    assert w.shape == (T, k), "weights shape"
    assert ids.min(initial=0) >= 0 and ids.max(initial=0) < num_experts, "expert id out of range"
    s = np.sort(ids, axis=1)
    assert not np.any(s[:, 1:] == s[:, :-1]), "an expert appears twice for one token"
    assert np.all(w >= 0), "negative combine weight"
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=atol), "combine weights do not sum to 1"


def check_permutation(ids, offsets, sorted_token, row_of_slot):
    """The expert-grouped permutation of the T*k slots is complete, grouped and stable."""
    ids = np.asarray(ids).astype(np.int64)
    T, k = ids.shape
    n = T * k
    off = np.asarray(offsets).astype(np.int64)
    st = np.asarray(sorted_token).astype(np.int64)
    ros = np.asarray(row_of_slot).astype(np.int64)
    E = off.size - 1
    assert off[0] == 0 and off[-1] == n, "offsets must run from 0 to T*k"
    assert np.all(np.diff(off) >= 0), "offsets must be non-decreasing"
    counts = np.diff(off)
    assert counts.sum() == n, "counts must sum to T*k"
    assert np.array_equal(counts, np.bincount(ids.reshape(-1), minlength=E)[:E]), \
        "counts disagree with the expert ids"
    assert st.shape == (n,) and ros.shape == (n,), "permutation array shapes"
    assert np.array_equal(np.sort(ros), np.arange(n)), "row_of_slot is not a bijection"
    slot = np.arange(n)
    e_of_slot = ids.reshape(-1)
    assert np.all(st[ros] == slot // k), "sorted_token does not invert row_of_slot"
    assert np.all((ros >= off[e_of_slot]) & (ros < off[e_of_slot + 1])), \
        "a slot landed outside its expert's row range"
    # stability: within each expert, rows are in ascending slot order
    slot_of_row = np.empty(n, dtype=np.int64)
    slot_of_row[ros] = slot
    for e in range(E):
        seg = slot_of_row[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0), "rows of one expert are not in ascending token order"
    # every token appears in exactly k slots
    assert np.array_equal(np.bincount(st, minlength=T), np.full(T, k)), \
        "a token does not appear in exactly k rows"


def check_fp8_blocks(codes, scales, block=F.FP8_BLOCK):
    """Codes finite; in every non-zero block the largest |code value| lies in [224, 448].

    Before rounding, the scaled block maximum lies in (224, 448]; rounding to
    the e4m3 grid (spacing 16 in [128, 256)) can bring it down to 224 exactly.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    R, C = codes.shape
    v = F.decode_e4m3(codes)
    assert not np.any(np.isnan(v)), "NaN code"
    bmax = np.abs(v).reshape(R, C // block, block).max(axis=-1)
    nz = bmax > 0
    assert np.all((bmax[nz] >= 224) & (bmax[nz] <= 448)), "block maximum outside [224, 448]"
    assert np.asarray(scales).shape == (R, C // block), "scale shape"


def topk_is_valid(ids, keys, tol):
    """True where the chosen ids are *a* correct top-k under key uncertainty `tol`.

    Valid means: distinct ids, and every chosen key is >= every unchosen key
    minus 2*tol (so no unchosen key is certainly larger).  Returns a [T] bool array.
    """
    ids = np.asarray(ids).astype(np.int64)
    keys = np.asarray(keys, dtype=np.float64)
    T, E = keys.shape
    chosen = np.zeros((T, E), dtype=bool)
    np.put_along_axis(chosen, ids, True, axis=1)
    distinct = chosen.sum(axis=1) == ids.shape[1]
    min_chosen = np.where(chosen, keys, np.inf).min(axis=1)
    max_other = np.where(chosen, -np.inf, keys).max(axis=1)
    tol = np.broadcast_to(np.asarray(tol, dtype=np.float64), (T,))
    return distinct & (min_chosen >= max_other - 2 * tol)
