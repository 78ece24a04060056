"""Pins of the oracle's layer (CPU only).

What pins what:
  * selection: a brute-force sort with explicit (key desc, id asc) tuples;
    special cases (all keys equal, k = E, k = 1); the identity "softmax over
    the top-k = renormalised full softmax"; a selection-only bias leaves the
    weights unchanged whenever it leaves the selection unchanged.
  * permutation: a pure-Python counting sort, plus the invariant checker.
  * routed sum: brute-force dense evaluation of every expert on every token,
    masked by the top-k weights (a different algorithm than the routed
    oracle: no permutation, no grouping).
  * expert formula: with all experts identical, the layer must equal one dense
    SwiGLU MLP built from torch's own silu and float64 matmuls.
  * the pages' size arithmetic (tests/golden/page_sizes.json): expert
    parameter counts and MXFP4 bytes.
  * planted mistakes in the oracle must fail at least one pin.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from oracle import layer as OL
from oracle import checks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_topk(L, k, bias=None, score="softmax"):
    L = np.asarray(L, dtype=np.float32)
    T, E = L.shape
    ids = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        keys = []
        for e in range(E):
            base = np.float32(L[t, e])
            if score == "sigmoid":   # torch's sigmoid in float64, rounded to float32
                base = np.float32(torch.sigmoid(torch.tensor(float(L[t, e]), dtype=torch.float64)).item())
            key = base + (np.float32(0) if bias is None else np.float32(bias[e]))
            key = float(np.float32(key))
            keys.append((-key if key != 0 else 0.0, e))
        keys.sort()
        ids[t] = [e for _, e in keys[:k]]
    return ids


def test_select_topk_matches_brute_force(syngen):
    rng = np.random.default_rng(0)
    for T, E, k in [(40, 8, 2), (20, 64, 8), (10, 384, 8), (5, 7, 7)]:
        L = rng.standard_normal((T, E)).astype(np.float32)
        ids, w = OL.select_topk(L, k)
        assert np.array_equal(ids, _brute_topk(L, k))
        checks.check_routing(ids, w, E)
    # many exact ties, including -0 and +0, and a tied bias
    L = syngen.tie_logits(50, 32)
    b = np.where(np.arange(32) % 3 == 0, np.float32(0.25), np.float32(0)).astype(np.float32)
    for bias in (None, b):
        ids, w = OL.select_topk(L, 8, bias)
        assert np.array_equal(ids, _brute_topk(L, 8, bias))


def test_sigmoid_select_topk_matches_brute_force(syngen):
    rng = np.random.default_rng(5)
    for T, E, k in [(30, 8, 2), (12, 64, 8), (6, 384, 8)]:
        L = (2 * rng.standard_normal((T, E))).astype(np.float32)
        for bias in (None, (0.05 * rng.standard_normal(E)).astype(np.float32)):
            ids, w = OL.select_topk(L, k, bias, "sigmoid")
            assert np.array_equal(ids, _brute_topk(L, k, bias, "sigmoid"))
            checks.check_routing(ids, w, E)
            # weights: the selected sigmoid scores over their sum (torch's sigmoid)
            s = torch.sigmoid(torch.from_numpy(np.take_along_axis(L, ids, 1).astype(np.float64))).numpy()
            assert np.allclose(w, s / s.sum(1, keepdims=True), rtol=1e-14, atol=0)
    # ties (equal logits, -0/+0) go to the lower id
    L = syngen.tie_logits(40, 32)
    ids, _ = OL.select_topk(L, 8, None, "sigmoid")
    assert np.array_equal(ids, _brute_topk(L, 8, None, "sigmoid"))


def test_sigmoid_without_bias_selects_like_softmax():
    # the sigmoid is increasing: without a bias both scorings pick the same experts
    # (logits on a grid far coarser than float32 spacing, so no two scores collide)
    rng = np.random.default_rng(6)
    L = (rng.permuted(np.tile(np.arange(64), (20, 1)), axis=1) * 0.05 - 1.6).astype(np.float32)
    ids_s, w_s = OL.select_topk(L, 8, None, "sigmoid")
    ids_m, w_m = OL.select_topk(L, 8)
    assert np.array_equal(ids_s, ids_m)
    assert not np.allclose(w_s, w_m)   # the weights differ


def test_select_topk_special_cases():
    L = np.full((3, 16), 0.7, dtype=np.float32)
    ids, w = OL.select_topk(L, 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 3 and np.allclose(w, 0.25, atol=0, rtol=1e-15)
    L = np.random.default_rng(1).standard_normal((4, 9)).astype(np.float32)
    ids, w = OL.select_topk(L, 9)                       # k = E: every expert, full softmax
    full = torch.softmax(torch.from_numpy(L.astype(np.float64)), dim=1).numpy()
    assert np.allclose(np.take_along_axis(full, ids, 1), w, rtol=1e-14, atol=0)
    ids1, w1 = OL.select_topk(L, 1)
    assert np.all(w1 == 1.0) and np.array_equal(ids1[:, 0], np.argmax(L, axis=1))
    # top-k softmax = full softmax restricted to the top k, renormalised
    idsk, wk = OL.select_topk(L, 3)
    sub = np.take_along_axis(full, idsk, 1)
    assert np.allclose(sub / sub.sum(1, keepdims=True), wk, rtol=1e-13, atol=0)


def test_selection_bias_does_not_enter_weights():
    rng = np.random.default_rng(2)
    L = rng.standard_normal((64, 32)).astype(np.float32)
    ids0, w0 = OL.select_topk(L, 4)
    bias = np.zeros(32, dtype=np.float32)
    bias[ids0[0, 0]] = 1e-3          # nudges one selected key; selection of token 0 unchanged
    ids1, w1 = OL.select_topk(L, 4, bias)
    same = np.all(ids1 == ids0, axis=1)
    assert same[0] and same.sum() >= 60
    assert np.array_equal(w1[same], w0[same])
    # a large bias moves the selection
    big = np.zeros(32, dtype=np.float32)
    big[31] = 100.0
    ids2, _ = OL.select_topk(L, 4, big)
    assert np.all(ids2[:, 0] == 31)
    # the same with sigmoid scores
    s0, v0 = OL.select_topk(L, 4, None, "sigmoid")
    s1, v1 = OL.select_topk(L, 4, bias, "sigmoid")
    same = np.all(s1 == s0, axis=1)
    assert same.sum() >= 60 and np.array_equal(v1[same], v0[same])
    s2, _ = OL.select_topk(L, 4, big, "sigmoid")
    assert np.all(s2[:, 0] == 31)


def _counting_sort(ids, E):
    T, k = ids.shape
    buckets = [[] for _ in range(E)]
    for s in range(T * k):
        buckets[int(ids[s // k, s % k])].append(s)
    rows = [s for b in buckets for s in b]
    off = [0]
    for b in buckets:
        off.append(off[-1] + len(b))
    ros = [0] * (T * k)
    for r, s in enumerate(rows):
        ros[s] = r
    return off, [s // k for s in rows], ros


def test_permutation_matches_counting_sort(syngen):
    for T, E, k, skew in [(64, 8, 2, None), (37, 64, 8, None), (100, 32, 4, 3.0), (1, 8, 8, None)]:
        ids = syngen.random_ids(T, E, k, seed=T, skew=skew)
        p = OL.permutation(ids, E)
        off, st, ros = _counting_sort(ids, E)
        assert p["offsets"].tolist() == off
        assert p["sorted_token"].tolist() == st
        assert p["row_of_slot"].tolist() == ros
        checks.check_permutation(ids, p["offsets"], p["sorted_token"], p["row_of_slot"])


def test_permutation_checker_rejects_mutations(syngen):
    ids = syngen.random_ids(20, 8, 2, seed=3)
    p = OL.permutation(ids, 8)
    ros = p["row_of_slot"].copy()
    e = int(ids[0, 0])
    r0 = int(p["offsets"][e])
    # swap the first two rows of expert e: breaks stability
    a, b = np.flatnonzero(ros == r0)[0], np.flatnonzero(ros == r0 + 1)[0]
    ros[a], ros[b] = ros[b], ros[a]
    st = p["sorted_token"].copy()
    st[r0], st[r0 + 1] = st[r0 + 1], st[r0]
    with pytest.raises(AssertionError):
        checks.check_permutation(ids, p["offsets"], st, ros)
    off = p["offsets"].copy()
    off[3] += 1
    with pytest.raises(AssertionError):
        checks.check_permutation(ids, off, p["sorted_token"], p["row_of_slot"])


def _dense_bruteforce(layer):
    """Every expert on every token, masked by the top-k weights; no grouping."""
    x = layer["x"]
    T, H = x.shape
    E = layer["w13"].shape[0]
    k = layer["top_k"]
    L = (F.decode_bf16(x) @ F.decode_bf16(layer["w_router"]).T).astype(np.float32)
    score = layer.get("score", "softmax")
    ids = _brute_topk(L, k, layer.get("bias"), score)
    mask = np.zeros((T, E))
    for t in range(T):
        sel = L[t, ids[t]].astype(np.float64)
        p = torch.sigmoid(torch.from_numpy(sel)).numpy() if score == "sigmoid" else np.exp(sel - sel.max())
        mask[t, ids[t]] = p / p.sum()
    xq, xs = F.quantize_fp8_blocks(F.decode_bf16(x))
    a = F.dequantize_fp8_blocks(xq, xs)
    inter = layer["w13"].shape[1] // 2
    y = np.zeros((T, H))
    for e in range(E):
        w13 = F.decode_mxfp4(layer["w13"][e], layer["w13_s"][e])
        w2 = F.decode_mxfp4(layer["w2"][e], layer["w2_s"][e])
        g = a @ w13[:inter].T
        u = a @ w13[inter:].T
        h = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u
        hq, hs = F.quantize_fp8_blocks(h)
        ye = F.dequantize_fp8_blocks(hq, hs) @ w2.T
        y += mask[:, e:e + 1] * ye
    return y


@pytest.mark.parametrize("over", [{}, dict(T=13, E=16, k=4), dict(T=9, E=6, k=6, H=128, I=256)])
def test_routed_oracle_equals_dense_bruteforce(syngen, over):
    layer = syngen.make_layer("tiny", seed=1, **over)
    ref = _dense_bruteforce(layer)
    out = OL.forward(layer)
    scale = np.abs(ref).max()
    assert np.max(np.abs(out["y"] - ref)) <= 1e-12 * scale
    checks.check_routing(out["ids"], out["w"], layer["w13"].shape[0])
    checks.check_permutation(out["ids"], out["offsets"], out["sorted_token"], out["row_of_slot"])
    checks.check_fp8_blocks(out["xq"], out["xs"])
    checks.check_fp8_blocks(out["hq_perm"], out["hs_perm"])


def test_routed_oracle_with_sigmoid_scores_equals_dense_bruteforce(syngen):
    for bias in ("zero", "zipf"):
        layer = syngen.make_layer("tiny", seed=7, T=30, E=16, k=4, bias=bias)
        layer["score"] = "sigmoid"
        ref = _dense_bruteforce(layer)
        out = OL.forward(layer)
        assert np.max(np.abs(out["y"] - ref)) <= 1e-12 * np.abs(ref).max()
        toks = np.array([0, 7, 29])
        assert np.max(np.abs(OL.forward_tokens(layer, toks)["y"] - out["y"][toks])) <= 1e-12 * np.abs(ref).max()


def test_routed_oracle_with_zipf_bias_equals_dense_bruteforce(syngen):
    layer = syngen.make_layer("tiny", seed=2, T=40, E=32, k=4, bias="zipf")
    ref = _dense_bruteforce(layer)
    out = OL.forward(layer)
    assert np.max(np.abs(out["y"] - ref)) <= 1e-12 * np.abs(ref).max()


def _dense_swiglu_mlp(x_bits, w13, w13_s, w2, w2_s):
    """One dense SwiGLU MLP with FP8 activations, from torch's silu and float64 matmuls."""
    xq, xs = F.quantize_fp8_blocks(F.decode_bf16(x_bits))
    a = torch.from_numpy(F.dequantize_fp8_blocks(xq, xs))
    wg_wu = torch.from_numpy(F.decode_mxfp4(w13, w13_s))
    inter = wg_wu.shape[0] // 2
    gate, up = wg_wu[:inter], wg_wu[inter:]
    h = torch.nn.functional.silu(a @ gate.T) * (a @ up.T)
    hq, hs = F.quantize_fp8_blocks(h.numpy())
    w_down = torch.from_numpy(F.decode_mxfp4(w2, w2_s))
    return (torch.from_numpy(F.dequantize_fp8_blocks(hq, hs)) @ w_down.T).numpy()


def test_identical_experts_equal_one_dense_mlp(syngen):
    layer = syngen.make_layer("tiny", seed=3)
    for key in ("w13", "w13_s", "w2", "w2_s"):
        layer[key] = np.repeat(layer[key][:1], layer[key].shape[0], axis=0)
    out = OL.forward(layer)
    ref = _dense_swiglu_mlp(layer["x"], layer["w13"][0], layer["w13_s"][0], layer["w2"][0], layer["w2_s"][0])
    assert np.max(np.abs(out["y"] - ref)) <= 1e-12 * np.abs(ref).max()


def test_forward_tokens_equals_forward(syngen):
    layer = syngen.make_layer("tiny", seed=4, bias="zipf")
    full = OL.forward(layer)
    toks = np.array([0, 5, 17, 63])
    part = OL.forward_tokens(layer, toks)
    assert np.array_equal(part["ids"], full["ids"][toks])
    assert np.max(np.abs(part["y"] - full["y"][toks])) <= 1e-13 * np.abs(full["y"]).max()


# --- planted mistakes: each must break at least one pin --------------------

def _mutants():
    def silu_identity(z):
        return z

    def gate_up_swapped(a, w13_e, w13_s_e, w2_e, w2_s_e, fmt="mxfp4"):
        inter = w13_e.shape[0] // 2
        sw = np.concatenate([w13_e[inter:], w13_e[:inter]])
        sws = np.concatenate([w13_s_e[inter:], w13_s_e[:inter]])
        return _orig_ffn(a, sw, sws, w2_e, w2_s_e, fmt)

    def no_h_quant(a, w13_e, w13_s_e, w2_e, w2_s_e, fmt="mxfp4"):
        out = _orig_ffn(a, w13_e, w13_s_e, w2_e, w2_s_e, fmt)
        out["y"] = out["h"] @ OL.decode_expert_matrix(w2_e, w2_s_e, fmt).T
        return out

    def biased_softmax(logits, k, bias=None, score="softmax"):
        L = np.asarray(logits, dtype=np.float32)
        key = L if bias is None else L + np.asarray(bias, dtype=np.float32)
        return _orig_select(key, k, None, score)

    def nibbles_swapped(packed):
        p = np.asarray(packed, dtype=np.uint8)
        return _orig_unpack(((p & 15) << 4) | (p >> 4))

    return [("silu", "_silu", silu_identity, OL), ("gate_up", "expert_ffn", gate_up_swapped, OL),
            ("hquant", "expert_ffn", no_h_quant, OL), ("bias", "select_topk", biased_softmax, OL),
            ("nibble", "unpack_fp4", nibbles_swapped, F)]


_orig_ffn = OL.expert_ffn
_orig_select = OL.select_topk
_orig_unpack = F.unpack_fp4


def _pins_pass(syngen):
    try:
        test_identical_experts_equal_one_dense_mlp(syngen)
        test_selection_bias_does_not_enter_weights()
        test_mxfp4_nibble_pin()
        layer = syngen.make_layer("tiny", seed=2, T=24, E=16, k=4, bias="zipf")
        ref = _dense_bruteforce(layer)
        out = OL.forward(layer)
        assert np.max(np.abs(out["y"] - ref)) <= 1e-12 * np.abs(ref).max()
    except AssertionError:
        return False
    return True


def test_mxfp4_nibble_pin():
    # element 0 of a row is the low nibble of byte 0 (the reading of two e2m1 values per byte)
    v = F.decode_mxfp4(np.array([[0x71] + [0] * 15], dtype=np.uint8), np.array([[127]], dtype=np.uint8))
    assert v[0, 0] == 0.5 and v[0, 1] == 6.0


@pytest.mark.parametrize("name", ["silu", "gate_up", "hquant", "bias", "nibble"])
def test_planted_mistakes_are_caught(syngen, monkeypatch, name):
    assert _pins_pass(syngen)
    for nm, attr, fn, mod in _mutants():
        if nm == name:
            monkeypatch.setattr(mod, attr, fn)
    assert not _pins_pass(syngen), "planted mistake %r went unnoticed" % name


# --- the pages' size arithmetic ---------------------------------------------

def _rounds_to(x, printed, unit):
    return abs(round(x / unit) * unit - printed) < unit / 2


def test_page_size_arithmetic(syngen):
    g = json.load(open(os.path.join(GOLDEN, "page_sizes.json")))
    inter = g["middle_width"]["value"]
    for model, H, E in [("flash", g["flash_hidden"]["value"], g["flash_experts"]["value"]),
                        ("pro", g["pro_hidden"]["value"], g["pro_experts"]["value"])]:
        cfg = syngen.config({"flash": "flash_decode", "pro": "pro_decode"}[model])
        assert (cfg["H"], cfg["E"], cfg["I"]) == (H, E, inter)
        # parameters of one expert as the oracle lays it out: W13 [2I, H] and W2 [H, I]
        params = 2 * inter * H + H * inter
        assert _rounds_to(params, g[model + "_expert_params"]["value"], g[model + "_expert_params"]["round_to"])
        # bytes: codes (two per byte) + one scale byte per 32 values
        w13_bytes = 2 * inter * (H // 2 + H // 32)
        w2_bytes = H * (inter // 2 + inter // 32)
        assert (w13_bytes + w2_bytes) * 8 / params == g["bits_per_expert_weight"]["value"]
    flash_params = 2 * inter * 4096 + 4096 * inter
    moe_layers = g["flash_layers"]["value"] - g["flash_layers"]["dense_ffn_layers"]
    total = moe_layers * g["flash_experts"]["value"] * flash_params
    assert _rounds_to(total, g["flash_expert_weights"]["value"], g["flash_expert_weights"]["round_to"])
    assert _rounds_to(total * 4.25 / 8, g["flash_expert_bytes"]["value"], g["flash_expert_bytes"]["round_to"])
    # the generator lays tensors out with the same shapes
    lay = syngen.make_layer("tiny")
    H, E, inter_t = 256, 8, 128
    assert lay["w13"].shape == (E, 2 * inter_t, H // 2) and lay["w13_s"].shape == (E, 2 * inter_t, H // 32)
    assert lay["w2"].shape == (E, H, inter_t // 2) and lay["w2_s"].shape == (E, H, inter_t // 32)
