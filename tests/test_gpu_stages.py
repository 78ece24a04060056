"""GPU parity of each stage of the layer against the oracle, through the C ABI.

Each stage is fed seeded synthetic inputs (never another stage's GPU output)
and compared with the oracle on the same inputs, at sizes the oracle
finishes in seconds that still span several tiles and ragged tails.
Bars are in tests/moe_testutil.py.
"""

import os

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import checks
from oracle import formats as F
from oracle import layer as OL
from moe_testutil import (dev, host, log, weights, logit_tol, unambiguous_tokens, key_margin, WEIGHT_ATOL, ACC_REL,
                          ACC_REL_GEMM2,
                          h_rounding_allowance, pack_codes_reference, pack_scales_reference)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import sparse_moe_expert_route_amd as m
    m.load()
    return m


def test_one_hip_runtime_in_process(moe):
    torch.zeros(1, device="cuda")
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    log("hip runtimes mapped: %s" % sorted(libs))
    assert len(libs) == 1
    assert any(os.path.basename(moe.lib_path) in line for line in maps.splitlines())


# ---------------------------------------------------------------------------
# top-k on given logits: bit-exact ids, weights within 1e-6
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k,kind,bias", [
    (64, 8, 2, "normal", None), (37, 64, 8, "ties", None), (129, 256, 8, "normal", None),
    (70, 384, 8, "ties", "zipf"), (33, 512, 8, "normal", "zipf"), (5, 8, 8, "normal", None),
    (50, 384, 1, "ties", None), (1, 3, 3, "normal", None), (200, 100, 7, "ties", "tied"),
])
def test_topk_given_logits_bitexact(moe, T, E, k, kind, bias):
    log("topk T=%d E=%d k=%d %s bias=%s" % (T, E, k, kind, bias))
    if kind == "ties":
        L = S.tie_logits(T, E, seed=T)
    else:
        L = S.normal_f32(7, 1000 + E, T * E, 1.3).reshape(T, E)
    b = None
    if bias == "zipf":
        b = S.zipf_bias(E, 4096, seed=1)
    elif bias == "tied":
        b = np.where(np.arange(E) % 2 == 0, np.float32(0.25), np.float32(-0.0)).astype(np.float32)
    p = moe.Problem.make(T, 128, 128, E, k)
    Ld = dev(L)
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    moe.route(p, None, None, None if b is None else dev(b), Ld, ids, w)
    torch.cuda.synchronize()
    ref_ids, ref_w = OL.select_topk(L, k, b)
    assert np.array_equal(host(ids), ref_ids)
    assert np.max(np.abs(host(w) - ref_w)) <= WEIGHT_ATOL
    assert np.array_equal(host(Ld), L)   # input logits untouched


# sigmoid scores: both sides evaluate the sigmoid in float64 and round it once
# to float32 (reading R18), so the keys agree bit for bit and the ids given the
# same logits are compared exactly on every token, ties included; the weights
# (selected scores over their sum, float32 on the GPU) within 1e-6
@pytest.mark.parametrize("T,E,k,kind,bias", [
    (64, 8, 2, "normal", None), (37, 64, 8, "ties", None), (129, 256, 8, "normal", "zipf"),
    (70, 384, 8, "normal", "zipf"), (33, 512, 8, "normal", None), (50, 384, 1, "ties", None),
    (200, 100, 7, "ties", "tied"), (1, 3, 3, "normal", None),
])
def test_topk_sigmoid_given_logits(moe, T, E, k, kind, bias):
    log("topk sigmoid T=%d E=%d k=%d %s bias=%s" % (T, E, k, kind, bias))
    L = S.tie_logits(T, E, seed=T) if kind == "ties" else S.normal_f32(8, 1000 + E, T * E, 1.3).reshape(T, E)
    if bias == "zipf":
        b = S.zipf_bias(E, 4096, seed=1) * np.float32(0.05)
    elif bias == "tied":
        b = np.where(np.arange(E) % 2 == 0, np.float32(0.25), np.float32(-0.0)).astype(np.float32)
    else:
        b = None
    p = moe.Problem.make(T, 128, 128, E, k, 1)
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    moe.route(p, None, None, None if b is None else dev(b), dev(L), ids, w)
    torch.cuda.synchronize()
    ids_g, w_g = host(ids), host(w)
    checks.check_routing(ids_g, w_g, E)
    ref_ids, ref_w = OL.select_topk(L, k, b, "sigmoid")
    assert np.array_equal(ids_g, ref_ids)
    assert np.max(np.abs(w_g - ref_w)) <= WEIGHT_ATOL


# ---------------------------------------------------------------------------
# router logits vs the float64 oracle, and the routing they produce
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,over", [("tiny", {}), ("tiny", dict(T=300, E=40, k=5)),
                                      ("tiny", dict(T=257, H=512, E=96, k=8)),
                                      ("flash_decode", dict(E=64)), ("pro_decode", dict(E=48)),
                                      ("tiny", dict(T=1000, H=1024, E=384, k=8, bias="zipf"))])
def test_route_parity(moe, cfg, over):
    lay = S.make_layer(cfg, seed=3, experts=False, **over)
    T, H = lay["x"].shape
    E, k = lay["w_router"].shape[0], lay["top_k"]
    log("route %s %s T=%d H=%d E=%d" % (cfg, over, T, H, E))
    p = moe.Problem.make(T, H, 128, E, k)
    L = torch.empty(T, E, dtype=torch.float32, device="cuda")
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    bias = lay["bias"]
    moe.route(p, dev(lay["x"]), dev(lay["w_router"]), None if bias is None else dev(bias), L, ids, w)
    torch.cuda.synchronize()
    L_ref = OL.router_logits(lay["x"], lay["w_router"])
    tol = logit_tol(L_ref)
    Lg = host(L).astype(np.float64)
    assert np.all(np.abs(Lg - L_ref) <= tol), np.max(np.abs(Lg - L_ref) / tol)
    ids_g, w_g = host(ids), host(w)
    checks.check_routing(ids_g, w_g, E)
    ref_ids, ref_w = OL.select_topk(L_ref.astype(np.float32), k, bias)
    margin = key_margin(Lg, L_ref, bias)
    log("  max |L_gpu - L_ref| = %.3e (tolerance floor %.3e)" % (np.max(np.abs(Lg - L_ref)), np.min(tol)))
    clear_set = unambiguous_tokens(L_ref, k, bias, margin, order=False)
    clear = unambiguous_tokens(L_ref, k, bias, margin)
    log("  tokens clear of ties: set %d / %d, order %d / %d" % (clear_set.sum(), T, clear.sum(), T))
    assert clear_set.mean() > 0.95
    assert np.array_equal(np.sort(ids_g[clear_set], 1), np.sort(ref_ids[clear_set], 1))
    assert np.array_equal(ids_g[clear], ref_ids[clear])
    keys = L_ref + (0 if bias is None else bias.astype(np.float64)[None, :])
    assert np.all(checks.topk_is_valid(ids_g, keys, margin))
    # weights: softmax of the GPU's own selected logits, within 1e-6
    sel = np.take_along_axis(Lg, ids_g.astype(np.int64), 1)
    z = np.exp(sel - sel.max(1, keepdims=True))
    assert np.max(np.abs(w_g - z / z.sum(1, keepdims=True))) <= WEIGHT_ATOL


# ---------------------------------------------------------------------------
# permutation + FP8 activations: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,H,E,k,skew", [(64, 256, 8, 2, None), (300, 512, 384, 8, 2.0), (1, 128, 8, 8, None),
                                          (2500, 256, 256, 8, None), (777, 384, 17, 3, 4.0),
                                          (16384, 128, 384, 8, 1.5)])
def test_permute_bitexact(moe, T, H, E, k, skew):
    log("permute T=%d H=%d E=%d k=%d skew=%s" % (T, H, E, k, skew))
    ids = S.random_ids(T, E, k, seed=T + E, skew=skew)
    x = S.bf16_normal(5, 77, (T, H))
    x[0, :128] = 0   # an all-zero block
    if T > 1:
        x[1, 128 - 8:128] = np.array([0x3F80, 0xBF80, 0x0001, 0x8001, 0x7F7F, 0, 0x8000, 0x4000], dtype=np.uint16)
    p = moe.Problem.make(T, H, 128, E, k)
    N = T * k
    ws = moe.alloc_workspace(p)
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    st = torch.empty(N, dtype=torch.int32, device="cuda")
    ros = torch.empty(N, dtype=torch.int32, device="cuda")
    xq = torch.empty(N, H, dtype=torch.uint8, device="cuda")
    xs = torch.empty(N, H // 128, dtype=torch.uint8, device="cuda")
    moe.permute(p, dev(ids), dev(x), off, st, ros, xq, xs, ws)
    torch.cuda.synchronize()
    ref = OL.permutation(ids, E)
    assert np.array_equal(host(off), ref["offsets"])
    assert np.array_equal(host(st), ref["sorted_token"])
    assert np.array_equal(host(ros), ref["row_of_slot"])
    qx, sx = OL.quantize_activations(x)
    assert np.array_equal(host(xs), sx[ref["sorted_token"]])
    assert np.array_equal(host(xq), qx[ref["sorted_token"]])


# ---------------------------------------------------------------------------
# block-scaled GEMMs: bit-exact on operands whose float32 sums are exact
# ---------------------------------------------------------------------------
def _offsets_for(T, E, k, seed, skew=None):
    ids = S.random_ids(T, E, k, seed=seed, skew=skew)
    return OL.permutation(ids, E)["offsets"]


# ---------------------------------------------------------------------------
# packed weight layout: a byte permutation, checked against its definition
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("H,I,E", [(256, 128, 3), (4096, 2048, 2), (384, 640, 5), (6144, 512, 1)])
def test_prepack_bitexact(moe, H, I, E):
    log("prepack H=%d I=%d E=%d" % (H, I, E))
    rng = np.random.default_rng(H + I + E)
    w13 = rng.integers(0, 256, size=(E, 2 * I, H // 2), dtype=np.uint8)
    w2 = rng.integers(0, 256, size=(E, H, I // 2), dtype=np.uint8)
    s13 = rng.integers(0, 256, size=(E, 2 * I, H // 32), dtype=np.uint8)
    s2 = rng.integers(0, 256, size=(E, H, I // 32), dtype=np.uint8)
    p = moe.Problem.make(1, H, I, E, 1)
    Wp = moe.prepack_weights(p, moe.ExpertWeights(dev(w13), dev(s13), dev(w2), dev(s2)))
    torch.cuda.synchronize()
    assert Wp.layout == moe.WEIGHTS_PACKED
    assert np.array_equal(host(Wp.w13).reshape(-1), pack_codes_reference(w13.reshape(E * 2 * I, H // 2)))
    assert np.array_equal(host(Wp.w2).reshape(-1), pack_codes_reference(w2.reshape(E * H, I // 2)))
    assert np.array_equal(host(Wp.w13_scale).reshape(-1), pack_scales_reference(s13.reshape(E * 2 * I, H // 32)))
    assert np.array_equal(host(Wp.w2_scale).reshape(-1), pack_scales_reference(s2.reshape(E * H, I // 32)))


# Shapes with few rows per expert run the weight-streaming kernel; those with
# >= 32 rows per expert on average and H, I multiples of 512 (at most 6144)
# the LDS-tiled kernel.  Each runs with canonical and with packed weights.
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("T,H,I,E,k,skew", [(64, 256, 128, 8, 2, None), (40, 512, 256, 16, 4, 3.0),
                                            (9, 4096, 2048, 8, 8, None), (150, 1024, 384, 12, 3, 2.0),
                                            (3, 6144, 256, 4, 2, None), (300, 512, 512, 8, 4, 2.0),
                                            (200, 1024, 256, 16, 8, None), (700, 256, 768, 8, 2, 6.0),
                                            (5, 8192, 256, 4, 2, None), (200, 1024, 512, 16, 8, None),
                                            (700, 512, 1536, 8, 2, 6.0), (150, 6144, 512, 8, 4, 1.5),
                                            # expert counts that are not a multiple of 64
                                            (70, 256, 128, 65, 4, None), (20, 512, 256, 200, 8, 2.0)])
def test_gemm1_preact_lossless_bitexact(moe, T, H, I, E, k, skew, packed):
    log("gemm1 lossless T=%d H=%d I=%d E=%d k=%d packed=%s" % (T, H, I, E, k, packed))
    N = T * k
    off = _offsets_for(T, E, k, seed=H + I, skew=skew)
    a, a_s, w13, w13_s = S.lossless_gemm_inputs(N, H, 2 * I, seed=1, batch=E)
    _, _, w2, w2_s = S.lossless_gemm_inputs(1, I, H, seed=2, batch=E)
    p = moe.Problem.make(T, H, I, E, k)
    ws = moe.alloc_workspace(p)
    W = moe.ExpertWeights(dev(w13), dev(w13_s), dev(w2), dev(w2_s))
    if packed:
        W = moe.prepack_weights(p, W)
    gu = torch.full((N, 2 * I), float("nan"), dtype=torch.float32, device="cuda")
    moe.grouped_gemm1_preact(p, dev(a), dev(a_s), dev(off), W, gu, ws)
    torch.cuda.synchronize()
    A = F.dequantize_fp8_blocks(a, a_s)
    ref = np.zeros((N, 2 * I))
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            ref[r0:r1] = OL.expert_gate_up(A[r0:r1], w13[e], w13_s[e])
    assert np.array_equal(host(gu).astype(np.float64), ref)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("T,H,I,E,k", [(64, 256, 128, 8, 2), (40, 512, 256, 16, 4), (9, 4096, 2048, 8, 8),
                                       (33, 384, 640, 5, 2), (300, 512, 512, 8, 4), (200, 1280, 256, 16, 8),
                                       (50, 384, 512, 6, 2), (200, 1536, 1024, 16, 8), (150, 6144, 512, 8, 4),
                                       (70, 256, 128, 65, 4), (20, 512, 256, 200, 8)])
def test_gemm2_lossless_bitexact(moe, T, H, I, E, k, packed):
    log("gemm2 lossless T=%d H=%d I=%d E=%d k=%d packed=%s" % (T, H, I, E, k, packed))
    N = T * k
    off = _offsets_for(T, E, k, seed=7 + H)
    hq, hs, w2, w2_s = S.lossless_gemm_inputs(N, I, H, seed=3, batch=E)
    _, _, w13, w13_s = S.lossless_gemm_inputs(1, H, 2 * I, seed=4, batch=E)
    p = moe.Problem.make(T, H, I, E, k)
    ws = moe.alloc_workspace(p)
    W = moe.ExpertWeights(dev(w13), dev(w13_s), dev(w2), dev(w2_s))
    if packed:
        W = moe.prepack_weights(p, W)
    y = torch.full((N, H), float("nan"), dtype=torch.float32, device="cuda")
    moe.grouped_gemm2(p, dev(hq), dev(hs), dev(off), W, y, ws)
    torch.cuda.synchronize()
    Hd = F.dequantize_fp8_blocks(hq, hs)
    ref = np.zeros((N, H))
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            ref[r0:r1] = Hd[r0:r1] @ F.decode_mxfp4(w2[e], w2_s[e]).T
    assert np.array_equal(host(y).astype(np.float64), ref)


# Expert offsets handed in directly (the staged entry points take any
# non-decreasing offsets): every row in the first or in the last expert, rows
# only in the odd experts, rows dealt one by one over all experts.  The
# streaming kernels find each m-tile from these offsets alone.
# H = 1024, I = 512 runs the down GEMM with its scales staged in LDS.
@pytest.mark.parametrize("pattern", ["first", "last", "alternate", "dealt"])
@pytest.mark.parametrize("E", [130, 512])
@pytest.mark.parametrize("H,I", [(256, 128), (1024, 512)])
def test_gemm2_lossless_given_offsets(moe, pattern, E, H, I):
    T, k = 40, 4
    N = T * k
    log("gemm2 lossless given offsets %s E=%d H=%d I=%d" % (pattern, E, H, I))
    counts = np.zeros(E, dtype=np.int64)
    if pattern == "first":
        counts[0] = N
    elif pattern == "last":
        counts[E - 1] = N
    elif pattern == "alternate":
        odd = np.arange(1, E, 2)
        np.add.at(counts, odd[np.arange(N) % len(odd)], 1)
    else:
        np.add.at(counts, np.arange(N) % E, 1)   # dealt
    assert counts.sum() == N
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    hq, hs, w2, w2_s = S.lossless_gemm_inputs(N, I, H, seed=5, batch=E)
    _, _, w13, w13_s = S.lossless_gemm_inputs(1, H, 2 * I, seed=6, batch=E)
    p = moe.Problem.make(T, H, I, E, k)
    ws = moe.alloc_workspace(p)
    W = moe.prepack_weights(p, moe.ExpertWeights(dev(w13), dev(w13_s), dev(w2), dev(w2_s)))
    y = torch.full((N, H), float("nan"), dtype=torch.float32, device="cuda")
    moe.grouped_gemm2(p, dev(hq), dev(hs), dev(off), W, y, ws)
    torch.cuda.synchronize()
    Hd = F.dequantize_fp8_blocks(hq, hs)
    ref = np.zeros((N, H))
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            ref[r0:r1] = Hd[r0:r1] @ F.decode_mxfp4(w2[e], w2_s[e]).T
    assert np.array_equal(host(y).astype(np.float64), ref)


# ---------------------------------------------------------------------------
# SwiGLU + FP8 requantisation epilogue on random operands
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("cfg,over", [("tiny", {}), ("tiny", dict(T=90, H=512, I=384, E=16, k=4)),
                                      ("flash_decode", dict(E=16, T=24)), ("tiny", dict(T=400, H=512, I=512, E=8, k=4)),
                                      ("flash_decode", dict(E=8, T=160)), ("tiny", dict(T=300, H=1024, I=1024, E=8, k=4))])
def test_gemm1_swiglu_parity(moe, cfg, over, packed):
    lay = S.make_layer(cfg, seed=5, **over)
    T, H = lay["x"].shape
    E, k = lay["w13"].shape[0], lay["top_k"]
    inter = lay["w2"].shape[2] * 2
    log("gemm1 swiglu %s %s packed=%s" % (cfg, over, packed))
    N = T * k
    ids = S.random_ids(T, E, k, seed=11)
    perm = OL.permutation(ids, E)
    xq, xs = OL.quantize_activations(lay["x"])
    xq, xs = xq[perm["sorted_token"]], xs[perm["sorted_token"]]
    p = moe.Problem.make(T, H, inter, E, k)
    ws = moe.alloc_workspace(p)
    hq = torch.empty(N, inter, dtype=torch.uint8, device="cuda")
    hs = torch.empty(N, inter // 128, dtype=torch.uint8, device="cuda")
    moe.grouped_gemm1_swiglu(p, dev(xq), dev(xs), dev(perm["offsets"]), weights(lay, packed), hq, hs, ws)
    torch.cuda.synchronize()
    A = F.dequantize_fp8_blocks(xq, xs)
    off = perm["offsets"]
    ref_q = np.zeros((N, inter), np.uint8)
    ref_s = np.zeros((N, inter // 128), np.uint8)
    ref_h = np.zeros((N, inter))
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            o = OL.expert_ffn(A[r0:r1], lay["w13"][e], lay["w13_s"][e], lay["w2"][e], lay["w2_s"][e])
            ref_q[r0:r1], ref_s[r0:r1], ref_h[r0:r1] = o["hq"], o["hs"], o["h"]
    gq, gs = host(hq), host(hs)
    checks.check_fp8_blocks(gq, gs)
    # the scale decision agrees except where the float64 block maximum sits on a power-of-two boundary
    assert np.mean(gs == ref_s) > 0.999
    same = np.repeat(gs == ref_s, 128, axis=1)
    # compare code values (0x00 and 0x80 are both zero)
    gv, rv = F.decode_e4m3(gq), F.decode_e4m3(ref_q)
    frac_exact = np.mean(gv[same] == rv[same])
    log("  exact h codes: %.5f" % frac_exact)
    assert frac_exact > 0.99
    # every GPU code is within one e4m3 step of the exact h
    dq = F.dequantize_fp8_blocks(gq, gs)
    step = np.repeat(np.exp2(gs.astype(np.float64) - 127), 128, axis=1) * 32.0   # 448's grid step is 32
    assert np.all(np.abs(dq - ref_h) <= step)
    # and every code or scale that differs from the oracle's is one the oracle flags as ambiguous
    flag_el = np.zeros((N, inter), bool)
    flag_blk = np.zeros((N, inter // 128), bool)
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            _, _, fl = h_rounding_allowance(A[r0:r1], lay["w13"][e], lay["w13_s"][e], lay["w2"][e], lay["w2_s"][e])
            flag_el[r0:r1], flag_blk[r0:r1] = fl["element"], fl["block"]
    assert np.all(flag_blk[gs != ref_s])
    differ = (gv != rv) & same
    log("  differing codes: %d of %d, all flagged: %s (flagged %d)"
        % (differ.sum(), differ.size, bool(np.all(flag_el[differ])), flag_el.sum()))
    assert np.all(flag_el[differ])


@pytest.mark.parametrize("T,H,I,E,k", [(64, 4096, 2048, 8, 8), (40, 1024, 640, 12, 3), (30, 6144, 256, 6, 4),
                                       (300, 1024, 512, 8, 4), (100, 6144, 2048, 8, 8)])
def test_gemm1_accumulation_error_bound(moe, T, H, I, E, k):
    """On random operands the float32 pre-activations are within ACC_REL * sum|a_k w_k| of
    the exact values: the premise of the rounding allowance of the output checks."""
    lay = S.make_layer("tiny", seed=9, T=T, H=H, I=I, E=E, k=k)
    log("gemm1 accumulation bound T=%d H=%d I=%d E=%d" % (T, H, I, E))
    N = T * k
    ids = S.random_ids(T, E, k, seed=12)
    perm = OL.permutation(ids, E)
    xq, xs = OL.quantize_activations(lay["x"])
    xq, xs = xq[perm["sorted_token"]], xs[perm["sorted_token"]]
    p = moe.Problem.make(T, H, I, E, k)
    ws = moe.alloc_workspace(p)
    gu = torch.empty(N, 2 * I, dtype=torch.float32, device="cuda")
    moe.grouped_gemm1_preact(p, dev(xq), dev(xs), dev(perm["offsets"]), weights(lay), gu, ws)
    torch.cuda.synchronize()
    A = F.dequantize_fp8_blocks(xq, xs)
    off = perm["offsets"]
    g = host(gu).astype(np.float64)
    worst = 0.0
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            W = F.decode_mxfp4(lay["w13"][e], lay["w13_s"][e])
            d = np.abs(g[r0:r1] - A[r0:r1] @ W.T) / (np.abs(A[r0:r1]) @ np.abs(W).T + 1e-300)
            worst = max(worst, float(d.max()))
    log("  max |g_gpu - g| / sum|a w| = %.3e (bound %.1e)" % (worst, ACC_REL))
    assert worst <= ACC_REL


@pytest.mark.parametrize("T,H,I,E,k", [(64, 4096, 2048, 8, 8), (64, 4096, 512, 8, 8), (300, 1024, 512, 8, 4),
                                       (300, 6144, 512, 8, 4), (400, 4096, 2048, 8, 8), (40, 1024, 640, 12, 3)])
def test_gemm2_accumulation_error_bound(moe, T, H, I, E, k):
    """The down projection of real SwiGLU h codes (the oracle's, from a random layer) is
    within ACC_REL_GEMM2 * sum|h_k w_k| of the exact float64 product: the premise of the
    y_perm bar of the full-size staged tests.  Also logs the error against the largest
    single product, eps32 * max_k |h_k w_k|, to show which of the two it follows."""
    lay = S.make_layer("tiny", seed=13, T=T, H=H, I=I, E=E, k=k)
    log("gemm2 accumulation bound T=%d H=%d I=%d E=%d" % (T, H, I, E))
    N = T * k
    ids = S.random_ids(T, E, k, seed=14)
    perm = OL.permutation(ids, E)
    xq, xs = OL.quantize_activations(lay["x"])
    A = F.dequantize_fp8_blocks(xq, xs)[perm["sorted_token"]]
    off = perm["offsets"]
    hq = np.zeros((N, I), np.uint8)
    hs = np.zeros((N, I // 128), np.uint8)
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            o = OL.expert_ffn(A[r0:r1], lay["w13"][e], lay["w13_s"][e], lay["w2"][e], lay["w2_s"][e])
            hq[r0:r1], hs[r0:r1] = o["hq"], o["hs"]
    p = moe.Problem.make(T, H, I, E, k)
    ws = moe.alloc_workspace(p)
    y = torch.empty(N, H, dtype=torch.float32, device="cuda")
    moe.grouped_gemm2(p, dev(hq), dev(hs), dev(off), weights(lay, True), y, ws)
    torch.cuda.synchronize()
    Hd = F.dequantize_fp8_blocks(hq, hs)
    g = host(y).astype(np.float64)
    worst, at = 0.0, None
    eps = float(np.finfo(np.float32).eps)
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            W2 = F.decode_mxfp4(lay["w2"][e], lay["w2_s"][e])
            d = np.abs(g[r0:r1] - Hd[r0:r1] @ W2.T) / (np.abs(Hd[r0:r1]) @ np.abs(W2).T + 1e-300)
            i = np.unravel_index(np.argmax(d), d.shape)
            if d[i] > worst:
                prods = np.abs(Hd[r0 + i[0]] * W2[i[1]])
                at = (e, float(d[i]), float(np.abs(g[r0 + i[0], i[1]] - Hd[r0 + i[0]] @ W2[i[1]]) / (eps * prods.max())),
                      int(np.count_nonzero(prods)))
                worst = float(d[i])
    log("  max |y_gpu - y| / sum|h w| = %.3e (bound %.1e); at that element: expert %d, error = %.2f eps32 * max|h_k w_k|, "
        "%d non-zero products" % (worst, ACC_REL_GEMM2, at[0], at[2], at[3]))
    assert worst <= ACC_REL_GEMM2
