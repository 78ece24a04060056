"""GPU parity of the whole layer (moe_forward) against the oracle.

Small layers are compared on every token; the workloads at their full sizes
(tiny, Flash decode/prefill, Pro decode, Pro skewed prefill, their 4-way
tensor-parallel shares, the speculative-verify blocks and the FP8
block-scaled expert format) are run in the launch configuration the
benchmark times and compared on sampled tokens that the oracle evaluates one
by one, plus invariants over all tokens.

Tokens whose top-k decision lies within the measured logit deviation of a
tie can legitimately route differently on the GPU (float32) and in the
oracle (float64); they are excluded from the element-wise output comparison
and their routing is checked for validity instead.  Likewise an h element
whose exact value sits within the float32 accumulation error of an e4m3
rounding midpoint has two correct codes; the oracle flags those and, on the
small layers, the output bar is widened by exactly one code step on each
flagged element (tests/moe_testutil.py: h_rounding_allowance).  On the
full-size workloads the plain bar max |y - y_ref| <= 2e-2 * RMS(y_ref) is
asserted with no allowance.
"""

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import checks
from oracle import formats as F
from oracle import layer as OL
from moe_testutil import (dev, host, log, weights, problem, logit_tol, unambiguous_tokens, key_margin, bf16_rne,
                          oracle_with_allowance, check_output, full_layer, h_rounding_allowance, ACC_REL_FP8,
                          ACC_REL_GEMM2)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import sparse_moe_expert_route_amd as m
    m.load()
    return m


def _gpu_logits(moe, lay, p):
    T, E = lay["x"].shape[0], p.num_experts
    L = torch.empty(T, E, device="cuda")
    ids = torch.empty(T, p.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, p.top_k, device="cuda")
    b = lay["bias"]
    moe.route(p, dev(lay["x"]), dev(lay["w_router"]), None if b is None else dev(b), L, ids, w)
    torch.cuda.synchronize()
    return host(L), host(ids), host(w)


def _forward(moe, lay, p, W, out_dtype=0, ws=None):
    ws = moe.alloc_workspace(p) if ws is None else ws
    T, H = lay["x"].shape
    y = torch.empty(T, H, dtype=torch.float32 if out_dtype == 0 else torch.bfloat16, device="cuda")
    b = lay["bias"]
    moe.forward(p, dev(lay["x"]), dev(lay["w_router"]), None if b is None else dev(b), W, y, ws, out_dtype)
    torch.cuda.synchronize()
    return host(y)


SMALL = [("tiny", {}, False), ("tiny", dict(bias="zipf", E=32, k=4, T=100), False), ("tiny", dict(T=1), False),
         ("tiny", dict(E=4, k=4, T=33), False), ("tiny", dict(k=1, T=70), False),
         ("tiny", dict(T=129, H=512, I=256, E=24, k=8), False), ("tiny", dict(T=40, H=1024, I=640, E=12, k=3), False),
         ("tiny", dict(T=512, H=512, I=512, E=16, k=4, bias="zipf"), False),
         ("tiny", dict(T=300, H=256, I=256, E=8, k=8), False),
         # packed weights: streaming and tiled kernels
         ("tiny", dict(T=129, H=512, I=256, E=24, k=8), True), ("tiny", dict(T=40, H=1024, I=640, E=12, k=3), True),
         ("tiny", dict(T=512, H=512, I=512, E=16, k=4, bias="zipf"), True),
         ("tiny", dict(T=400, H=1024, I=1536, E=16, k=8), True),
         # at most 1024 slots (single-workgroup permutation) on the tiled kernel
         ("tiny", dict(T=100, H=512, I=512, E=8, k=4), True),
         # the largest expert count (512: eight keys per lane in the top-k)
         ("tiny", dict(T=100, H=512, I=256, E=512, k=8), True),
         # H above the tiled kernel's limit: many rows per expert on the streaming kernel
         ("tiny", dict(T=300, H=8192, I=256, E=8, k=4), True),
         # expert counts that are not a multiple of 64: the streaming kernels' m-tile
         # lookup gives lanes uneven runs of experts, some none
         ("tiny", dict(T=64, E=65, k=8), True), ("tiny", dict(T=100, H=512, I=256, E=200, k=8), False),
         ("tiny", dict(T=3, E=130, k=8), True)]


SIGMOID = [("tiny", dict(T=100, E=32, k=4, bias="zipf"), False), ("tiny", dict(T=300, H=512, I=512, E=8, k=4), True),
           ("flash_decode", dict(T=16, E=32), True)]

# FP8 block-scaled experts (e4m3 weights, float32 128 x 128 block scales); K not a
# multiple of 256 (H = 384, I = 640) takes the one-step stage
FP8 = [("tiny", dict(format="fp8_block"), False), ("tiny", dict(T=129, H=512, I=256, E=24, k=8, format="fp8_block"), True),
       ("tiny", dict(T=40, H=1024, I=640, E=12, k=3, format="fp8_block"), False),
       ("tiny", dict(T=300, H=384, I=384, E=8, k=8, bias="zipf", format="fp8_block"), True),
       ("tiny", dict(T=600, H=512, I=512, E=8, k=4, format="fp8_block"), True),
       ("tiny", dict(T=1, format="fp8_block"), True),
       ("tiny", dict(T=50, E=100, k=6, format="fp8_block"), True),
       # sigmoid scoring with FP8 block-scaled experts, streaming and tiled kernels
       ("tiny", dict(T=100, E=32, k=4, bias="zipf", format="fp8_block", score="sigmoid"), True),
       ("tiny", dict(T=600, H=512, I=512, E=8, k=4, format="fp8_block", score="sigmoid"), False)]


@pytest.mark.parametrize("cfg,over,packed", SMALL + [(c, dict(o, score="sigmoid"), pk) for c, o, pk in SIGMOID] +
                         [pytest.param(c, o, pk, id="fp8_block-%d" % i) for i, (c, o, pk) in enumerate(FP8)])
def test_forward_small_parity(moe, cfg, over, packed):
    over = dict(over)
    score = over.pop("score", "softmax")
    lay = S.make_layer(cfg, seed=0, **over)
    lay["score"] = score
    p = problem(lay)
    log("forward %s %s score=%s packed=%s" % (cfg, over, score, packed))
    W = weights(lay, packed)
    y = _forward(moe, lay, p, W)
    ref = oracle_with_allowance(lay)
    L_ref = ref["logits"]
    Lg, ids_g, _ = _gpu_logits(moe, lay, p)
    assert np.all(np.abs(Lg - L_ref) <= logit_tol(L_ref))
    clear = unambiguous_tokens(L_ref, lay["top_k"], lay["bias"], key_margin(Lg, L_ref, lay["bias"], score),
                               order=False, score=score)
    assert np.array_equal(np.sort(ids_g[clear], 1), np.sort(ref["ids"][clear], 1))
    err, share = check_output(y, ref, rows=clear)
    log("  max err / RMS = %.3e on %d/%d tokens; share of elements beyond the plain bar: %.2e"
        % (err, clear.sum(), clear.size, share))
    # bf16 output is the round-to-nearest-even of the float32 output
    yb = _forward(moe, lay, p, W, out_dtype=1)
    assert np.array_equal(yb, bf16_rne(y))
    # deterministic
    assert np.array_equal(_forward(moe, lay, p, W), y)


@pytest.mark.parametrize("packed,fmt", [(False, "mxfp4"), (True, "mxfp4"), (False, "fp8_block"), (True, "fp8_block")])
def test_staged_entry_points_equal_forward(moe, packed, fmt):
    lay = S.make_layer("tiny", seed=4, T=200, E=16, k=4, bias="zipf", format=fmt)
    p = problem(lay)
    T, H = lay["x"].shape
    E, k, inter = p.num_experts, p.top_k, p.intermediate
    N = T * k
    W = weights(lay, packed)
    y_fused = _forward(moe, lay, p, W)
    ws = moe.alloc_workspace(p)
    x = dev(lay["x"])
    L = torch.empty(T, E, device="cuda")
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, device="cuda")
    moe.route(p, x, dev(lay["w_router"]), dev(lay["bias"]), L, ids, w)
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    st = torch.empty(N, dtype=torch.int32, device="cuda")
    ros = torch.empty(N, dtype=torch.int32, device="cuda")
    xq = torch.empty(N, H, dtype=torch.uint8, device="cuda")
    xs = torch.empty(N, H // 128, dtype=moe.scale_dtype(p), device="cuda")
    moe.permute(p, ids, x, off, st, ros, xq, xs, ws)
    yp = torch.empty(N, H, device="cuda")
    moe.grouped_gemm_swiglu(p, xq, xs, off, W, yp, ws)
    hq = torch.empty(N, inter, dtype=torch.uint8, device="cuda")
    hs = torch.empty(N, inter // 128, dtype=moe.scale_dtype(p), device="cuda")
    moe.grouped_gemm1_swiglu(p, xq, xs, off, W, hq, hs, ws)
    yp2 = torch.empty(N, H, device="cuda")
    moe.grouped_gemm2(p, hq, hs, off, W, yp2, ws)
    y = torch.empty(T, H, device="cuda")
    moe.combine(p, yp, ros, w, y)
    torch.cuda.synchronize()
    assert np.array_equal(host(yp), host(yp2))
    assert np.array_equal(host(y), y_fused)
    checks.check_permutation(host(ids), host(off), host(st), host(ros))


# the benchmarked path (packed weights) on every workload, and canonical
# weights on one decode and one prefill workload; grouped by expert weight set
# (Flash, Pro, their tensor-parallel shares, FP8 block-scaled) so that the
# weights are generated once per set
FULL = [("tiny", True), ("flash_decode", True), ("flash_decode", False), ("flash_prefill", True),
        ("flash_prefill", False),
        # speculative-decoding verify blocks (32 sequences x 8 positions)
        ("flash_verify", True),
        ("pro_decode", True), ("pro_skewed_prefill", True), ("pro_verify", True),
        # one GPU's share of the 4-way tensor-parallel layer (I = 512), all four workloads
        ("flash_decode_tp4", True), ("flash_prefill_tp4", True), ("pro_decode_tp4", True),
        ("pro_skewed_prefill_tp4", True),
        # FP8 block-scaled experts
        ("flash_decode_fp8", True), ("flash_decode_fp8", False), ("flash_prefill_fp8", True), ("pro_decode_fp8", True)]
# sigmoid scoring at full size: zero bias (Flash decode) and the Zipf
# selection bias (Pro skewed prefill)
FULL_SIGMOID = [("flash_decode", True), ("pro_skewed_prefill", True)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,packed,score", [(c, pk, "softmax") for c, pk in FULL] +
                         [pytest.param(c, pk, "sigmoid", id="sigmoid-%s" % c) for c, pk in FULL_SIGMOID])
def test_forward_full_size_sampled(moe, cfg, packed, score):
    log("full-size %s packed=%s score=%s: generating layer" % (cfg, packed, score))
    lay = full_layer(cfg)
    lay["score"] = score
    p = problem(lay)
    T, H = lay["x"].shape
    E, k = p.num_experts, p.top_k
    log("  uploading")
    W = weights(lay, packed)
    ws = moe.alloc_workspace(p)
    log("  forward")
    y = _forward(moe, lay, p, W, ws=ws)
    assert np.all(np.isfinite(y))
    # routing over every token (staged call on the same inputs)
    b = lay["bias"]
    Lall, ids_g, w_g = _gpu_logits(moe, lay, p)
    checks.check_routing(ids_g, w_g, E)
    counts = np.bincount(ids_g.reshape(-1), minlength=E)
    log("  rows per expert: max %d mean %.1f min %d, experts >10x mean: %d, touched %d"
        % (counts.max(), counts.mean(), counts.min(), (counts > 10 * counts.mean()).sum(), (counts > 0).sum()))
    # sampled tokens, evaluated by the oracle one by one
    rng = np.random.default_rng(1)
    toks = np.sort(rng.choice(T, size=min(6, T), replace=False))
    log("  oracle on tokens %s" % toks.tolist())
    ref = oracle_with_allowance(lay, toks)
    tol = logit_tol(ref["logits"])
    Lg = Lall[toks].astype(np.float64)
    assert np.all(np.abs(Lg - ref["logits"]) <= tol)
    margin = key_margin(Lg, ref["logits"], b, score)
    clear = unambiguous_tokens(ref["logits"], k, b, margin, order=False, score=score)
    assert np.array_equal(np.sort(ids_g[toks][clear], 1), np.sort(ref["ids"][clear], 1))
    assert clear.any()
    err, share = check_output(y[toks], ref, rows=clear)
    log("  max err / RMS = %.3e (%d of %d sampled tokens unambiguous); beyond the plain bar: %.2e"
        % (err, clear.sum(), len(toks), share))
    # at full size no output element needs the rounding allowance: the plain bar holds
    assert share == 0.0, "%.2e of the elements exceed 2e-2 x RMS" % share


# ---------------------------------------------------------------------------
# Full size, staged, whole experts.  The stages run on the GPU one after the
# other on the workload's seeded inputs, each fed the previous stage's GPU
# output (the staging of the oracle comparison: routing from the GPU's
# logits, GEMM-2 on the GPU's h), and every row of a chosen set of experts is
# compared with the oracle:
#   * permutation of every slot: bit-exact (oracle counting sort of the GPU's ids);
#   * FP8 activation codes and scales of the chosen rows: bit-exact;
#   * h codes and scales: equal except where the oracle flags the rounding as
#     ambiguous (reading R16; FP8 block-scaled experts: every scale inside the
#     interval the accumulation error allows);
#   * y_perm: within ACC_REL_GEMM2 * sum|h w| (the measured float32 accumulation
#     bound of the down projection) of the oracle's down projection of the GPU's
#     own h (no allowance for anything else);
#   * the combine on 256 sampled tokens: within k float32 roundings of the
#     weighted sum of the GPU's own y_perm rows;
#   * the fused forward equals the staged path bit for bit on every token.
# The chosen experts: the most and the least loaded, the owners of the first
# and last work item of each XCD's share of the LDS-tiled GEMMs' item lists
# (both GEMMs), and a few more at random.  The most loaded expert of the
# skewed workload has ~10k rows: 80 m-tiles of 128 rows in chunks of four,
# the last one partial.
# ---------------------------------------------------------------------------
STAGED_FULL = ["flash_decode", "flash_verify", "flash_prefill", "pro_decode", "pro_skewed_prefill", "flash_prefill_tp4",
               "pro_skewed_prefill_tp4", "pro_decode_tp4", "flash_prefill_fp8", "flash_decode_fp8"]


def _xcd_boundary_experts(counts, NB, rows_per_tile=128, xcds=8):
    tiles = (counts + rows_per_tile - 1) // rows_per_tile
    ts = np.concatenate([[0], np.cumsum(tiles)])
    total = int(ts[-1]) * NB
    out = set()
    for x in range(xcds):
        lo, hi = (total * x) // xcds, (total * (x + 1)) // xcds
        for item in ((lo, hi - 1) if lo < hi else ()):
            out.add(int(np.searchsorted(ts, item // NB, side="right") - 1))
    return out


def _check_h(gq, gs, fl, fmt):
    """GPU h codes/scales of one expert's rows against the oracle's, under the flag rule."""
    gv, rv = F.decode_e4m3(gq), F.decode_e4m3(fl["hq"])
    if fmt == "fp8_block":
        g64 = gs.astype(np.float64)
        assert np.all((g64 >= fl["scale_lo"]) & (g64 <= fl["scale_hi"])), "h scale outside its interval"
        differ = gv != rv
        bmax = np.abs(gv).reshape(gv.shape[0], -1, 128).max(-1)
        assert np.all(bmax[g64 > 0] == 448.0)
    else:
        assert np.all(fl["block"][gs != fl["hs"]]), "an h scale differs where the oracle flags nothing"
        differ = (gv != rv) & np.repeat(gs == fl["hs"], 128, axis=1)
    assert np.all(fl["element"][differ]), "an h code differs where the oracle flags nothing"
    return int(differ.sum()), int(fl["element"].sum())


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", STAGED_FULL)
def test_staged_full_size_whole_experts(moe, cfg):
    log("staged full-size %s: generating layer" % cfg)
    lay = full_layer(cfg)
    p = problem(lay)
    fmt = OL.expert_format(lay)
    T, H = lay["x"].shape
    E, k, inter = p.num_experts, p.top_k, p.intermediate
    N = T * k
    W = weights(lay, True)
    ws = moe.alloc_workspace(p)
    x = dev(lay["x"])
    b = None if lay["bias"] is None else dev(lay["bias"])
    sdt = moe.scale_dtype(p)
    L = torch.empty(T, E, device="cuda")
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    st = torch.empty(N, dtype=torch.int32, device="cuda")
    ros = torch.empty(N, dtype=torch.int32, device="cuda")
    xq = torch.empty(N, H, dtype=torch.uint8, device="cuda")
    xs = torch.empty(N, H // 128, dtype=sdt, device="cuda")
    hq = torch.empty(N, inter, dtype=torch.uint8, device="cuda")
    hs = torch.empty(N, inter // 128, dtype=sdt, device="cuda")
    yp = torch.empty(N, H, device="cuda")
    y = torch.empty(T, H, device="cuda")
    log("  stages on the GPU")
    moe.route(p, x, dev(lay["w_router"]), b, L, ids, w)
    moe.permute(p, ids, x, off, st, ros, xq, xs, ws)
    moe.grouped_gemm1_swiglu(p, xq, xs, off, W, hq, hs, ws)
    moe.grouped_gemm2(p, hq, hs, off, W, yp, ws)
    moe.combine(p, yp, ros, w, y)
    assert moe.error_words(ws) == (0, 0)
    y_fused = torch.empty(T, H, device="cuda")
    moe.forward(p, x, dev(lay["w_router"]), b, W, y_fused, ws)
    torch.cuda.synchronize()
    assert torch.equal(y_fused, y), "the fused forward differs from the staged path"
    assert moe.error_words(ws) == (0, 0)
    ids_g, w_g = host(ids), host(w)
    checks.check_routing(ids_g, w_g, E)
    ref = OL.permutation(ids_g, E)
    off_g, st_g, ros_g = host(off), host(st), host(ros)
    assert np.array_equal(off_g, ref["offsets"])
    assert np.array_equal(st_g, ref["sorted_token"])
    assert np.array_equal(ros_g, ref["row_of_slot"])
    counts = np.diff(off_g).astype(np.int64)
    touched = np.nonzero(counts)[0]
    rng = np.random.default_rng(7)
    sel = {int(np.argmax(counts)), int(touched[np.argmin(counts[touched])]), int(touched[0]), int(touched[-1])}
    if N >= 32 * E:   # the LDS-tiled kernels' persistent item split
        sel |= _xcd_boundary_experts(counts, inter // 256) | _xcd_boundary_experts(counts, H // 512)
    sel |= {int(e) for e in rng.choice(touched, size=min(4, len(touched)), replace=False)}
    sel = sorted(sel)
    log("  experts %s with %s rows (%d of %d rows)" % (sel, counts[sel].tolist(), counts[sel].sum(), N))
    acc = max(ACC_REL_FP8, ACC_REL_GEMM2) if fmt == "fp8_block" else ACC_REL_GEMM2
    worst, n_diff, n_flag = 0.0, 0, 0
    for e in sel:
        r0, r1 = int(off_g[e]), int(off_g[e + 1])
        tok = st_g[r0:r1]
        qx, sx = OL.quantize_activations(lay["x"][tok], fmt)
        assert np.array_equal(host(xq[r0:r1]), qx) and np.array_equal(host(xs[r0:r1]), sx), "x codes, expert %d" % e
        a = F.dequantize_fp8_blocks_f32(qx, sx) if fmt == "fp8_block" else F.dequantize_fp8_blocks(qx, sx)
        _, _, fl = h_rounding_allowance(a, lay["w13"][e], lay["w13_s"][e], lay["w2"][e], lay["w2_s"][e], fmt=fmt)
        gq, gs = host(hq[r0:r1]), host(hs[r0:r1])
        d, f = _check_h(gq, gs, fl, fmt)
        n_diff, n_flag = n_diff + d, n_flag + f
        Hd = F.dequantize_fp8_blocks_f32(gq, gs) if fmt == "fp8_block" else F.dequantize_fp8_blocks(gq, gs)
        W2 = OL.decode_expert_matrix(lay["w2"][e], lay["w2_s"][e], fmt)
        y_ref = Hd @ W2.T
        ssum = np.abs(Hd) @ np.abs(W2).T + 1e-300
        dy = np.abs(host(yp[r0:r1]).astype(np.float64) - y_ref)
        worst = max(worst, float(np.max(dy / ssum)))
        log("    expert %d: %d rows, %d h codes differ (all flagged), max |dy| / sum|h w| = %.2e"
            % (e, r1 - r0, d, float(np.max(dy / ssum))))
    log("  h codes differing from the oracle: %d (all flagged; %d flagged); max |dy| / sum|h w| = %.3e (bound %.1e)"
        % (n_diff, n_flag, worst, acc))
    assert worst <= acc
    # combine on sampled tokens, from the GPU's own y_perm rows
    toks = np.sort(rng.choice(T, size=min(T, 256), replace=False))
    rows = ros_g.reshape(T, k)[toks]
    Yp = host(yp[torch.from_numpy(rows.reshape(-1).astype(np.int64)).cuda()]).reshape(len(toks), k, H).astype(np.float64)
    wt = w_g[toks].astype(np.float64)[:, :, None]
    ref_y = np.sum(wt * Yp, axis=1)
    bound = k * np.finfo(np.float32).eps * np.sum(np.abs(wt * Yp), axis=1) + 1e-30
    assert np.all(np.abs(host(y)[toks] - ref_y) <= bound)


# ---------------------------------------------------------------------------
# Graph capture: the whole forward is device work on one stream (no host
# synchronisation, allocation or memset), so it can be captured once and
# replayed; every replay must reproduce the eager result bit for bit, also
# after eager calls that reuse the workspace with other inputs.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,over,packed", [("tiny", dict(T=129, H=512, I=256, E=24, k=8), True),
                                             ("tiny", dict(T=512, H=512, I=512, E=16, k=4, bias="zipf"), True),
                                             ("tiny", dict(T=100, E=32, k=4), False),
                                             ("flash_decode", dict(T=64, E=32), True),
                                             pytest.param("flash_decode", dict(T=64, E=32, format="fp8_block"), True,
                                                          id="fp8_block-flash_decode")])
def test_forward_graph_replay_matches_eager(moe, cfg, over, packed):
    log("graph replay %s %s packed=%s" % (cfg, over, packed))
    lay = S.make_layer(cfg, seed=5, **over)
    other = S.make_layer(cfg, seed=6, experts=False, **over)
    p = problem(lay)
    T, H = lay["x"].shape
    W = weights(lay, packed)
    ws = moe.alloc_workspace(p)
    x, wr = dev(lay["x"]), dev(lay["w_router"])
    b = None if lay["bias"] is None else dev(lay["bias"])
    x2 = dev(other["x"])
    y_ref = torch.empty(T, H, dtype=torch.float32, device="cuda")
    moe.forward(p, x, wr, b, W, y_ref, ws)
    torch.cuda.synchronize()
    y = torch.empty_like(y_ref)
    y2 = torch.empty_like(y_ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.forward(p, x, wr, b, W, y, ws)      # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.forward(p, x, wr, b, W, y, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(float("nan"))
        moe.forward(p, x2, wr, b, W, y2, ws)     # eager work on other inputs, same workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), "replay %d differs from the eager forward" % rep
    assert not torch.equal(y2, y_ref)
