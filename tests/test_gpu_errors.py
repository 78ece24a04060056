"""Device-side data errors: the error words of the workspace, and that every
kernel stays in bounds and exits normally on such data.

Every case here runs the library's own guards (ids out of range get no row,
invalid expert offsets are clamped or give an empty tile plan, the combine
skips slots without a row), so no access leaves its buffer; the tests check
the reported bits and that the valid part of each result is still exact.
"""

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import formats as F
from oracle import layer as OL
from moe_testutil import dev, host, log, weights, problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import sparse_moe_expert_route_amd as m
    m.load()
    return m


def _permute(moe, p, ids, x):
    T, H, E, k = p.num_tokens, p.hidden, p.num_experts, p.top_k
    N = T * k
    ws = moe.alloc_workspace(p)
    ws.fill_(0xAB)   # the words must be written, not inherited
    out = dict(off=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
               st=torch.empty(N, dtype=torch.int32, device="cuda"),
               ros=torch.empty(N, dtype=torch.int32, device="cuda"),
               xq=torch.empty(N, H, dtype=torch.uint8, device="cuda"),
               xs=torch.empty(N, H // 128, dtype=torch.uint8, device="cuda"))
    moe.permute(p, dev(ids), dev(x), out["off"], out["st"], out["ros"], out["xq"], out["xs"], ws)
    torch.cuda.synchronize()
    return ws, {k_: host(v) for k_, v in out.items()}


# N <= 1024 slots: the one-workgroup permutation; larger: count, scan, scatter
@pytest.mark.parametrize("T,E,k", [(40, 16, 4), (300, 64, 8), (2000, 256, 8)])
@pytest.mark.parametrize("kind", ["valid", "range", "negative", "duplicate", "both"])
def test_permute_error_word(moe, T, E, k, kind):
    log("permute error word T=%d E=%d k=%d %s" % (T, E, k, kind))
    ids = S.random_ids(T, E, k, seed=T)
    H = 256
    x = S.bf16_normal(5, 78, (T, H))
    bad_tokens = np.array([1, T // 2, T - 1])
    expect = 0
    if kind in ("range", "both"):
        ids[bad_tokens[0], 1] = E
        ids[bad_tokens[1], k - 1] = E + 100
        expect |= moe.DEVERR_EXPERT_ID_RANGE
    if kind == "negative":
        ids[bad_tokens[2], 0] = -1
        expect |= moe.DEVERR_EXPERT_ID_RANGE
    if kind in ("duplicate", "both"):
        ids[bad_tokens[2], k - 1] = ids[bad_tokens[2], 0]
        expect |= moe.DEVERR_EXPERT_ID_DUPLICATE
    p = moe.Problem.make(T, H, 128, E, k)
    ws, out = _permute(moe, p, ids, x)
    w0, _ = moe.error_words(ws)
    log("  error word 0 = %#x (expected %#x)" % (w0, expect))
    assert w0 == expect
    # the slots with ids in range are permuted exactly as the oracle permutes them alone
    flat = ids.reshape(-1)
    ok = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[ok], minlength=E)
    assert np.array_equal(np.diff(out["off"]), counts) and out["off"][0] == 0
    assert np.all(out["ros"][~ok] == -1)
    order = np.argsort(np.where(ok, flat, E), kind="stable")[:ok.sum()]
    ros_ref = np.full(flat.size, -1)
    ros_ref[order] = np.arange(ok.sum())
    assert np.array_equal(out["ros"], ros_ref)
    assert np.array_equal(out["st"][:ok.sum()], order // k)


def test_combine_skips_slots_without_a_row(moe):
    T, H, E, k = 50, 256, 8, 4
    N = T * k
    log("combine: rows -1 and past T*k contribute nothing")
    rng = np.random.default_rng(3)
    y_perm = rng.normal(size=(N, H)).astype(np.float32)
    ros = rng.permutation(N).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    ros[5] = -1
    ros[17] = N          # one past the end
    ros[N - 1] = 1 << 30
    p = moe.Problem.make(T, H, 128, E, k)
    y = torch.empty(T, H, device="cuda")
    moe.combine(p, dev(y_perm), dev(ros), dev(w), y)
    torch.cuda.synchronize()
    rows = ros.reshape(T, k)
    ref = np.zeros((T, H))
    for j in range(k):
        valid = (rows[:, j] >= 0) & (rows[:, j] < N)
        ref[valid] += w[valid, j:j + 1].astype(np.float64) * y_perm[rows[valid, j]]
    err = np.max(np.abs(host(y) - ref))
    assert err <= 1e-5 * np.max(np.abs(ref)), err


def _offsets_cases(N, E):
    base = np.linspace(0, N, E + 1).astype(np.int64)
    cases = {"valid": base}
    c = base.copy(); c[-1] = N + 64;                 cases["total_past_end"] = c
    c = base.copy(); c[-1] = N - 3;                  cases["total_short"] = c
    c = base.copy(); c[E // 2] = c[E // 2 + 1] + 5;  cases["decreasing"] = c
    c = base.copy(); c[0] = 2;                       cases["first_not_zero"] = c
    c = np.zeros(E + 1, np.int64); c[1::2] = N; c[-1] = N
    cases["zigzag"] = c                              # every odd expert claims all N rows
    return cases


# streaming kernels (few rows per expert) and LDS-tiled kernels (many)
@pytest.mark.parametrize("T,H,I,E,k", [(40, 256, 128, 8, 2), (300, 512, 512, 8, 4)])
@pytest.mark.parametrize("case", ["valid", "total_past_end", "total_short", "decreasing", "first_not_zero", "zigzag"])
def test_gemm_offsets_error_word(moe, T, H, I, E, k, case):
    N = T * k
    off = _offsets_cases(N, E)[case].astype(np.int32)
    log("gemm offsets %s T=%d H=%d I=%d E=%d: %s" % (case, T, H, I, E, off.tolist()))
    hq, hs, w2, w2_s = S.lossless_gemm_inputs(N, I, H, seed=3, batch=E)
    xq, xs, w13, w13_s = S.lossless_gemm_inputs(N, H, 2 * I, seed=4, batch=E)
    p = moe.Problem.make(T, H, I, E, k)
    ws = moe.alloc_workspace(p)
    ws.fill_(0xAB)
    W = moe.prepack_weights(p, moe.ExpertWeights(dev(w13), dev(w13_s), dev(w2), dev(w2_s)))
    y = torch.full((N, H), float("nan"), dtype=torch.float32, device="cuda")
    moe.grouped_gemm2(p, dev(hq), dev(hs), dev(off), W, y, ws)
    torch.cuda.synchronize()
    _, w1 = moe.error_words(ws)
    expect = 0 if case == "valid" else moe.DEVERR_EXPERT_OFFSETS
    log("  error word 1 = %#x (expected %#x)" % (w1, expect))
    assert w1 == expect
    hqo = torch.empty(N, I, dtype=torch.uint8, device="cuda")
    hso = torch.empty(N, I // 128, dtype=torch.uint8, device="cuda")
    ws.fill_(0xAB)
    moe.grouped_gemm1_swiglu(p, dev(xq), dev(xs), dev(off), W, hqo, hso, ws)
    torch.cuda.synchronize()
    assert moe.error_words(ws)[1] == expect
    if case == "valid":
        Hd = F.dequantize_fp8_blocks(hq, hs)
        ref = np.zeros((N, H))
        for e in range(E):
            r0, r1 = off[e], off[e + 1]
            if r1 > r0:
                ref[r0:r1] = Hd[r0:r1] @ F.decode_mxfp4(w2[e], w2_s[e]).T
        assert np.array_equal(host(y).astype(np.float64), ref)


@pytest.mark.parametrize("cfg,over", [("tiny", dict(T=100, E=16, k=4)), ("tiny", dict(T=600, H=512, I=512, E=8, k=4))])
def test_forward_leaves_both_words_clear(moe, cfg, over):
    lay = S.make_layer(cfg, seed=2, **over)
    p = problem(lay)
    T, H = lay["x"].shape
    ws = moe.alloc_workspace(p)
    ws.fill_(0xFF)
    y = torch.empty(T, H, device="cuda")
    moe.forward(p, dev(lay["x"]), dev(lay["w_router"]), None, weights(lay, True), y, ws)
    torch.cuda.synchronize()
    assert moe.error_words(ws) == (0, 0)
