"""Shared helpers of the GPU parity tests: device transfer and comparison bars.

Tolerances (written here once, used by every parity test):
  * router logits: |L_gpu - L_ref| <= 1e-3 * max(|L_ref|, RMS(L_ref)) elementwise
    (1e-3 relative, with the RMS floor so the bound stays meaningful near 0);
  * combine weights: |w_gpu - w_ref| <= 1e-6;
  * layer output: max |y_gpu - y_ref| <= 2e-2 * RMS(y_ref);
  * integer and byte results (ids given the same logits, permutation,
    activation FP8 codes and scales, lossless GEMM results): bit-exact.
"""

import collections
import sys

import numpy as np
import torch

LOGIT_RTOL = 1e-3
WEIGHT_ATOL = 1e-6
OUTPUT_RTOL = 2e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    """numpy -> device tensor; uint16 arrays become bfloat16 (bit pattern preserved)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    t = torch.from_numpy(a).cuda()
    return t if dtype is None else t.to(dtype)


def host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


_EXPERT_CACHE = collections.OrderedDict()
_EXPERT_CACHE_BYTES = 24 << 30


def full_layer(name, seed=0):
    """make_layer(name, seed) with the expert weights shared between workloads of the same
    (H, I, E, format, seed) within one test session (least recently used dropped past 24 GiB)."""
    import synthetic as S
    cfg = S.config(name)
    key = (cfg["H"], cfg["I"], cfg["E"], cfg["format"], seed)
    if key in _EXPERT_CACHE:
        _EXPERT_CACHE.move_to_end(key)
    else:
        _EXPERT_CACHE[key] = S.make_experts(name, seed)
        while len(_EXPERT_CACHE) > 1 and sum(sum(a.nbytes for a in v.values())
                                             for v in _EXPERT_CACHE.values()) > _EXPERT_CACHE_BYTES:
            _EXPERT_CACHE.popitem(last=False)
    return S.make_layer(name, seed=seed, experts=_EXPERT_CACHE[key])


def weights(layer, packed=False):
    """Device expert weights of a layer; packed=True reorders codes and scales with moe_prepack_weights."""
    import sparse_moe_expert_route_amd as moe
    W = moe.ExpertWeights(dev(layer["w13"]), dev(layer["w13_s"]), dev(layer["w2"]), dev(layer["w2_s"]))
    if not packed:
        return W
    return moe.prepack_weights(problem(layer), W)


def is_fp8_block(layer):
    return layer.get("format", "mxfp4") == "fp8_block"


def pack_codes_reference(codes):
    """The packed layout of moe.h written out in numpy: codes [R, K/2] uint8 (R % 16 == 0,
    K % 128 == 0) -> [R * K/2] uint8 with row 16q + r, bytes [64c + 16p, +16) of step c at
    block (q, c), offset (16p + r) * 16."""
    R, KB = codes.shape
    u = codes.reshape(R // 16, 16, KB // 64, 4, 16)        # q, r, c, p, byte
    return np.ascontiguousarray(u.transpose(0, 2, 3, 1, 4)).reshape(-1)


def pack_scales_reference(scales):
    """The packed scale layout of moe.h written out in numpy: scales [R, K/32] uint8 (R % 16 == 0,
    K % 128 == 0) -> [R * K/32] uint8 with row 16q + r, the 4 bytes of 128-column step c at
    block (q, c) of 64 bytes, offset 4r."""
    R, SB = scales.shape
    u = scales.reshape(R // 16, 16, SB // 4, 4)            # q, r, c, byte
    return np.ascontiguousarray(u.transpose(0, 2, 1, 3)).reshape(-1)


def problem(layer):
    import sparse_moe_expert_route_amd as moe
    T, H = layer["x"].shape
    E = layer["w13"].shape[0]
    inter = layer["w13"].shape[1] // 2
    return moe.Problem.make(T, H, inter, E, layer["top_k"], 1 if layer.get("score") == "sigmoid" else 0,
                            moe.EXPERTS_FP8_BLOCK if is_fp8_block(layer) else moe.EXPERTS_MXFP4)


def logit_tol(L_ref):
    rms = np.sqrt(np.mean(L_ref ** 2))
    return LOGIT_RTOL * np.maximum(np.abs(L_ref), rms)


def _score(L, score):
    from oracle import layer as OL
    return OL.sigmoid_scores(L) if score == "sigmoid" else np.asarray(L, np.float64)


def key_margin(L_gpu, L_ref, bias=None, score="softmax"):
    """Per-token uncertainty of the float32 selection keys: the measured |L_gpu - L_ref|
    (times 1/4, the sigmoid's largest slope, for sigmoid scores) plus a few float32
    roundings (of the score, of the sigmoid evaluation and of the bias addition)."""
    key = np.abs(_score(L_ref, score)) + (0.0 if bias is None else np.abs(bias.astype(np.float64))[None, :])
    dev_ = np.max(np.abs(np.asarray(L_gpu, np.float64) - L_ref), axis=1)
    if score == "sigmoid":
        dev_ = dev_ / 4 + 4 * np.finfo(np.float32).eps
    return dev_ + 4 * np.finfo(np.float32).eps * np.max(key, axis=1)


def unambiguous_tokens(L_ref, k, bias, margin, order=True, score="softmax"):
    """Tokens whose top-k decision is clear of ties by more than 2*margin.

    order=True: every adjacent gap among the k+1 largest keys (set and order);
    order=False: only the gap between the k-th and (k+1)-th key (the set)."""
    key = _score(L_ref, score) + (0.0 if bias is None else bias.astype(np.float64)[None, :])
    E = key.shape[1]
    srt = -np.sort(-key, axis=1)[:, :min(k + 1, E)]
    if srt.shape[1] <= k:      # k == E: the set is every expert
        gaps = srt[:, :-1] - srt[:, 1:] if order else np.full((key.shape[0], 1), np.inf)
    else:
        gaps = srt[:, :-1] - srt[:, 1:] if order else srt[:, k - 1:k] - srt[:, k:k + 1]
    m = np.broadcast_to(np.asarray(margin, np.float64), (key.shape[0],))
    return np.all(gaps > 2 * m[:, None], axis=1)


def max_rel_err(y, y_ref):
    rms = np.sqrt(np.mean(y_ref ** 2))
    return float(np.max(np.abs(y - y_ref)) / rms)


def bf16_rne(y32):
    """float32 -> bf16 bit patterns by torch's round-to-nearest-even cast."""
    return torch.from_numpy(np.ascontiguousarray(y32, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


# ---------------------------------------------------------------------------
# Several correct results: FP8 rounding of h near a rounding midpoint.
#
# The gate/up pre-activations are float32 accumulations on the GPU and exact
# float64 values in the oracle; they differ by at most ACC_REL * sum_k |a_k w_k|
# (the measured worst case is 1.7e-6; ACC_REL leaves a margin).  Where that
# uncertainty, carried through h = silu(g) * u, straddles a midpoint of the
# e4m3 grid (or the power-of-two threshold of the block scale), either
# neighbouring code is a correct result.  The oracle alone flags those
# elements; one code step on each flagged element, carried through |W2| and
# the combine weights, is the only freedom a correct GPU result has beyond the
# stated tolerance.
# ---------------------------------------------------------------------------
ACC_REL = 4e-6
# The down projection: h (silu(g) * u, requantised per 128 channels) is far more
# heavy-tailed within a row than the activations, and the error of the block-scaled
# MFMA's sums follows the largest product, not the total (measured 1,000 - 2,200
# float32 ulps of max_k |h_k w_k| over K = 512 .. 2048); relative to sum_k |h_k w_k|
# it is largest at the narrow middle of the tensor-parallel share (I = 512):
# measured worst 4.2e-5 (test_gemm2_accumulation_error_bound), bound 1e-4.
ACC_REL_GEMM2 = 1e-4
# FP8 block-scaled experts: e4m3 x e4m3 products carry 8 significant bits (e4m3 x e2m1: 5),
# so more of the float32 sums round, and each 128-deep block adds the rounding of its scale
# product and of the fold into the running sum.  Measured worst case 4.2e-6 (tiled kernel,
# K = 1024); the bound keeps the same factor-of-two margin.
ACC_REL_FP8 = 8e-6
_EPS32 = float(np.finfo(np.float32).eps)


def _e4m3_neighbours(v):
    """For |v| <= 448: the grid point q nearest v and the spacing to the next point up/down."""
    from oracle import formats as F
    a = np.abs(v)
    q = np.abs(F.decode_e4m3(F.encode_e4m3_rne(a)))
    _, ex = np.frexp(np.maximum(q, 2.0 ** -9))
    step_up = np.exp2(np.maximum(ex - 1, -6) - 3.0)
    _, exd = np.frexp(np.maximum(q - 2.0 ** -10, 2.0 ** -10))
    step_dn = np.where(q > 0, np.exp2(np.maximum(exd - 1, -6) - 3.0), step_up)
    return q, step_up, step_dn


def h_rounding_allowance(a, w13_e, w13_s_e, w2_e, w2_s_e, acc_rel=None, fmt="mxfp4"):
    """Oracle-side flags of ambiguous h codes for one expert's rows, and their effect on y.

    a: [n, H] float64 dequantised activations.
    returns (y [n, H] oracle expert output, allow [n, H] >= 0, flags) where flags is a
    dict with the oracle's h codes/scales and boolean masks "element" [n, I] and "block" [n, I/128]."""
    from oracle import formats as F
    from oracle import layer as OL
    if acc_rel is None:
        acc_rel = ACC_REL_FP8 if fmt == "fp8_block" else ACC_REL
    W13 = OL.decode_expert_matrix(w13_e, w13_s_e, fmt)
    W2 = OL.decode_expert_matrix(w2_e, w2_s_e, fmt)
    inter = W13.shape[0] // 2
    gu = a @ W13.T
    S = np.abs(a) @ np.abs(W13).T
    g, u = gu[:, :inter], gu[:, inter:]
    dg, du = acc_rel * S[:, :inter], acc_rel * S[:, inter:]
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = np.abs(sig * (1.0 + g * (1.0 - sig))) + 0.25 * dg       # |d silu/dg| over the interval (|silu''| <= 1/2)
    h = silu * u
    dh = dsilu * np.abs(u) * dg + (np.abs(silu) + dsilu * dg) * du + 16 * _EPS32 * np.abs(h)
    if fmt == "fp8_block":
        return _h_allowance_f32(h, dh, W2)
    hq, hs = F.quantize_fp8_blocks(h)
    R, C = h.shape
    e = np.repeat(hs.astype(np.float64) - 127, 128, axis=1)
    sc = np.exp2(e)
    v, dv = np.abs(h) / sc, dh / sc
    q, up, dn = _e4m3_neighbours(v)
    cross_up = v + dv >= q + up / 2
    cross_dn = (v - dv <= q - dn / 2) & (q > 0)
    allow_el = np.where(cross_up, up, 0.0) + np.where(cross_dn, dn, 0.0)
    # an interval around 0 can round to either sign: the code may be any of the smallest codes of either sign
    allow_el = np.where(v <= dv, np.maximum(allow_el, q + up), allow_el)
    # block scale: the exponent changes if the amax interval reaches the 1.75 * 2^q threshold
    blk = lambda z: z.reshape(R, C // 128, 128)
    amax = blk(np.abs(h)).max(-1)
    amax_hi = blk(np.abs(h) + dh).max(-1)
    amax_lo = np.maximum(blk(np.abs(h) - dh).max(-1), 0)
    e_hi = F.quantize_fp8_blocks(np.repeat(amax_hi, 128, axis=1))[1]
    e_lo = F.quantize_fp8_blocks(np.repeat(amax_lo, 128, axis=1))[1]
    amb_blk = (e_hi != hs) | (e_lo != hs)
    # a block quantised one power of two coarser moves each element by at most one coarse step
    allow_el = np.where(np.repeat(amb_blk, 128, axis=1), np.maximum(allow_el, 2 * np.maximum(up, dn)), allow_el)
    allow_h = allow_el * sc
    hd = F.dequantize_fp8_blocks(hq, hs)
    flags = {"hq": hq, "hs": hs, "element": allow_el > 0, "block": amb_blk}
    return hd @ W2.T, allow_h @ np.abs(W2).T, flags


def _h_allowance_f32(h, dh, W2):
    """h_rounding_allowance for float32 block scales (s = amax / 448): the GPU's scale can
    move with its block maximum, so each element's quotient h / s is known only to an
    interval; an element is ambiguous where that interval reaches a rounding midpoint."""
    from oracle import formats as F
    R, C = h.shape
    hq, hs = F.quantize_fp8_blocks_f32(h)
    blk = lambda z: z.reshape(R, C // 128, 128)
    amax_hi = blk(np.abs(h) + dh).max(-1)
    amax_lo = np.maximum(blk(np.abs(h) - dh).max(-1), 0)
    s = np.repeat(hs.astype(np.float64), 128, axis=1)
    s_hi = np.repeat(amax_hi / 448.0, 128, axis=1) * (1 + 4 * _EPS32) + 1e-300
    s_lo = np.repeat(amax_lo / 448.0, 128, axis=1) * (1 - 4 * _EPS32)
    q = np.abs(F.decode_e4m3(hq))
    _, up, dn = _e4m3_neighbours(q)
    v_hi = np.minimum((np.abs(h) + dh) / np.maximum(s_lo, 1e-300), 448.0 * (1 + 4 * _EPS32))
    v_lo = np.maximum(np.abs(h) - dh, 0) / s_hi
    cross_up = v_hi >= q + up / 2
    cross_dn = (v_lo <= q - dn / 2) & (q > 0)
    allow_el = np.where(cross_up, up, 0.0) + np.where(cross_dn, dn, 0.0)
    allow_el = np.where(v_lo <= 0, np.maximum(allow_el, q + up), allow_el)
    # a flagged element may land one grid step away, at the GPU's scale (at most s_hi);
    # every element also carries the difference of the two scales
    allow_h = allow_el * s_hi + q * np.maximum(s_hi - s, s - s_lo)
    hd = F.dequantize_fp8_blocks_f32(hq, hs)
    flags = {"hq": hq, "hs": hs, "element": allow_el > 0, "block": np.zeros((R, C // 128), bool),
             "scale_lo": s_lo[:, ::128], "scale_hi": s_hi[:, ::128]}
    return hd @ W2.T, allow_h @ np.abs(W2).T, flags


def oracle_with_allowance(layer, tokens=None):
    """Oracle output of the chosen tokens (all if None) and the allowance of ambiguous h codes.

    Routing is the oracle's own; returns dict(ids, w, logits, y, allow)."""
    from oracle import formats as F
    from oracle import layer as OL
    k = int(layer["top_k"])
    x = layer["x"] if tokens is None else layer["x"][np.asarray(tokens)]
    L = OL.router_logits(x, layer["w_router"])
    ids, w = OL.select_topk(L.astype(np.float32), k, layer.get("bias"), layer.get("score", "softmax"))
    fmt = OL.expert_format(layer)
    xq, xs = OL.quantize_activations(x, fmt)
    a = F.dequantize_fp8_blocks_f32(xq, xs) if fmt == "fp8_block" else F.dequantize_fp8_blocks(xq, xs)
    n, H = x.shape
    y = np.zeros((n, H))
    allow = np.zeros((n, H))
    for e in np.unique(ids):
        sel = np.argwhere(ids == e)
        ye, al, _ = h_rounding_allowance(a[sel[:, 0]], layer["w13"][e], layer["w13_s"][e], layer["w2"][e],
                                         layer["w2_s"][e], fmt=fmt)
        wj = w[sel[:, 0], sel[:, 1]][:, None]
        np.add.at(y, sel[:, 0], wj * ye)
        np.add.at(allow, sel[:, 0], wj * al)
    return {"ids": ids, "w": w, "logits": L, "y": y, "allow": allow}


def check_output(y_gpu, ref, rows=None, rtol=OUTPUT_RTOL):
    """|y_gpu - y_ref| <= rtol * RMS(y_ref) + allowance, elementwise; returns (max err/RMS, share needing allowance)."""
    y_ref, allow = ref["y"], ref["allow"]
    if rows is not None:
        y_ref, allow = y_ref[rows], allow[rows]
        y_gpu = y_gpu[rows]
    rms = np.sqrt(np.mean(y_ref ** 2))
    err = np.abs(y_gpu - y_ref)
    bar = rtol * rms
    assert np.all(err <= bar + allow + 1e-6 * rms), "max excess %.3e x RMS" % np.max((err - bar - allow) / rms)
    return float(err.max() / rms), float(np.mean(err > bar))
