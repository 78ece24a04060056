"""The routed MoE feed-forward layer, computed step by step in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the layer is (the pages, by section):
  * teardown "What Did Xiaomi Release?": 256 routed experts per layer (Flash)
    or 384 (Pro), 8 active per token;
  * teardown "How Big Is Each Expert?": a router picks 8 experts per token;
    three matrices per expert (gate, up, down) with intermediate width I = 2048;
  * teardown "How Is the Backbone Built?" and devupai "No shared expert":
    there is no shared expert, so the output is the routed sum alone;
  * teardown "Why Are the V2.6 Files Half the Size of V2.5?": experts are
    stored as MXFP4, the router is BF16;
  * vLLM recipe "Overview": the arithmetic runs in block-scaled FP8 e4m3;
  * teardown "Why Are the V2.6 Files Half the Size of V2.5?", V2.5 column:
    the earlier expert format: e4m3 codes, each 128-row by 128-column tile with
    its own float32 multiplier (layer["format"] == "fp8_block").

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * combine weights are a softmax over the k selected router logits (the
    measured workload) or, with layer["score"] == "sigmoid", the selected
    sigmoid scores over their sum; the selection key may carry an additive
    per-expert bias that does not enter the weights;
  * ties in the selection key go to the lower expert id, -0 equals +0;
  * the load-balancing rule of the selection bias (no formula on the page):
    after a batch an expert below the mean load gains +step, one above it
    loses step (``update_selection_bias``);
  * the expert is SwiGLU: h = silu(gate) * up, silu(z) = z / (1 + exp(-z));
  * W13 stores the I gate rows first, then the I up rows;
  * activations and h are quantised with one power-of-two (e8m0) scale per
    row per 128 channels and round-to-nearest-even e4m3 codes; with FP8
    block-scaled experts, with one float32 scale amax / 448 per row per 128
    channels instead (formats.quantize_fp8_blocks_f32);
  * combine weights apply after the down projection, summed in slot order.

Layouts (row-major, "[A, B]" means B contiguous):
  x        [T, H]      bf16 bits (uint16)
  w_router [E, H]      bf16 bits
  bias     [E]         float32 (selection only) or None
  w13      [E, 2I, H/2] uint8 MXFP4 codes,   w13_s [E, 2I, H/32] uint8 e8m0
  w2       [E, H, I/2]  uint8 MXFP4 codes,   w2_s  [E, H, I/32]  uint8 e8m0
  or, with layer["format"] == "fp8_block":
  w13      [E, 2I, H]   uint8 e4m3 codes,    w13_s [E, 2I/128, H/128] float32
  w2       [E, H, I]    uint8 e4m3 codes,    w2_s  [E, H/128, I/128]  float32
"""

import numpy as np

from . import formats as F

__all__ = [
    "router_logits",
    "select_topk",
    "sigmoid_scores",
    "permutation",
    "quantize_activations",
    "expert_ffn",
    "combine",
    "forward",
    "forward_tokens",
    "expert_gate_up",
    "decode_expert_matrix",
    "expert_format",
]

MXFP4 = "mxfp4"
FP8_BLOCK = "fp8_block"


def expert_format(layer):
    """The layer's expert weight format: "mxfp4" (default) or "fp8_block"."""
    fmt = layer.get("format", MXFP4)
    if fmt not in (MXFP4, FP8_BLOCK):
        raise ValueError("unknown expert format %r" % (fmt,))
    return fmt


def decode_expert_matrix(codes, scales, fmt=MXFP4):
    """One expert weight matrix -> float64 [rows, K] in the given storage format."""
    if fmt == FP8_BLOCK:
        return F.decode_fp8_block(codes, scales)
    return F.decode_mxfp4(codes, scales)


def _quantize(v, fmt):
    return F.quantize_fp8_blocks_f32(v) if fmt == FP8_BLOCK else F.quantize_fp8_blocks(v)


def _dequantize(codes, scales, fmt):
    return F.dequantize_fp8_blocks_f32(codes, scales) if fmt == FP8_BLOCK else F.dequantize_fp8_blocks(codes, scales)


def router_logits(x_bits, w_router_bits):
    """Router logits L = x . W_r^T from the exact bf16 values, in float64.  [T, E]."""
    x = F.decode_bf16(x_bits)
    w = F.decode_bf16(w_router_bits)
    return x @ w.T


def sigmoid_scores(logits):
    """Sigmoid expert scores s = 1 / (1 + exp(-L)) in float64 (teardown "How
    Big Is Each Expert?": the router scores experts with a sigmoid)."""
    L = np.asarray(logits, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-L))


def select_topk(logits, k, bias=None, score="softmax"):
    """Top-k expert selection and combine weights for every token.

    score="softmax" (the measured workloads): the selection key is the
    float32 sum of the float32 logit and the float32 selection bias (an IEEE
    binary32 addition); the weights are a softmax over the k selected
    *unbiased* logits, computed in float64 with the maximum subtracted.

    score="sigmoid" (teardown "How Big Is Each Expert?": sigmoid scores and a
    per-expert load-balancing bias): s = sigmoid(L) rounded to float32;
    the key is the float32 sum s + b; the weights are the k selected scores
    (float64) divided by their sum.

    In both, the k largest keys are taken in descending order; equal keys go
    to the lower expert id (a stable sort of the negated keys); -0 and +0
    compare equal.

    logits: [T, E] float32 (or anything castable to it)
    returns (ids [T, k] int32, w [T, k] float64)
    """
    L = np.asarray(logits, dtype=np.float32)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("k must lie in [1, E]")
    if score == "softmax":
        base = L
    elif score == "sigmoid":
        s64 = sigmoid_scores(L)
        base = s64.astype(np.float32)
    else:
        raise ValueError("unknown score function %r" % (score,))
    key = base if bias is None else (base + np.asarray(bias, dtype=np.float32)[None, :])
    key = key.astype(np.float32)
    order = np.argsort(-key, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    if score == "softmax":
        sel = np.take_along_axis(L, ids, axis=1).astype(np.float64)
        z = np.exp(sel - sel.max(axis=1, keepdims=True))
    else:
        z = np.take_along_axis(s64, ids, axis=1)
    w = z / z.sum(axis=1, keepdims=True)
    return ids, w


def update_selection_bias(expert_offsets, step, bias):
    """One step of the load-balancing rule for the selection bias.

    Teardown "How Big Is Each Expert?": a small per-expert correction bias
    on the sigmoid scores keeps the load across experts even, with no extra
    training loss.  The page gives no update formula; the reading used here
    is the plainest one that evens out the load: after a batch, an expert
    that received fewer rows than the mean load N / E has its bias raised by
    step, one that received more has it lowered by step, and one exactly at
    the mean keeps it.  The comparison is exact (E * n_e against N as
    integers); the new bias is one float32 addition b + (+-step).

    expert_offsets: [E + 1] ints, the rows of expert e are
        [expert_offsets[e], expert_offsets[e + 1])
    step: the step size (a float32 value)
    bias: [E] float32
    returns the new bias, [E] float32
    """
    off = np.asarray(expert_offsets, dtype=np.int64)
    E = off.size - 1
    if E < 1:
        raise ValueError("need at least one expert")
    n = off[1:] - off[:-1]
    total = off[-1] - off[0]
    direction = np.sign(total - E * n)            # +1 below the mean load, -1 above
    step32 = np.float32(step)
    delta = np.where(direction > 0, step32, np.where(direction < 0, -step32, np.float32(0.0))).astype(np.float32)
    return (np.asarray(bias, dtype=np.float32) + delta).astype(np.float32)


def permutation(ids, num_experts):
    """Group the T*k routing slots by expert (a stable counting sort).

    Slots are numbered token-major, s = t*k + j.  Within one expert the rows
    keep ascending slot (hence token) order.

    returns dict with
      counts       [E]      rows per expert
      offsets      [E+1]    exclusive prefix sum of counts
      sorted_token [T*k]    token of each expert-ordered row
      row_of_slot  [T*k]    expert-ordered row of each slot
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=num_experts)[:num_experts]
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")          # expert-ordered slots
    row_of_slot = np.empty(T * k, dtype=np.int64)
    row_of_slot[order] = np.arange(T * k)
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "sorted_token": (order // k).astype(np.int32),
        "row_of_slot": row_of_slot.astype(np.int32),
    }


def quantize_activations(x_bits, fmt=MXFP4):
    """Dynamic FP8 quantisation of the bf16 activations, per token per 128 channels
    (e8m0 scales with MXFP4 experts, float32 scales with FP8 block-scaled experts)."""
    return _quantize(F.decode_bf16(x_bits), fmt)


def _silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_gate_up(a, w13_e, w13_s_e, fmt=MXFP4):
    """Pre-activations of one expert: [G | U] = A . W13_e^T in float64.

    a: [n, H] float64 (already dequantised activations)
    returns [n, 2I] float64 with columns 0..I-1 = gate, I..2I-1 = up
    """
    w13 = decode_expert_matrix(w13_e, w13_s_e, fmt)
    return a @ w13.T


def expert_ffn(a, w13_e, w13_s_e, w2_e, w2_s_e, fmt=MXFP4):
    """One expert on the rows routed to it.

    a: [n, H] float64 dequantised FP8 activations
    returns dict with
      gu  [n, 2I] float64 pre-activations (gate | up)
      h   [n, I]  float64 silu(gate) * up
      hq, hs      FP8 codes [n, I] and scales [n, I/128] of h (e8m0 bytes, or
                  float32 with FP8 block-scaled experts, where h is rounded to
                  float32 before it is quantised)
      y   [n, H]  float64 down projection of the dequantised h
    """
    gu = expert_gate_up(a, w13_e, w13_s_e, fmt)
    inter = gu.shape[1] // 2
    h = _silu(gu[:, :inter]) * gu[:, inter:]
    hq, hs = _quantize(h, fmt)
    hd = _dequantize(hq, hs, fmt)
    w2 = decode_expert_matrix(w2_e, w2_s_e, fmt)
    return {"gu": gu, "h": h, "hq": hq, "hs": hs, "y": hd @ w2.T}


def combine(y_perm, row_of_slot, w):
    """y[t] = sum over j of w[t, j] * y_perm[row_of_slot[t*k + j]], summed in slot order j = 0..k-1."""
    w = np.asarray(w, dtype=np.float64)
    T, k = w.shape
    rows = np.asarray(row_of_slot).reshape(T, k)
    y = np.zeros((T, y_perm.shape[1]), dtype=np.float64)
    for j in range(k):
        y += w[:, j:j + 1] * y_perm[rows[:, j]]
    return y


def forward(layer, logits=None, keep_intermediates=True):
    """The whole layer on every token.

    layer: dict with x, w_router, bias, w13, w13_s, w2, w2_s, top_k
           (see the module docstring for layouts)
    logits: optional [T, E] router logits to route on; by default the
            oracle's own float64 logits, rounded to float32 for selection.
    """
    x = layer["x"]
    k = int(layer["top_k"])
    E = layer["w13"].shape[0]
    L64 = router_logits(x, layer["w_router"])
    L = L64.astype(np.float32) if logits is None else np.asarray(logits, dtype=np.float32)
    ids, w = select_topk(L, k, layer.get("bias"), layer.get("score", "softmax"))
    perm = permutation(ids, E)
    fmt = expert_format(layer)
    xq, xs = quantize_activations(x, fmt)
    st = perm["sorted_token"]
    xq_perm, xs_perm = xq[st], xs[st]
    a_perm = _dequantize(xq_perm, xs_perm, fmt)
    T, H = x.shape
    inter = layer["w13"].shape[1] // 2
    y_perm = np.zeros((T * k, H), dtype=np.float64)
    gu_perm = np.zeros((T * k, 2 * inter), dtype=np.float64) if keep_intermediates else None
    hq_perm = np.zeros((T * k, inter), dtype=np.uint8)
    hs_perm = np.zeros((T * k, inter // F.FP8_BLOCK), dtype=np.float32 if fmt == FP8_BLOCK else np.uint8)
    off = perm["offsets"]
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        out = expert_ffn(a_perm[r0:r1], layer["w13"][e], layer["w13_s"][e],
                         layer["w2"][e], layer["w2_s"][e], fmt)
        y_perm[r0:r1] = out["y"]
        hq_perm[r0:r1], hs_perm[r0:r1] = out["hq"], out["hs"]
        if keep_intermediates:
            gu_perm[r0:r1] = out["gu"]
    y = combine(y_perm, perm["row_of_slot"], w)
    res = {"logits": L64, "ids": ids, "w": w, "y": y, "y_perm": y_perm,
           "xq": xq, "xs": xs, "xq_perm": xq_perm, "xs_perm": xs_perm,
           "hq_perm": hq_perm, "hs_perm": hs_perm, **perm}
    if keep_intermediates:
        res["gu_perm"] = gu_perm
    return res


def forward_tokens(layer, tokens, logits=None):
    """The layer output for a subset of tokens only (for layers too large to run whole).

    Every step of the layer is row-local (routing, quantisation, the expert
    FFN on one row, the combine), so the output of a token does not depend on
    which other tokens are present; this evaluates the same arithmetic as
    ``forward`` on the chosen rows, decoding each needed expert once.

    tokens: 1-D array of token indices
    logits: optional [len(tokens), E] logits to route on (else the oracle's own)
    returns dict with ids, w, logits (float64), y [len(tokens), H] and
            y_slot [len(tokens), k, H] (the per-slot expert outputs)
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    k = int(layer["top_k"])
    x = layer["x"][tokens]
    L64 = router_logits(x, layer["w_router"])
    L = L64.astype(np.float32) if logits is None else np.asarray(logits, dtype=np.float32)
    ids, w = select_topk(L, k, layer.get("bias"), layer.get("score", "softmax"))
    fmt = expert_format(layer)
    xq, xs = quantize_activations(x, fmt)
    a = _dequantize(xq, xs, fmt)
    n, H = x.shape
    y_slot = np.zeros((n, k, H), dtype=np.float64)
    for e in np.unique(ids):
        sel = np.argwhere(ids == e)                     # (row, j) pairs routed to e
        out = expert_ffn(a[sel[:, 0]], layer["w13"][e], layer["w13_s"][e],
                         layer["w2"][e], layer["w2_s"][e], fmt)
        y_slot[sel[:, 0], sel[:, 1]] = out["y"]
    y = np.zeros((n, H), dtype=np.float64)
    for j in range(k):
        y += w[:, j:j + 1] * y_slot[:, j]
    return {"ids": ids, "w": w, "logits": L64, "y": y, "y_slot": y_slot}
