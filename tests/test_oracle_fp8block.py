"""Pins of the oracle's FP8 block-scaled expert format (CPU only).

The format is the earlier (V2.5) expert format in the teardown's table of
section "Why Are the V2.6 Files Half the Size of V2.5?": e4m3 codes with one
float32 scale per 128 x 128 block.  What pins what:
  * the block decoder: an element-by-element loop over torch's own
    float8_e4m3fn values and explicit block indices;
  * the float32-scale activation quantiser: torch's float32 arithmetic and
    its float32 -> e4m3 cast, a brute-force nearest-grid search, and the
    invariants of the rule (the block maximum maps to 448 exactly; every
    code is within half a grid step);
  * the layer in this format: brute-force dense evaluation of every expert on
    every token, masked by the top-k weights; identical experts equal one
    dense SwiGLU MLP built from torch's silu;
  * the byte cost: the printed V2.5 and V2.6 checkpoint sizes of Flash differ
    by what moving the experts from this format to MXFP4 (and the router from
    F32 to BF16) saves;
  * planted mistakes in the new functions fail at least one pin.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import layer as OL
from oracle import checks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
_TORCH_E4M3 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 1, c).astype(np.uint8)   # no NaN codes


def test_decode_fp8_block_elementwise():
    rng = np.random.default_rng(11)
    R, K = 256, 384
    codes = _finite_codes(rng, (R, K))
    scales = np.exp2(rng.uniform(-12, 4, size=(R // 128, K // 128))).astype(np.float32)
    ours = F.decode_fp8_block(codes, scales)
    for i in range(R):
        for j in range(K):
            assert ours[i, j] == _TORCH_E4M3[codes[i, j]] * float(scales[i // 128][j // 128])


def _torch_quant(v32):
    """The float32-scale rule with torch's float32 ops and torch's e4m3 cast."""
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32))
    R, C = t.shape
    b = t.reshape(R, C // 128, 128)
    amax = b.abs().amax(dim=-1)
    s = amax / torch.tensor(448.0, dtype=torch.float32)
    d = torch.where(amax > 0, s, torch.ones_like(s))
    q = (b / d[..., None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(R, C).numpy(), s.numpy()


def _test_rows(rng):
    R, C = 24, 512
    mag = np.exp2(rng.integers(-20, 12, size=(R, C // 128, 1)))
    v = (rng.standard_normal((R, C // 128, 128)) * mag).reshape(R, C).astype(np.float32)
    v[3, :128] = 0.0
    v[4, 128:256] = -0.0
    v[5, 256:384] = 0.0
    v[5, 300] = -3e-5                                 # a lone value: maps to -448 exactly
    v[6, :] = np.float32(2.0 ** -133)                 # float32 subnormals
    v[7, :128] = np.float32(1e30)
    return v


def test_quantize_f32_matches_torch():
    rng = np.random.default_rng(12)
    v = _test_rows(rng)
    codes, s = F.quantize_fp8_blocks_f32(v)
    tc, ts = _torch_quant(v)
    assert s.dtype == np.float32 and np.array_equal(s.view(np.uint32), ts.view(np.uint32))
    assert np.array_equal(codes, tc)
    # an all-zero run: scale 0, signed zeros
    assert s[3, 0] == 0 and np.all(codes[3, :128] == 0) and np.all(codes[4, 128:256] == 0x80)


def test_quantize_f32_bruteforce_and_invariants():
    rng = np.random.default_rng(13)
    v = _test_rows(rng)
    codes, s = F.quantize_fp8_blocks_f32(v)
    grid = _TORCH_E4M3.copy()
    finite = ~np.isnan(grid)
    R, C = v.shape
    for i in range(R):
        for b in range(C // 128):
            sc = s[i, b]
            d = sc if sc > 0 else np.float32(1)
            for j in range(b * 128, b * 128 + 128, 7):
                x = float(np.float32(v[i, j]) / d)          # the binary32 quotient
                x = min(max(x, -448.0), 448.0)
                dist = np.where(finite, np.abs(grid - x), np.inf)
                best = np.flatnonzero(dist == dist.min())
                best = best[np.signbit(grid[best]) == np.signbit(x)] if len(best) > 1 else best
                if len(best) > 1:                            # a tie: the even code
                    best = best[(best & 1) == 0]
                assert codes[i, j] == best[0], (i, j, x)
    # the block maximum maps to +-448 exactly; dequantised values within half a step
    val = F.decode_e4m3(codes).reshape(R, C // 128, 128)
    nz = s > 0
    assert np.all(np.abs(val).max(-1)[nz] == 448.0)
    deq = F.dequantize_fp8_blocks_f32(codes, s)
    v64 = v.astype(np.float64)
    half_step = np.repeat(s.astype(np.float64), 128, axis=1) * np.maximum(np.abs(v64) / np.repeat(s.astype(np.float64) + (s == 0), 128, axis=1), 2.0 ** -6) * 2.0 ** -4
    assert np.all(np.abs(deq - v64) <= half_step * (1 + 1e-6) + 1e-300)


def _dense_bruteforce_fp8(layer):
    """Every expert on every token, masked by the top-k softmax weights, in the FP8 block format."""
    x = layer["x"]
    T, H = x.shape
    E = layer["w13"].shape[0]
    k = layer["top_k"]
    L = (F.decode_bf16(x) @ F.decode_bf16(layer["w_router"]).T).astype(np.float32)
    mask = np.zeros((T, E))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(L[t, e]), e))[:k]
        sel = L[t, order].astype(np.float64)
        p = np.exp(sel - sel.max())
        mask[t, order] = p / p.sum()
    xq, xs = F.quantize_fp8_blocks_f32(F.decode_bf16(x))
    a = F.dequantize_fp8_blocks_f32(xq, xs)
    inter = layer["w13"].shape[1] // 2
    y = np.zeros((T, H))
    for e in range(E):
        w13 = F.decode_fp8_block(layer["w13"][e], layer["w13_s"][e])
        w2 = F.decode_fp8_block(layer["w2"][e], layer["w2_s"][e])
        h = torch.nn.functional.silu(torch.from_numpy(a @ w13[:inter].T)).numpy() * (a @ w13[inter:].T)
        hq, hs = F.quantize_fp8_blocks_f32(h)
        y += mask[:, e:e + 1] * (F.dequantize_fp8_blocks_f32(hq, hs) @ w2.T)
    return y


@pytest.mark.parametrize("over", [dict(T=40, E=8, k=2, H=256, I=128), dict(T=13, E=16, k=4, H=384, I=256)])
def test_fp8_block_layer_equals_dense_bruteforce(syngen, over):
    layer = syngen.make_layer("tiny", seed=21, format="fp8_block", **over)
    assert layer["w13"].dtype == np.uint8 and layer["w13_s"].dtype == np.float32
    ref = _dense_bruteforce_fp8(layer)
    out = OL.forward(layer)
    assert np.max(np.abs(out["y"] - ref)) <= 1e-12 * np.abs(ref).max()
    checks.check_routing(out["ids"], out["w"], layer["w13"].shape[0])
    checks.check_permutation(out["ids"], out["offsets"], out["sorted_token"], out["row_of_slot"])
    toks = np.array([0, 5, over["T"] - 1])
    assert np.max(np.abs(OL.forward_tokens(layer, toks)["y"] - out["y"][toks])) <= 1e-13 * np.abs(ref).max()


def test_fp8_block_identical_experts_equal_one_dense_mlp(syngen):
    layer = syngen.make_layer("tiny", seed=22, format="fp8_block")
    for key in ("w13", "w13_s", "w2", "w2_s"):
        layer[key] = np.repeat(layer[key][:1], layer[key].shape[0], axis=0)
    out = OL.forward(layer)
    xq, xs = F.quantize_fp8_blocks_f32(F.decode_bf16(layer["x"]))
    a = torch.from_numpy(F.dequantize_fp8_blocks_f32(xq, xs))
    w13 = torch.from_numpy(F.decode_fp8_block(layer["w13"][0], layer["w13_s"][0]))
    inter = w13.shape[0] // 2
    h = torch.nn.functional.silu(a @ w13[:inter].T) * (a @ w13[inter:].T)
    hq, hs = F.quantize_fp8_blocks_f32(h.numpy())
    ref = F.dequantize_fp8_blocks_f32(hq, hs) @ F.decode_fp8_block(layer["w2"][0], layer["w2_s"][0]).T
    assert np.max(np.abs(out["y"] - ref)) <= 1e-12 * np.abs(ref).max()


def test_fp8_block_weights_are_the_mxfp4_normals(syngen):
    # both formats encode the same normals: decoded weights agree to within
    # the coarser format's rounding
    a = syngen.make_layer("tiny", seed=23, format="fp8_block")
    b = syngen.make_layer("tiny", seed=23)
    wa = F.decode_fp8_block(a["w13"][1], a["w13_s"][1])
    wb = F.decode_mxfp4(b["w13"][1], b["w13_s"][1])
    assert np.corrcoef(wa.ravel(), wb.ravel())[0, 1] > 0.98


def test_page_sizes_pin_the_fp8_block_byte_cost(syngen):
    g = json.load(open(os.path.join(GOLDEN, "page_sizes.json")))
    H, E, inter = g["flash_hidden"]["value"], g["flash_experts"]["value"], g["middle_width"]["value"]
    layers = g["flash_layers"]["value"] - g["flash_layers"]["dense_ffn_layers"]
    # bytes of one expert as the generator lays the two formats out (tiny shapes, scaled up)
    lay8 = syngen.make_layer("tiny", format="fp8_block")
    lay4 = syngen.make_layer("tiny")
    Ht, It = 256, 128
    per_w8 = sum(lay8[kk][0].nbytes for kk in ("w13", "w13_s", "w2", "w2_s")) / (3 * Ht * It)
    per_w4 = sum(lay4[kk][0].nbytes for kk in ("w13", "w13_s", "w2", "w2_s")) / (3 * Ht * It)
    assert per_w8 == 1 + 4 / (128 * 128) and per_w4 == 17 / 32
    weights = layers * E * 3 * H * inter
    router_bytes_saved = layers * E * H * (4 - 2)        # router F32 -> BF16
    saved = weights * (per_w8 - per_w4) + router_bytes_saved
    v25, v26 = g["flash_checkpoint_v25"], g["flash_checkpoint_v26"]
    # each printed size is rounded to 0.1 GB, so their difference is known to +-0.1 GB
    assert abs(saved - (v25["value"] - v26["value"])) <= v25["round_to"]
    # a wrong scale granularity (one per 128 values, or per 32) misses the printed difference
    for wrong in (1 + 4 / 128, 1 + 1 / 32):
        assert abs(weights * (wrong - per_w4) + router_bytes_saved - (v25["value"] - v26["value"])) > v25["round_to"]


# --- planted mistakes in the FP8 block-scaled functions -----------------------

_orig_decode = F.decode_fp8_block
_orig_quant = F.quantize_fp8_blocks_f32


def _mut_decode_transposed(codes, scales, block=128):
    sc = np.asarray(scales, dtype=np.float32)
    if sc.shape[0] == sc.shape[1]:
        sc = sc.T
    else:
        sc = sc.T.reshape(sc.shape)
    return _orig_decode(codes, sc, block)


def _mut_quant_truncate(v, block=128):
    v32 = np.asarray(v).astype(np.float32)
    R, C = v32.shape
    b = v32.reshape(R, C // block, block)
    amax = np.abs(b).max(-1)
    s = (amax / np.float32(448)).astype(np.float32)
    d = np.where(amax > 0, s, np.float32(1))
    q = (b / d[..., None]).astype(np.float64)
    grid = np.sort(np.unique(np.abs(_TORCH_E4M3[~np.isnan(_TORCH_E4M3)])))
    idx = np.searchsorted(grid, np.abs(q), side="right") - 1     # toward zero
    mag = grid[np.clip(idx, 0, len(grid) - 1)]
    return F.encode_e4m3_rne(np.copysign(mag, q)).reshape(R, C), s


def _mut_quant_scale(v, block=128):
    codes, s = _orig_quant(v, block)
    return codes, (s * np.float32(2)).astype(np.float32)


def _fp8_pins_pass(syngen):
    try:
        test_decode_fp8_block_elementwise()
        test_quantize_f32_matches_torch()
        test_quantize_f32_bruteforce_and_invariants()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name", ["decode_transposed", "quant_truncate", "quant_scale"])
def test_fp8_block_planted_mistakes_are_caught(syngen, monkeypatch, name):
    assert _fp8_pins_pass(syngen)
    fn = {"decode_transposed": ("decode_fp8_block", _mut_decode_transposed),
          "quant_truncate": ("quantize_fp8_blocks_f32", _mut_quant_truncate),
          "quant_scale": ("quantize_fp8_blocks_f32", _mut_quant_scale)}[name]
    monkeypatch.setattr(F, fn[0], fn[1])
    assert not _fp8_pins_pass(syngen), "planted mistake %r went unnoticed" % name
