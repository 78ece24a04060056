"""Routed MoE feed-forward layer for AMD Instinct MI355X: Python binding of the C ABI.

The computation lives in ``libmoe_mi355x.so`` (hand-written HIP for gfx950,
declared in ``include/moe.h``).  This module only marshals arguments: it
checks tensor dtypes/shapes, passes device pointers and torch's current HIP
stream to the library, and turns status codes into exceptions.  There is no
fallback: if the library is missing, every call raises.

Names follow the C ABI: ``prepack_weights``, ``route``, ``permute``,
``grouped_gemm_swiglu``, ``grouped_gemm1_swiglu``, ``grouped_gemm1_preact``,
``grouped_gemm2``, ``combine``, ``forward``.
"""

import ctypes
import os

import torch

__all__ = [
    "MoeError", "Problem", "ExpertWeights", "lib_path", "load", "abi_version", "workspace_size",
    "alloc_workspace", "prepack_weights", "route", "permute", "grouped_gemm_swiglu", "grouped_gemm1_swiglu",
    "grouped_gemm1_preact", "grouped_gemm2", "combine", "forward", "forward_noalloc", "update_selection_bias",
    "OUT_F32", "OUT_BF16",
    "WEIGHTS_CANONICAL", "WEIGHTS_PACKED", "EXPERTS_MXFP4", "EXPERTS_FP8_BLOCK", "EXPORTED_SYMBOLS",
    "scale_dtype", "error_words", "DEVERR_EXPERT_ID_RANGE", "DEVERR_EXPERT_ID_DUPLICATE", "DEVERR_EXPERT_OFFSETS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libmoe_mi355x.so")

OUT_F32 = 0
OUT_BF16 = 1
WEIGHTS_CANONICAL = 0
WEIGHTS_PACKED = 1
EXPERTS_MXFP4 = 0
EXPERTS_FP8_BLOCK = 1
DEVERR_EXPERT_ID_RANGE = 1
DEVERR_EXPERT_ID_DUPLICATE = 2
DEVERR_EXPERT_OFFSETS = 4

EXPORTED_SYMBOLS = [
    "moe_abi_version", "moe_status_string", "moe_workspace_size", "moe_error_words_offset", "moe_prepack_weights",
    "moe_route", "moe_permute",
    "moe_grouped_gemm_swiglu", "moe_grouped_gemm1_swiglu", "moe_grouped_gemm1_preact",
    "moe_grouped_gemm2", "moe_combine", "moe_forward", "moe_forward_noalloc", "moe_update_selection_bias",
]


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s (status %d)" % (fn, msg, status))
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("hidden", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("score_func", ctypes.c_int32), ("expert_format", ctypes.c_int32)]

    @classmethod
    def make(cls, T, H, I, E, k, score_func=0, expert_format=EXPERTS_MXFP4):
        return cls(int(T), int(H), int(I), int(E), int(k), int(score_func), int(expert_format))

    @property
    def N(self):
        return self.num_tokens * self.top_k


class _Weights(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p), ("layout", ctypes.c_int32)]


def _weight_specs(p):
    """(dtype, shape) of w13, w13_scale, w2, w2_scale for the problem's expert format."""
    E, H, I = p.num_experts, p.hidden, p.intermediate
    if p.expert_format == EXPERTS_FP8_BLOCK:
        return [(torch.uint8, (E, 2 * I, H)), (torch.float32, (E, 2 * I // 128, H // 128)),
                (torch.uint8, (E, H, I)), (torch.float32, (E, H // 128, I // 128))]
    return [(torch.uint8, (E, 2 * I, H // 2)), (torch.uint8, (E, 2 * I, H // 32)),
            (torch.uint8, (E, H, I // 2)), (torch.uint8, (E, H, I // 32))]


def scale_dtype(p):
    """dtype of the activation and h scales: uint8 (e8m0) or float32 (FP8 block-scaled experts)."""
    return torch.float32 if p.expert_format == EXPERTS_FP8_BLOCK else torch.uint8


class ExpertWeights:
    """Device tensors of the experts.  MXFP4 (uint8): w13 [E, 2I, H/2], w13_scale
    [E, 2I, H/32], w2 [E, H, I/2], w2_scale [E, H, I/32].  FP8 block-scaled: w13 [E, 2I, H]
    uint8, w13_scale [E, 2I/128, H/128] float32, w2 [E, H, I] uint8, w2_scale
    [E, H/128, I/128] float32.  ``layout`` says how the code bytes are ordered:
    WEIGHTS_CANONICAL (row-major) or WEIGHTS_PACKED (as written by ``prepack_weights``;
    same shapes)."""

    def __init__(self, w13, w13_scale, w2, w2_scale, layout=WEIGHTS_CANONICAL):
        self.w13, self.w13_scale, self.w2, self.w2_scale = w13, w13_scale, w2, w2_scale
        self.layout = int(layout)

    def check(self, p):
        for t, (dt, shape), name in zip((self.w13, self.w13_scale, self.w2, self.w2_scale), _weight_specs(p),
                                        ("w13", "w13_scale", "w2", "w2_scale")):
            _check(t, dt, shape, name)

    def struct(self):
        return _Weights(self.w13.data_ptr(), self.w13_scale.data_ptr(),
                        self.w2.data_ptr(), self.w2_scale.data_ptr(), self.layout)


_lib = None


def load():
    """Load the HIP library (torch is imported first so its HIP runtime is the one in use)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError("libmoe_mi355x.so is not built: run `python -m sparse_moe_expert_route_amd.build` "
                           "(there is no fallback implementation)")
    L = ctypes.CDLL(lib_path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER(Problem)
    W = ctypes.POINTER(_Weights)
    L.moe_abi_version.restype = ctypes.c_int
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_workspace_size.restype = sz
    L.moe_workspace_size.argtypes = [P]
    L.moe_error_words_offset.restype = sz
    L.moe_error_words_offset.argtypes = []
    L.moe_prepack_weights.argtypes = [P, W, vp, vp, vp, vp, vp]
    L.moe_route.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    L.moe_permute.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_grouped_gemm_swiglu.argtypes = [P, vp, vp, vp, W, vp, vp, sz, vp]
    L.moe_grouped_gemm1_swiglu.argtypes = [P, vp, vp, vp, W, vp, vp, vp, sz, vp]
    L.moe_grouped_gemm1_preact.argtypes = [P, vp, vp, vp, W, vp, vp, sz, vp]
    L.moe_grouped_gemm2.argtypes = [P, vp, vp, vp, W, vp, vp, sz, vp]
    L.moe_combine.argtypes = [P, vp, vp, vp, vp, i32, vp]
    L.moe_forward.argtypes = [P, vp, vp, vp, W, vp, i32, vp, sz, vp]
    L.moe_forward_noalloc.argtypes = [P, vp, vp, vp, W, vp, i32, vp]
    for name in EXPORTED_SYMBOLS:
        if name not in ("moe_abi_version", "moe_status_string", "moe_workspace_size", "moe_error_words_offset"):
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def abi_version():
    return load().moe_abi_version()


def _raise(fn, st):
    if st != 0:
        raise MoeError(fn, st, load().moe_status_string(st).decode())


def _check(t, dtype, shape, name):
    if t is None:
        raise ValueError("%s is required" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def workspace_size(p):
    n = load().moe_workspace_size(ctypes.byref(p))
    if n == 0:
        raise MoeError("moe_workspace_size", 1, "invalid problem")
    return n


def alloc_workspace(p, device="cuda"):
    return torch.empty(workspace_size(p), dtype=torch.uint8, device=device)


def error_words(ws, stream=None):
    """The two device error words of a workspace, as Python ints (word 0: expert ids of the
    latest permutation; word 1: expert offsets of the latest grouped GEMM).  Waits for the
    stream's work so far."""
    off = load().moe_error_words_offset()
    s = torch.cuda.current_stream() if stream is None else stream
    with torch.cuda.stream(s):
        w = ws[off:off + 8].cpu()
    v = w.view(torch.int32).tolist()
    return v[0] & 0xFFFFFFFF, v[1] & 0xFFFFFFFF


def prepack_weights(p, weights, w13_packed=None, w2_packed=None, w13_scale_packed=None, w2_scale_packed=None,
                    stream=None):
    """Reorder canonical expert codes and scales into the packed layout; returns packed
    ExpertWeights.  Output tensors are allocated unless given."""
    if weights.layout != WEIGHTS_CANONICAL:
        raise ValueError("prepack_weights needs canonical weights")
    weights.check(p)
    outs = []
    for given, src, name in ((w13_packed, weights.w13, "w13_packed"), (w13_scale_packed, weights.w13_scale, "w13_scale_packed"),
                             (w2_packed, weights.w2, "w2_packed"), (w2_scale_packed, weights.w2_scale, "w2_scale_packed")):
        t = torch.empty_like(src) if given is None else given
        _check(t, src.dtype, tuple(src.shape), name)
        outs.append(t)
    W = weights.struct()
    st = load().moe_prepack_weights(ctypes.byref(p), ctypes.byref(W), _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]),
                                    _ptr(outs[3]), _stream(stream))
    _raise("moe_prepack_weights", st)
    return ExpertWeights(outs[0], outs[1], outs[2], outs[3], WEIGHTS_PACKED)


def route(p, x, w_router, sel_bias, logits, topk_ids, topk_w, stream=None):
    """x [T,H] bf16 and w_router [E,H] bf16 (or both None: select on the given logits)."""
    T, H, E, k = p.num_tokens, p.hidden, p.num_experts, p.top_k
    if (x is None) != (w_router is None):
        raise ValueError("give both x and w_router, or neither")
    if x is not None:
        _check(x, torch.bfloat16, (T, H), "x")
        _check(w_router, torch.bfloat16, (E, H), "w_router")
    if sel_bias is not None:
        _check(sel_bias, torch.float32, (E,), "sel_bias")
    _check(logits, torch.float32, (T, E), "logits")
    _check(topk_ids, torch.int32, (T, k), "topk_ids")
    _check(topk_w, torch.float32, (T, k), "topk_w")
    st = load().moe_route(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(sel_bias), _ptr(logits),
                          _ptr(topk_ids), _ptr(topk_w), _stream(stream))
    _raise("moe_route", st)


def update_selection_bias(p, expert_offsets, step, sel_bias, stream=None):
    """One load-balancing step of the selection bias, in place (moe_update_selection_bias):
    experts below the mean load N / E get +step, those above it -step."""
    E = p.num_experts
    _check(expert_offsets, torch.int32, (E + 1,), "expert_offsets")
    _check(sel_bias, torch.float32, (E,), "sel_bias")
    st = load().moe_update_selection_bias(ctypes.byref(p), _ptr(expert_offsets), ctypes.c_float(step), _ptr(sel_bias),
                                          _stream(stream))
    _raise("moe_update_selection_bias", st)


def permute(p, topk_ids, x, expert_offsets, sorted_token, row_of_slot, xq_perm, xs_perm, ws, stream=None):
    T, H, E, k = p.num_tokens, p.hidden, p.num_experts, p.top_k
    N = T * k
    _check(topk_ids, torch.int32, (T, k), "topk_ids")
    _check(x, torch.bfloat16, (T, H), "x")
    _check(expert_offsets, torch.int32, (E + 1,), "expert_offsets")
    _check(sorted_token, torch.int32, (N,), "sorted_token")
    _check(row_of_slot, torch.int32, (N,), "row_of_slot")
    _check(xq_perm, torch.uint8, (N, H), "xq_perm")
    _check(xs_perm, scale_dtype(p), (N, H // 128), "xs_perm")
    st = load().moe_permute(ctypes.byref(p), _ptr(topk_ids), _ptr(x), _ptr(expert_offsets), _ptr(sorted_token),
                            _ptr(row_of_slot), _ptr(xq_perm), _ptr(xs_perm), _ptr(ws), ws.numel(),
                            _stream(stream))
    _raise("moe_permute", st)


def _gemm_inputs(p, act, act_scale, K, expert_offsets, weights):
    N = p.N
    _check(act, torch.uint8, (N, K), "activations")
    _check(act_scale, scale_dtype(p), (N, K // 128), "activation scales")
    _check(expert_offsets, torch.int32, (p.num_experts + 1,), "expert_offsets")
    weights.check(p)


def grouped_gemm_swiglu(p, xq_perm, xs_perm, expert_offsets, weights, y_perm, ws, stream=None):
    _gemm_inputs(p, xq_perm, xs_perm, p.hidden, expert_offsets, weights)
    _check(y_perm, torch.float32, (p.N, p.hidden), "y_perm")
    w = weights.struct()
    st = load().moe_grouped_gemm_swiglu(ctypes.byref(p), _ptr(xq_perm), _ptr(xs_perm), _ptr(expert_offsets),
                                        ctypes.byref(w), _ptr(y_perm), _ptr(ws), ws.numel(), _stream(stream))
    _raise("moe_grouped_gemm_swiglu", st)


def grouped_gemm1_swiglu(p, xq_perm, xs_perm, expert_offsets, weights, hq_perm, hs_perm, ws, stream=None):
    _gemm_inputs(p, xq_perm, xs_perm, p.hidden, expert_offsets, weights)
    _check(hq_perm, torch.uint8, (p.N, p.intermediate), "hq_perm")
    _check(hs_perm, scale_dtype(p), (p.N, p.intermediate // 128), "hs_perm")
    w = weights.struct()
    st = load().moe_grouped_gemm1_swiglu(ctypes.byref(p), _ptr(xq_perm), _ptr(xs_perm), _ptr(expert_offsets),
                                         ctypes.byref(w), _ptr(hq_perm), _ptr(hs_perm), _ptr(ws), ws.numel(),
                                         _stream(stream))
    _raise("moe_grouped_gemm1_swiglu", st)


def grouped_gemm1_preact(p, xq_perm, xs_perm, expert_offsets, weights, gu_perm, ws, stream=None):
    _gemm_inputs(p, xq_perm, xs_perm, p.hidden, expert_offsets, weights)
    _check(gu_perm, torch.float32, (p.N, 2 * p.intermediate), "gu_perm")
    w = weights.struct()
    st = load().moe_grouped_gemm1_preact(ctypes.byref(p), _ptr(xq_perm), _ptr(xs_perm), _ptr(expert_offsets),
                                         ctypes.byref(w), _ptr(gu_perm), _ptr(ws), ws.numel(), _stream(stream))
    _raise("moe_grouped_gemm1_preact", st)


def grouped_gemm2(p, hq_perm, hs_perm, expert_offsets, weights, y_perm, ws, stream=None):
    _gemm_inputs(p, hq_perm, hs_perm, p.intermediate, expert_offsets, weights)
    _check(y_perm, torch.float32, (p.N, p.hidden), "y_perm")
    w = weights.struct()
    st = load().moe_grouped_gemm2(ctypes.byref(p), _ptr(hq_perm), _ptr(hs_perm), _ptr(expert_offsets),
                                  ctypes.byref(w), _ptr(y_perm), _ptr(ws), ws.numel(), _stream(stream))
    _raise("moe_grouped_gemm2", st)


def combine(p, y_perm, row_of_slot, topk_w, y, out_dtype=OUT_F32, stream=None):
    T, H, k = p.num_tokens, p.hidden, p.top_k
    _check(y_perm, torch.float32, (T * k, H), "y_perm")
    _check(row_of_slot, torch.int32, (T * k,), "row_of_slot")
    _check(topk_w, torch.float32, (T, k), "topk_w")
    _check(y, torch.float32 if out_dtype == OUT_F32 else torch.bfloat16, (T, H), "y")
    st = load().moe_combine(ctypes.byref(p), _ptr(y_perm), _ptr(row_of_slot), _ptr(topk_w), _ptr(y),
                            int(out_dtype), _stream(stream))
    _raise("moe_combine", st)


def forward(p, x, w_router, sel_bias, weights, y, ws, out_dtype=OUT_F32, stream=None):
    T, H, E = p.num_tokens, p.hidden, p.num_experts
    _check(x, torch.bfloat16, (T, H), "x")
    _check(w_router, torch.bfloat16, (E, H), "w_router")
    if sel_bias is not None:
        _check(sel_bias, torch.float32, (E,), "sel_bias")
    weights.check(p)
    _check(y, torch.float32 if out_dtype == OUT_F32 else torch.bfloat16, (T, H), "y")
    w = weights.struct()
    st = load().moe_forward(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(sel_bias), ctypes.byref(w), _ptr(y),
                            int(out_dtype), _ptr(ws), ws.numel(), _stream(stream))
    _raise("moe_forward", st)


NOALLOC_SCRATCH_BYTES = 96 << 20   # MOE_NOALLOC_SCRATCH_BYTES of moe.h


def forward_noalloc(p, x, w_router, sel_bias, weights, y, out_dtype=OUT_F32, stream=None):
    """moe_forward without a workspace: the library's static scratch array on the current
    device holds the intermediates (problems up to NOALLOC_SCRATCH_BYTES of workspace).
    Calls that overlap on one device share that array."""
    T, H, E = p.num_tokens, p.hidden, p.num_experts
    _check(x, torch.bfloat16, (T, H), "x")
    _check(w_router, torch.bfloat16, (E, H), "w_router")
    if sel_bias is not None:
        _check(sel_bias, torch.float32, (E,), "sel_bias")
    weights.check(p)
    _check(y, torch.float32 if out_dtype == OUT_F32 else torch.bfloat16, (T, H), "y")
    w = weights.struct()
    st = load().moe_forward_noalloc(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(sel_bias), ctypes.byref(w),
                                    _ptr(y), int(out_dtype), _stream(stream))
    _raise("moe_forward_noalloc", st)
