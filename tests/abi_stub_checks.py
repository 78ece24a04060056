"""Valid calls of every C-ABI entry point against the host-only build of the
library (tests/abi_host_stubs.cpp: the launchers only check their arguments
and count the call), run by tests/test_abi_sanitize.py under AddressSanitizer
and UndefinedBehaviorSanitizer.  It covers the host code on the paths a GPU
run takes (workspace carving, kernel choice, launch sequence) at every
workload's full size, including the largest (T*k = 131,072 rows, a 4 GiB
workspace), without touching a byte of device memory.

Not collected by the default test run (no test_ prefix): it needs the stub
library, which tests/test_abi_sanitize.py builds and loads.
"""

import ctypes

import pytest

import sparse_moe_expert_route_amd as moe

A = 1 << 20   # an aligned fake device address: the stubs never dereference it


@pytest.fixture(scope="module")
def lib():
    L = moe.load()
    assert hasattr(L, "moe_stub_calls"), "these checks need the host-only stub build"
    L.moe_stub_calls.argtypes = [ctypes.c_char_p]
    L.moe_stub_calls.restype = ctypes.c_int
    return L


def _calls(lib, *names):
    return {n: lib.moe_stub_calls(n.encode()) for n in names}


def _w(fmt_layout=0):
    return moe._Weights(A, A, A, A, fmt_layout)


NAMES = ["launch_router_logits", "launch_router_quant", "launch_topk", "launch_perm_small", "launch_perm_count",
         "launch_perm_scan", "launch_perm_scatter", "launch_quant_gather", "launch_tile_plan", "launch_expert_gemm",
         "launch_expert_gemm_tiled", "launch_expert_gemm_fp8", "launch_expert_gemm_fp8_tiled", "launch_combine",
         "launch_prepack", "launch_prepack_scales", "launch_bias_update", "hipMemcpyAsync"]


def _delta(lib, fn):
    before = _calls(lib, *NAMES)
    st = fn()
    after = _calls(lib, *NAMES)
    return st, {n: after[n] - before[n] for n in NAMES if after[n] != before[n]}


@pytest.mark.parametrize("T,H,I,E,k,fmt,expect", [
    # decode: router + FP8 copy of x in one launch, one-workgroup permutation, streaming GEMMs
    (64, 4096, 2048, 256, 8, 0, {"launch_router_quant": 1, "launch_topk": 1, "launch_perm_small": 1,
                                 "launch_expert_gemm": 2, "launch_combine": 1}),
    (128, 6144, 2048, 384, 8, 0, {"launch_router_quant": 1, "launch_topk": 1, "launch_perm_small": 1,
                                  "launch_expert_gemm": 2, "launch_combine": 1}),
    # prefill: LDS-tiled router, three-pass permutation, token-order quantisation, tile plan, tiled GEMMs
    (8192, 4096, 2048, 256, 8, 0, {"launch_router_logits": 1, "launch_topk": 1, "launch_perm_count": 1,
                                   "launch_perm_scan": 1, "launch_perm_scatter": 1, "launch_quant_gather": 1,
                                   "launch_tile_plan": 1, "launch_expert_gemm_tiled": 2, "launch_combine": 1}),
    (16384, 6144, 2048, 384, 8, 0, {"launch_router_logits": 1, "launch_topk": 1, "launch_perm_count": 1,
                                    "launch_perm_scan": 1, "launch_perm_scatter": 1, "launch_quant_gather": 1,
                                    "launch_tile_plan": 1, "launch_expert_gemm_tiled": 2, "launch_combine": 1}),
    # speculative verify: 256 tokens, decode router, multi-block permutation
    (256, 4096, 2048, 256, 8, 0, {"launch_router_quant": 1, "launch_topk": 1, "launch_perm_count": 1,
                                  "launch_perm_scan": 1, "launch_perm_scatter": 1, "launch_expert_gemm": 2,
                                  "launch_combine": 1}),
    # small tiled layer: the one-workgroup permutation writes the tile plan
    (100, 512, 512, 8, 4, 0, {"launch_router_quant": 1, "launch_topk": 1, "launch_perm_small": 1,
                              "launch_expert_gemm_tiled": 2, "launch_combine": 1}),
    # FP8 block-scaled experts
    (64, 4096, 2048, 256, 8, 1, {"launch_router_quant": 1, "launch_topk": 1, "launch_perm_small": 1,
                                 "launch_expert_gemm_fp8": 2, "launch_combine": 1}),
    (8192, 4096, 2048, 256, 8, 1, {"launch_router_logits": 1, "launch_topk": 1, "launch_perm_count": 1,
                                   "launch_perm_scan": 1, "launch_perm_scatter": 1, "launch_quant_gather": 1,
                                   "launch_tile_plan": 1, "launch_expert_gemm_fp8_tiled": 2, "launch_combine": 1}),
])
def test_forward_launch_sequence(lib, T, H, I, E, k, fmt, expect):
    p = moe.Problem.make(T, H, I, E, k, 0, fmt)
    ws = lib.moe_workspace_size(ctypes.byref(p))
    assert ws > 0
    w = _w(1)
    vp = ctypes.c_void_p
    st, d = _delta(lib, lambda: lib.moe_forward(ctypes.byref(p), vp(A), vp(A), None, ctypes.byref(w), vp(A), 0,
                                                vp(A), ws, None))
    assert st == 0
    assert d == expect


@pytest.mark.parametrize("T,H,I,E,k", [(64, 4096, 2048, 256, 8), (16384, 6144, 2048, 384, 8), (1, 128, 128, 1, 1),
                                       (3, 256, 128, 512, 8), (2000, 384, 640, 17, 3)])
def test_staged_entry_points(lib, T, H, I, E, k):
    p = moe.Problem.make(T, H, I, E, k)
    ws = lib.moe_workspace_size(ctypes.byref(p))
    vp = ctypes.c_void_p
    w = _w(0)
    calls = [
        lambda: lib.moe_route(ctypes.byref(p), vp(A), vp(A), vp(A), vp(A), vp(A), vp(A), None),
        lambda: lib.moe_route(ctypes.byref(p), None, None, None, vp(A), vp(A), vp(A), None),
        lambda: lib.moe_permute(ctypes.byref(p), *[vp(A)] * 7, vp(A), ws, None),
        lambda: lib.moe_grouped_gemm_swiglu(ctypes.byref(p), vp(A), vp(A), vp(A), ctypes.byref(w), vp(A), vp(A), ws,
                                            None),
        lambda: lib.moe_grouped_gemm1_swiglu(ctypes.byref(p), vp(A), vp(A), vp(A), ctypes.byref(w), vp(A), vp(A),
                                             vp(A), ws, None),
        lambda: lib.moe_grouped_gemm1_preact(ctypes.byref(p), vp(A), vp(A), vp(A), ctypes.byref(w), vp(A), vp(A), ws,
                                             None),
        lambda: lib.moe_grouped_gemm2(ctypes.byref(p), vp(A), vp(A), vp(A), ctypes.byref(w), vp(A), vp(A), ws, None),
        lambda: lib.moe_combine(ctypes.byref(p), vp(A), vp(A), vp(A), vp(A), 1, None),
        lambda: lib.moe_update_selection_bias(ctypes.byref(p), vp(A), ctypes.c_float(0.001), vp(A), None),
    ]
    for c in calls:
        assert c() == 0
    # one byte short of the workspace is refused before any launch
    before = _calls(lib, *NAMES)
    assert lib.moe_permute(ctypes.byref(p), *[vp(A)] * 7, vp(A), ws - 1, None) == 3
    assert _calls(lib, *NAMES) == before


@pytest.mark.parametrize("fmt,expect", [(0, {"launch_prepack": 2, "launch_prepack_scales": 2}),
                                        (1, {"launch_prepack": 2, "hipMemcpyAsync": 2})])
def test_prepack_launches(lib, fmt, expect):
    E, H, I = 384, 6144, 2048
    p = moe.Problem.make(1, H, I, E, 8, 0, fmt)
    w = moe._Weights(A, A + (1 << 34), A + (2 << 34), A + (3 << 34), 0)
    outs = [ctypes.c_void_p(A + (q << 34)) for q in (4, 5, 6, 7)]
    st, d = _delta(lib, lambda: lib.moe_prepack_weights(ctypes.byref(p), ctypes.byref(w), *outs, None))
    assert st == 0 and d == expect


@pytest.mark.parametrize("T,H,I,E,k", [(64, 4096, 2048, 256, 8), (256, 6144, 2048, 384, 8)])
def test_forward_noalloc_runs_the_forward_in_the_scratch_array(lib, T, H, I, E, k):
    """The same launches as moe_forward, with the scratch array as the workspace."""
    p = moe.Problem.make(T, H, I, E, k)
    ws = lib.moe_workspace_size(ctypes.byref(p))
    w = _w(1)
    vp = ctypes.c_void_p
    st, d_ref = _delta(lib, lambda: lib.moe_forward(ctypes.byref(p), vp(A), vp(A), None, ctypes.byref(w), vp(A), 0,
                                                    vp(A), ws, None))
    assert st == 0
    st, d = _delta(lib, lambda: lib.moe_forward_noalloc(ctypes.byref(p), vp(A), vp(A), None, ctypes.byref(w), vp(A),
                                                        0, None))
    assert st == 0 and d == d_ref


@pytest.mark.parametrize("E", [1, 256, 512])
def test_selection_bias_update_launches_once(lib, E):
    p = moe.Problem.make(64, 256, 128, E, 1, 1)
    vp = ctypes.c_void_p
    st, d = _delta(lib, lambda: lib.moe_update_selection_bias(ctypes.byref(p), vp(A), ctypes.c_float(0.5), vp(A),
                                                              None))
    assert st == 0
    assert d == {"launch_bias_update": 1}
