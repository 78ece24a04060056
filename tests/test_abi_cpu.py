"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects invalid arguments before touching the GPU (no compute calls here)."""

import ctypes
import os
import re

import pytest

import sparse_moe_expert_route_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.lib_path):
        from sparse_moe_expert_route_amd import build
        build.build()
    return moe.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert _declared() == sorted(moe.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_micro_library_exports_every_declared_symbol():
    """The microbenchmark library (include/moe_micro.h) loads without a GPU and exports its calls."""
    from sparse_moe_expert_route_amd import build as B
    if not os.path.exists(B.MICRO_LIB):
        B.build()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "moe_micro.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(moe_micro_[a-z0-9_]+)\s*\(", text)))
    assert names == ["moe_micro_hbm_read", "moe_micro_hbm_read_groups", "moe_micro_hbm_write", "moe_micro_mfma"]
    L = ctypes.CDLL(B.MICRO_LIB)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(lib):
    assert moe.abi_version() == 6
    for st, text in [(0, b"ok"), (1, b"invalid argument"), (3, b"workspace too small"), (4, b"HIP launch failure")]:
        assert lib.moe_status_string(st) == text
    assert lib.moe_status_string(99) == b"unknown status"


def _P(T=64, H=256, I=128, E=8, k=2, sf=0, fmt=0):
    return moe.Problem.make(T, H, I, E, k, sf, fmt)


@pytest.mark.parametrize("bad", [dict(H=100), dict(H=0), dict(I=64), dict(E=0), dict(E=513), dict(k=0),
                                 dict(k=9), dict(E=4, k=5), dict(T=-1), dict(sf=2), dict(fmt=2), dict(fmt=-1)])
def test_workspace_size_rejects_invalid_problems(lib, bad):
    args = dict(T=64, H=256, I=128, E=8, k=2, sf=0, fmt=0)
    args.update(bad)
    p = _P(**args)
    assert lib.moe_workspace_size(ctypes.byref(p)) == 0


def test_workspace_size_covers_intermediates(lib):
    for (T, H, I, E, k) in [(64, 256, 128, 8, 2), (64, 4096, 2048, 256, 8), (16384, 6144, 2048, 384, 8), (0, 256, 128, 8, 2)]:
        p = _P(T, H, I, E, k)
        n = lib.moe_workspace_size(ctypes.byref(p))
        N = T * k
        need = N * H * 4 + N * H + N * I + T * E * 4   # y_perm + x codes + h codes + logits
        assert n >= need and n % 256 == 0
        # float32 activation and h scales with FP8 block-scaled experts
        n8 = lib.moe_workspace_size(ctypes.byref(_P(T, H, I, E, k, 0, 1)))
        assert n8 >= need + N * (H + I) // 128 * 4 and n8 % 256 == 0 and n8 >= n


FAKE = 1 << 20   # an aligned non-null address; never dereferenced (every call below fails validation or is a no-op)


def _w(ptr=FAKE, layout=0):
    return moe._Weights(ptr, ptr, ptr, ptr, layout)


def test_invalid_arguments_rejected_before_launch(lib):
    vp = ctypes.c_void_p
    p = _P()
    big = 1 << 40
    # route: x without w_router
    assert lib.moe_route(ctypes.byref(p), vp(FAKE), None, None, vp(FAKE), vp(FAKE), vp(FAKE), None) == 1
    # route: misaligned output
    assert lib.moe_route(ctypes.byref(p), None, None, None, vp(FAKE + 4), vp(FAKE), vp(FAKE), None) == 1
    # permute: workspace too small / null / misaligned
    assert lib.moe_permute(ctypes.byref(p), *[vp(FAKE)] * 7, vp(FAKE), 16, None) == 3
    assert lib.moe_permute(ctypes.byref(p), *[vp(FAKE)] * 7, None, big, None) == 1
    assert lib.moe_permute(ctypes.byref(p), *[vp(FAKE)] * 7, vp(FAKE + 16), big, None) == 1
    # gemm entries: missing weights pointer
    w0 = _w(0)
    assert lib.moe_grouped_gemm_swiglu(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), ctypes.byref(w0), vp(FAKE),
                                       vp(FAKE), big, None) == 1
    assert lib.moe_grouped_gemm2(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), None, vp(FAKE), vp(FAKE), big,
                                 None) == 1
    # combine: bad dtype enum
    assert lib.moe_combine(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 7, None) == 1
    # forward: invalid problem
    pb = _P(H=200)
    w = _w()
    assert lib.moe_forward(ctypes.byref(pb), vp(FAKE), vp(FAKE), None, ctypes.byref(w), vp(FAKE), 0, vp(FAKE), big,
                           None) == 1
    assert lib.moe_forward(None, vp(FAKE), vp(FAKE), None, ctypes.byref(w), vp(FAKE), 0, vp(FAKE), big, None) == 1
    # unknown weight layout
    wl = _w(layout=7)
    assert lib.moe_forward(ctypes.byref(p), vp(FAKE), vp(FAKE), None, ctypes.byref(wl), vp(FAKE), 0, vp(FAKE), big,
                           None) == 1
    # prepack: source must be canonical; outputs aligned, non-null and not overlapping the inputs or each other
    M = 1 << 20
    outs = [vp(2 * M), vp(3 * M), vp(4 * M), vp(5 * M)]

    def prepack(problem, weights, o):
        return lib.moe_prepack_weights(ctypes.byref(problem), ctypes.byref(weights), *o, None)

    wp = _w(layout=1)
    assert prepack(p, wp, outs) == 1
    assert prepack(p, w, [vp(2 * M + 8)] + outs[1:]) == 1          # misaligned
    assert prepack(p, w, outs[:3] + [None]) == 1                      # null output
    assert prepack(p, w, [vp(FAKE + 16)] + outs[1:]) == 1           # overlaps the inputs
    assert prepack(p, w, outs[:1] + [vp(2 * M + 256)] + outs[2:]) == 1   # scales overlap the codes
    assert prepack(p, w0, outs) == 1
    assert prepack(pb, w, outs) == 1
    # FP8 block-scaled experts: sizes of that format (w13 is 8 * 256 * 256 bytes = 512 KiB here)
    p8 = _P(fmt=1)
    assert prepack(p8, w, [vp(FAKE + 384 * 1024)] + outs[1:]) == 1   # inside the e4m3 w13 input
    assert prepack(p8, wp, outs) == 1
    # selection-bias update: null offsets, misaligned or null bias, non-finite step
    f = ctypes.c_float
    assert lib.moe_update_selection_bias(ctypes.byref(p), None, f(0.01), vp(FAKE), None) == 1
    assert lib.moe_update_selection_bias(ctypes.byref(p), vp(FAKE), f(0.01), vp(FAKE + 4), None) == 1
    assert lib.moe_update_selection_bias(ctypes.byref(p), vp(FAKE), f(0.01), None, None) == 1
    assert lib.moe_update_selection_bias(ctypes.byref(p), vp(FAKE), f(float("nan")), vp(FAKE), None) == 1
    assert lib.moe_update_selection_bias(ctypes.byref(p), vp(FAKE), f(float("inf")), vp(FAKE), None) == 1
    assert lib.moe_update_selection_bias(ctypes.byref(pb), vp(FAKE), f(0.01), vp(FAKE), None) == 1
    # unknown scoring function
    ps = _P(sf=2)
    assert lib.moe_route(ctypes.byref(ps), None, None, None, vp(FAKE), vp(FAKE), vp(FAKE), None) == 2


def test_forward_noalloc_validates_before_touching_the_gpu(lib):
    """Invalid arguments and problems whose workspace exceeds the scratch array are refused,
    and zero tokens return at once, all before any HIP call (there is no GPU here)."""
    vp = ctypes.c_void_p
    w = _w()
    p = _P()
    assert lib.moe_forward_noalloc(None, vp(FAKE), vp(FAKE), None, ctypes.byref(w), vp(FAKE), 0, None) == 1
    assert lib.moe_forward_noalloc(ctypes.byref(p), vp(FAKE + 4), vp(FAKE), None, ctypes.byref(w), vp(FAKE), 0,
                                   None) == 1
    assert lib.moe_forward_noalloc(ctypes.byref(p), vp(FAKE), vp(FAKE), None, ctypes.byref(w), vp(FAKE), 5,
                                   None) == 1
    assert lib.moe_forward_noalloc(ctypes.byref(_P(T=0)), vp(FAKE), vp(FAKE), None, ctypes.byref(w), vp(FAKE), 0,
                                   None) == 0
    # Flash prefill needs far more than the 96 MiB array; Pro verify (64.6 MiB) fits
    big = _P(T=8192, H=4096, I=2048, E=256, k=8)
    assert lib.moe_workspace_size(ctypes.byref(big)) > moe.NOALLOC_SCRATCH_BYTES
    assert lib.moe_forward_noalloc(ctypes.byref(big), vp(FAKE), vp(FAKE), None, ctypes.byref(w), vp(FAKE), 0,
                                   None) == 3
    fits = _P(T=256, H=6144, I=2048, E=384, k=8)
    assert lib.moe_workspace_size(ctypes.byref(fits)) <= moe.NOALLOC_SCRATCH_BYTES


def test_zero_tokens_is_a_no_op(lib):
    vp = ctypes.c_void_p
    p = _P(T=0)
    big = 1 << 40
    w = _w()
    assert lib.moe_route(ctypes.byref(p), None, None, None, vp(FAKE), vp(FAKE), vp(FAKE), None) == 0
    assert lib.moe_permute(ctypes.byref(p), *[vp(FAKE)] * 7, vp(FAKE), big, None) == 0
    assert lib.moe_grouped_gemm_swiglu(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), ctypes.byref(w), vp(FAKE),
                                       vp(FAKE), big, None) == 0
    assert lib.moe_combine(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 0, None) == 0
    assert lib.moe_forward(ctypes.byref(p), vp(FAKE), vp(FAKE), None, ctypes.byref(w), vp(FAKE), 1, vp(FAKE), big,
                           None) == 0


def test_binding_refuses_host_tensors():
    import torch
    p = _P()
    with pytest.raises(ValueError):
        moe.route(p, None, None, None, torch.zeros(64, 8), torch.zeros(64, 2, dtype=torch.int32),
                  torch.zeros(64, 2), stream=None)
