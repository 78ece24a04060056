"""moe_forward_noalloc (the forward without a workspace: a static scratch array on
each device) against moe_forward with a caller workspace, through the C ABI.

Same kernels on the same inputs, so the outputs are compared bit for bit: two
calls in a row, the second with a smaller layer (the array keeps the first
call's intermediates; nothing of it has to start at zero), then the first
layer once more, and a bf16 output.
"""

import numpy as np
import pytest
import torch

import synthetic as S
from moe_testutil import dev, host, log, weights, problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import sparse_moe_expert_route_amd as m
    m.load()
    return m


def _inputs(moe, cfg, seed, over, packed=True):
    lay = S.make_layer(cfg, seed=seed, **over)
    p = problem(lay)
    return lay, p, weights(lay, packed)


def _both(moe, lay, p, W, out_dtype=0):
    T, H = lay["x"].shape
    x, wr = dev(lay["x"]), dev(lay["w_router"])
    b = None if lay["bias"] is None else dev(lay["bias"])
    dt = torch.float32 if out_dtype == 0 else torch.bfloat16
    y_ref = torch.empty(T, H, dtype=dt, device="cuda")
    moe.forward(p, x, wr, b, W, y_ref, moe.alloc_workspace(p), out_dtype)
    y = torch.full((T, H), float("nan"), dtype=dt, device="cuda")
    moe.forward_noalloc(p, x, wr, b, W, y, out_dtype)
    torch.cuda.synchronize()
    return host(y), host(y_ref)


def test_forward_noalloc_equals_forward_twice_the_second_smaller(moe):
    cases = [("pro_verify", 0, {}, True), ("tiny", 1, dict(T=40, E=16, k=4, bias="zipf"), False),
             ("pro_verify", 0, {}, True)]
    for cfg, seed, over, packed in cases:
        log("no-alloc forward %s %s" % (cfg, over))
        lay, p, W = _inputs(moe, cfg, seed, over, packed)
        y, y_ref = _both(moe, lay, p, W)
        assert np.all(np.isfinite(y))
        assert np.array_equal(y, y_ref)


@pytest.mark.parametrize("cfg,over", [("flash_decode", dict(E=64)), ("tiny", dict(T=300, H=512, I=512, E=8, k=4)),
                                      ("tiny", dict(format="fp8_block", T=50, E=100, k=6))])
def test_forward_noalloc_bf16_and_other_paths(moe, cfg, over):
    log("no-alloc forward bf16 %s %s" % (cfg, over))
    lay, p, W = _inputs(moe, cfg, 2, over)
    y, y_ref = _both(moe, lay, p, W, out_dtype=1)
    assert np.array_equal(y, y_ref)


def test_forward_noalloc_refuses_a_problem_beyond_the_array(moe):
    # 10,000 tokens x 8 slots at hidden 256: about 100 MiB of workspace, tiny weights
    lay = S.make_layer("tiny", seed=0, T=10000, k=8)
    p = problem(lay)
    assert moe.workspace_size(p) > moe.NOALLOC_SCRATCH_BYTES
    T, H = lay["x"].shape
    y = torch.empty(T, H, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.forward_noalloc(p, dev(lay["x"]), dev(lay["w_router"]), None, weights(lay), y)
    assert ei.value.status == 3
