"""GPU parity of the selection-bias load-balancing step (moe_update_selection_bias)
against the oracle (oracle.layer.update_selection_bias, pinned in
tests/test_oracle_bias.py): bit-exact on given expert offsets, and bit-exact
step by step along a routing loop (select on given logits -> permute ->
update), whose load it must even out."""

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import layer as OL
from moe_testutil import dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import sparse_moe_expert_route_amd as m
    m.load()
    return m


def _counts(rng, E, N, kind):
    if kind == "random":
        return rng.multinomial(N, rng.dirichlet(np.ones(E)))
    if kind == "even":
        return np.full(E, N // E)
    if kind == "some_at_mean":
        # mean N / E = 64 exactly; a third of the experts sit on it, the rest pair off around it
        c = np.full(E, 64)
        for e in range(0, E - 1, 3):
            d = int(rng.integers(1, 64))
            c[e] += d
            c[e + 1] -= d
        return c
    if kind == "skewed":
        w = np.arange(1, E + 1, dtype=np.float64) ** -1.1
        return rng.multinomial(N, w / w.sum())
    if kind == "empty":
        return np.zeros(E, np.int64)
    raise ValueError(kind)


@pytest.mark.parametrize("E", [1, 8, 384, 512])
@pytest.mark.parametrize("kind", ["random", "even", "some_at_mean", "skewed", "empty"])
@pytest.mark.parametrize("step", [0.01, -0.25, 2.0 ** -30])
def test_bias_update_bitexact(moe, E, kind, step):
    rng = np.random.default_rng(E * 7 + len(kind))
    N = 64 * E if kind in ("even", "some_at_mean") else 131072
    counts = _counts(rng, E, N, kind)
    base = 1000 if kind == "random" else 0            # offsets need not start at 0
    off = np.concatenate([[base], base + np.cumsum(counts)]).astype(np.int32)
    b0 = rng.normal(size=E).astype(np.float32)
    b0[::5] = 1.0                                     # 1 +- 2^-30 rounds back to 1 in float32
    log("bias update E=%d %s step=%g" % (E, kind, step))
    p = moe.Problem.make(max(int(counts.sum()), 1), 256, 128, E, 1, 1)
    b = dev(b0)
    moe.update_selection_bias(p, dev(off), step, b)
    torch.cuda.synchronize()
    ref = OL.update_selection_bias(off, step, b0)
    assert np.array_equal(host(b).view(np.uint32), ref.view(np.uint32))


def test_bias_update_evens_out_a_routing_loop(moe):
    T, E, k, H = 512, 16, 2, 256
    rng = np.random.default_rng(7)
    logits = (rng.normal(size=(T, E)) + np.where(np.arange(E) < 2, 1.5, 0.0)).astype(np.float32)
    x = S.bf16_normal(11, 0, (T, H))
    p = moe.Problem.make(T, H, 128, E, k, 1)
    ws = moe.alloc_workspace(p)
    L = dev(logits)
    xd = dev(x)
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    st = torch.empty(T * k, dtype=torch.int32, device="cuda")
    ros = torch.empty(T * k, dtype=torch.int32, device="cuda")
    xq = torch.empty(T * k, H, dtype=torch.uint8, device="cuda")
    xs = torch.empty(T * k, H // 128, dtype=torch.uint8, device="cuda")
    bias = torch.zeros(E, dtype=torch.float32, device="cuda")
    ratios = []
    for it in range(60):
        moe.route(p, None, None, bias, L, ids, w)
        moe.permute(p, ids, xd, off, st, ros, xq, xs, ws)
        torch.cuda.synchronize()
        off_h, b_h = host(off), host(bias)
        counts = np.diff(off_h)
        assert counts.sum() == T * k
        ratios.append(counts.max() / counts.mean())
        moe.update_selection_bias(p, off, 0.01, bias)
        torch.cuda.synchronize()
        assert np.array_equal(host(bias).view(np.uint32), OL.update_selection_bias(off_h, 0.01, b_h).view(np.uint32))
    log("  max/mean load: first %.2f, last %.2f" % (ratios[0], ratios[-1]))
    assert ratios[0] > 3.5 and ratios[-1] < 1.2
