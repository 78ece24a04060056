"""Host-side parts of bench.py that run without a GPU: the one-GPU guard and the
CPU-oracle baseline leg (its fields, its time split, and that the timing
wrappers it puts around two oracle functions are removed again)."""

import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.fixture(scope="module")
def bench():
    sys.path.insert(0, ROOT)
    import bench as B
    return B


def test_cpu_baseline_fields_and_split(bench):
    import synthetic as S
    from oracle import layer as OL
    dec, ffn = OL.decode_expert_matrix, OL.expert_ffn
    lay = S.make_layer("tiny", seed=0)
    out = bench.cpu_baseline(lay, types.SimpleNamespace(cpu_sample_tokens=8, config="tiny"), 64)
    # the oracle's functions are its own again
    assert OL.decode_expert_matrix is dec and OL.expert_ffn is ffn
    assert out["kind"] == "oracle" and out["unit"] == "tokens/s" and out["value"] > 0
    assert out["cores"] >= 1 and out["affinity_cores"] >= 1
    split = out["split_s"]
    assert set(split) == {"expert_decode", "expert_gemms_swiglu_requant", "rest"}
    assert all(v >= 0 for v in split.values())
    # the parts add up to the timed call (8 tokens in value tokens/s)
    total = 8 / out["value"]
    assert abs(sum(split.values()) - total) <= 0.01 + 0.05 * total
    assert "first 8 tokens of the tiny workload" in out["sample"]


def test_cpu_baseline_restores_the_oracle_after_an_error(bench):
    from oracle import layer as OL
    dec, ffn = OL.decode_expert_matrix, OL.expert_ffn
    with pytest.raises(Exception):
        bench.cpu_baseline({"x": None}, types.SimpleNamespace(cpu_sample_tokens=1, config="broken"), 1)
    assert OL.decode_expert_matrix is dec and OL.expert_ffn is ffn
