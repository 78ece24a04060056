"""CPU oracle for the routed MoE feed-forward layer (MiMo-V2.6 Flash/Pro backbone).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it.  It shares no code with the HIP library
(no kernels, headers, helpers, tables or constants); the only thing both sides
consume is the seeded input generator in ``synthetic/``, which holds none of
the layer's arithmetic.

Everything is written for clarity, not speed: formats are decoded exactly
into float64, every GEMM is a float64 numpy matmul, and the only fusion is the
one the definition itself states (SwiGLU between the two projections).

Sources (the pages; cited by page title and section):
  * "MiMo V2.6 Pro and Flash architecture teardown" (kgptalkie.com), sections
    "What Did Xiaomi Release?" (routed experts 256/8 and 384/8),
    "How Big Is Each Expert?" (router picks 8 experts; gate, up and down
    matrices, intermediate width 2,048), "Why Are the V2.6 Files Half the Size of V2.5?"
    (MXFP4: a byte holds two e2m1 codes, and each run of 32 values shares one e8m0 scale;
    BF16 router), "How Is the Backbone Built?" (no shared expert).
  * vLLM recipe "XiaomiMiMo/MiMo-V2.6-Pro-RL", section "Overview"
    (experts stored in MXFP4, the arithmetic done in block-scaled e4m3).
  * devupai.com "MiMo-V2.6-Flash", sections "No shared expert" and
    "Self-Hosting" (dynamic activation scheme).

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
something other than itself (library casts over all codes, brute force on tiny
inputs, closed forms, invariants, the pages' size arithmetic).  The one result
with no such pin is the whole layer on random weights beyond those checks: the
pages print no worked numeric example of a layer output, so that end-to-end
value is "parity unpinned" beyond the pins listed in the tests.
"""

from . import formats, layer, checks  # noqa: F401

__all__ = ["formats", "layer", "checks"]
