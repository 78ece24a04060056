"""Build the MoE HIP library (libmoe_mi355x.so) in-tree with hipcc for gfx950.

Each source is compiled to an object in parallel (one hipcc per file, under
_build/), then the objects are linked into the shared library.

Usage: python -m sparse_moe_expert_route_amd.build  (or build() from Python)
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
SOURCES = ["abi.cpp", "router.hip", "permute.hip", "prepack.hip", "expert_gemm.hip", "expert_gemm_tiled.hip",
           "expert_gemm_fp8.hip", "expert_gemm_fp8_tiled.hip", "combine.hip", "noalloc.hip"]
HEADERS = ["moe_launch.h", "moe_internal.h", "fp8_rows.h"]
# the microbenchmarks of the HBM and MFMA ceilings (include/moe_micro.h), a library of their own
MICRO_SOURCES = ["micro.hip"]
MICRO_LIB = os.path.join(HERE, "libmoe_micro.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    "--offload-arch=" + ARCH,
    # keep hipcc from emitting packed fp32 ops (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _filter(text):
    return "\n".join(l for l in text.splitlines()
                     if "packed-fp32-ops" not in l and "unknown target feature" not in l.lower())


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return res.returncode, _filter(res.stdout)


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    rc, out = _run([hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp])
    if rc != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc link failed:\n" + out)
    os.replace(tmp, lib)


def build(verbose=False, jobs=None):
    """Compile every HIP/C++ source and link the layer's library and the microbenchmark
    library; always rebuilds."""
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = SOURCES + MICRO_SOURCES
    objs, cmds = [], []
    for s in srcs:
        o = os.path.join(OBJ, os.path.splitext(s)[0] + ".o")
        objs.append(o)
        lang = ["-x", "hip"] if s.endswith(".hip") else []
        cmds.append([hipcc()] + HIPCC_FLAGS + inc + ["-c"] + lang + [os.path.join(CSRC, s), "-o", o])
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 4)), 8)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    errors = [(s, out) for s, (rc, out) in zip(srcs, results) if rc != 0]
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join("== %s ==\n%s" % e for e in errors))
    if verbose:
        for s, (_, out) in zip(srcs, results):
            if out.strip():
                print("== %s ==\n%s" % (s, out))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], MICRO_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
