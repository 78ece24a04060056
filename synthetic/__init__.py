"""Seeded synthetic inputs for the routed MoE layer (shared by the tests, bench and smoke run).

This module draws inputs; it implements none of the layer's arithmetic.  The
bulk generation (normals, bf16 rounding, MXFP4 encoding of weights) is in
``gen.c`` and is built with gcc into ``libsyngen.so`` next to it.

Workloads (shapes from the teardown page: hidden 4,096 / 6,144 in "How Is the
Backbone Built?", 256 / 384 routed experts with 8 active in "What Did Xiaomi
Release?", a 2,048-wide expert middle in "How Big Is Each Expert?"):

  tiny                T=64,    H=256,  E=8,   k=2, I=128
  flash_decode        T=64,    H=4096, E=256, k=8, I=2048
  flash_prefill       T=8192,  H=4096, E=256, k=8, I=2048
  pro_decode          T=128,   H=6144, E=384, k=8, I=2048
  pro_skewed_prefill  T=16384, H=6144, E=384, k=8, I=2048, Zipf-like load
  flash_verify        T=256,   H=4096, E=256, k=8, I=2048  (speculative verify:
  pro_verify          T=256,   H=6144, E=384, k=8, I=2048   32 sequences x 8 positions)
  *_tp4               the same with I=512 (one GPU's share of a 4-way split)
  *_fp8               the same shapes with FP8 block-scaled experts (e4m3 codes,
                      one float32 scale per 128 x 128 block: the V2.5 expert
                      format in the teardown's "Why Are the V2.6 Files Half the
                      Size of V2.5?" table)

Distributions: activations N(0,1) rounded to bf16; router weights 0.02*N(0,1)
rounded to bf16; expert weights 0.02*N(0,1) encoded as MXFP4 (or, with
format="fp8_block", as e4m3 codes with scale amax/448 per 128 x 128 block,
from the same normals).  The skewed
workload adds a selection bias b_e = -0.55 * (0.02*sqrt(H)) * ln(r_e), with
r a seeded permutation of 1..E, so that expert load falls off roughly as
rank^-1.1 (a Zipf law, capped at T rows per expert).
"""

import ctypes
import os
import subprocess

import numpy as np

__all__ = [
    "CONFIGS", "config", "make_layer", "zipf_bias", "lib", "build",
    "philox4x32_10", "normal_f32", "bf16_normal", "mxfp4_normal", "fp8block_normal",
    "lossless_gemm_inputs", "lossless_fp8_gemm_inputs", "tie_logits", "random_ids",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libsyngen.so")

CONFIGS = {
    "tiny": dict(T=64, H=256, E=8, k=2, I=128, bias="zero"),
    "flash_decode": dict(T=64, H=4096, E=256, k=8, I=2048, bias="zero"),
    "flash_prefill": dict(T=8192, H=4096, E=256, k=8, I=2048, bias="zero"),
    "pro_decode": dict(T=128, H=6144, E=384, k=8, I=2048, bias="zero"),
    "pro_skewed_prefill": dict(T=16384, H=6144, E=384, k=8, I=2048, bias="zipf"),
    # one GPU's share of a 4-way tensor-parallel layer: I split four ways
    "flash_decode_tp4": dict(T=64, H=4096, E=256, k=8, I=512, bias="zero"),
    "pro_decode_tp4": dict(T=128, H=6144, E=384, k=8, I=512, bias="zero"),
    "flash_prefill_tp4": dict(T=8192, H=4096, E=256, k=8, I=512, bias="zero"),
    "pro_skewed_prefill_tp4": dict(T=16384, H=6144, E=384, k=8, I=512, bias="zipf"),
    # speculative-decoding verify step: a block of 8 positions (one known, seven
    # drafted) for each of 32 sequences
    "flash_verify": dict(T=256, H=4096, E=256, k=8, I=2048, bias="zero"),
    "pro_verify": dict(T=256, H=6144, E=384, k=8, I=2048, bias="zero"),
    # FP8 block-scaled experts (the earlier expert format)
    "flash_decode_fp8": dict(T=64, H=4096, E=256, k=8, I=2048, bias="zero", format="fp8_block"),
    "pro_decode_fp8": dict(T=128, H=6144, E=384, k=8, I=2048, bias="zero", format="fp8_block"),
    "flash_prefill_fp8": dict(T=8192, H=4096, E=256, k=8, I=2048, bias="zero", format="fp8_block"),
}

# stream ids of the counter-based generator
STREAM_X = 1
STREAM_WR = 2
STREAM_W13 = 1 << 20
STREAM_W2 = 2 << 20

_lib = None


def build(force=False):
    """Compile gen.c into libsyngen.so with gcc (OpenMP, no FMA contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, i64, f32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        L.syn_philox4x32_10.argtypes = [vp, vp, vp]
        L.syn_normal_f32.argtypes = [u64, u64, i64, f32, vp]
        L.syn_bf16_normal.argtypes = [u64, u64, i64, f32, vp]
        L.syn_mxfp4_normal.argtypes = [u64, u64, i64, i64, f32, vp, vp]
        L.syn_mxfp4_normal_batched.argtypes = [u64, u64, i64, i64, i64, f32, vp, vp]
        L.syn_fp8block_normal_batched.argtypes = [u64, u64, i64, i64, i64, f32, vp, vp]
        L.syn_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().syn_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def normal_f32(seed, stream, n, scale=1.0):
    out = np.empty(n, dtype=np.float32)
    lib().syn_normal_f32(seed, stream, n, scale, _ptr(out))
    return out


def bf16_normal(seed, stream, shape, scale=1.0):
    out = np.empty(shape, dtype=np.uint16)
    lib().syn_bf16_normal(seed, stream, out.size, scale, _ptr(out))
    return out


def mxfp4_normal(seed, stream, rows, K, scale=0.02, batch=None):
    """MXFP4 encoding of scale*N(0,1) matrices: codes [.., rows, K/2], scales [.., rows, K/32]."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    if batch is None:
        codes = np.empty((rows, K // 2), dtype=np.uint8)
        scales = np.empty((rows, K // 32), dtype=np.uint8)
        lib().syn_mxfp4_normal(seed, stream, rows, K, scale, _ptr(codes), _ptr(scales))
    else:
        codes = np.empty((batch, rows, K // 2), dtype=np.uint8)
        scales = np.empty((batch, rows, K // 32), dtype=np.uint8)
        lib().syn_mxfp4_normal_batched(seed, stream, batch, rows, K, scale, _ptr(codes), _ptr(scales))
    return codes, scales


def fp8block_normal(seed, stream, rows, K, scale=0.02, batch=1):
    """FP8 block-scaled encoding of scale*N(0,1) matrices (the normals of mxfp4_normal with the
    same arguments): codes [batch, rows, K] uint8 e4m3, scales [batch, rows/128, K/128] float32."""
    if rows % 128 or K % 128:
        raise ValueError("rows and K must be multiples of 128")
    codes = np.empty((batch, rows, K), dtype=np.uint8)
    scales = np.empty((batch, rows // 128, K // 128), dtype=np.float32)
    lib().syn_fp8block_normal_batched(seed, stream, batch, rows, K, scale, _ptr(codes), _ptr(scales))
    return codes, scales


def config(name_or_cfg, **over):
    cfg = dict(CONFIGS[name_or_cfg]) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(over)
    if isinstance(name_or_cfg, str):
        cfg.setdefault("name", name_or_cfg)
    cfg.setdefault("name", "custom")
    cfg.setdefault("bias", "zero")
    cfg.setdefault("format", "mxfp4")
    return cfg


def zipf_bias(E, H, seed=0):
    """Selection bias b_e = -0.55 * sigma_L * ln(r_e), r = seeded permutation of 1..E.

    sigma_L = 0.02*sqrt(H) is the standard deviation of a router logit under
    the generator's distributions; the bias equals 0.5*sigma_L*ln(p_e) + const
    with p_e proportional to r_e**-1.1.
    """
    r = 1 + np.random.default_rng([seed, 3]).permutation(E)
    sigma = 0.02 * np.sqrt(H)
    return (-0.55 * sigma * np.log(r)).astype(np.float32)


def make_experts(name_or_cfg, seed=0, **over):
    """The expert weights of a layer: dict(w13, w13_s, w2, w2_s).  They depend only on
    (H, I, E, format, seed), so layers that differ only in T or bias share them."""
    cfg = config(name_or_cfg, **over)
    H, E, inter = cfg["H"], cfg["E"], cfg["I"]
    out = {}
    if cfg["format"] == "fp8_block":
        out["w13"], out["w13_s"] = fp8block_normal(seed, STREAM_W13, 2 * inter, H, 0.02, batch=E)
        out["w2"], out["w2_s"] = fp8block_normal(seed, STREAM_W2, H, inter, 0.02, batch=E)
    else:
        out["w13"], out["w13_s"] = mxfp4_normal(seed, STREAM_W13, 2 * inter, H, 0.02, batch=E)
        out["w2"], out["w2_s"] = mxfp4_normal(seed, STREAM_W2, H, inter, 0.02, batch=E)
    return out


def make_layer(name_or_cfg, seed=0, experts=True, **over):
    """All inputs of one layer as numpy arrays (see the module docstring for distributions).

    experts=False skips the expert weights (for router-only uses); a dict made by
    make_experts for the same shapes and seed is used as given."""
    cfg = config(name_or_cfg, **over)
    T, H, E, k, inter = cfg["T"], cfg["H"], cfg["E"], cfg["k"], cfg["I"]
    layer = dict(cfg=cfg, top_k=k, format=cfg["format"])
    layer["x"] = bf16_normal(seed, STREAM_X, (T, H), 1.0)
    layer["w_router"] = bf16_normal(seed, STREAM_WR, (E, H), 0.02)
    if experts is True:
        layer.update(make_experts(cfg, seed))
    elif experts:
        layer.update(experts)   # expert arrays made earlier by make_experts for the same shapes and seed
    if cfg["bias"] == "zipf":
        layer["bias"] = zipf_bias(E, H, seed)
    elif cfg["bias"] == "zero":
        layer["bias"] = None
    else:
        layer["bias"] = np.asarray(cfg["bias"], dtype=np.float32)
    return layer


# ---------------------------------------------------------------------------
# Special inputs for exactness tests
# ---------------------------------------------------------------------------

# e4m3 bit patterns with exponent field 7 or 8 (values 1 .. 3.75 in steps of
# 1/8), either sign, plus zero.  Products of these with e2m1 values and small
# power-of-two scales, summed over K <= 8192 terms, stay exactly representable
# in binary32 (every term is a multiple of 2**-5 below 46, so every partial sum
# is a multiple of 2**-5 below 2**19).
_SMALL_E4M3 = np.array([0x00] + list(range(0x38, 0x48)) + list(range(0xB8, 0xC8)), dtype=np.uint8)


def lossless_gemm_inputs(rows, K, n_out, seed=0, batch=None):
    """Operands of an FP8 x MXFP4 product whose float32 accumulation is exact.

    returns (a_codes [rows, K] uint8 e4m3, a_scales [rows, K/128] uint8 in {127, 128},
             w_codes [.., n_out, K/2] uint8, w_scales [.., n_out, K/32] uint8 in {126, 127})
    """
    rng = np.random.default_rng([seed, 77])
    a = rng.choice(_SMALL_E4M3, size=(rows, K)).astype(np.uint8)
    a_s = rng.integers(127, 129, size=(rows, K // 128)).astype(np.uint8)
    wshape = (n_out, K // 2) if batch is None else (batch, n_out, K // 2)
    sshape = (n_out, K // 32) if batch is None else (batch, n_out, K // 32)
    w = rng.integers(0, 256, size=wshape).astype(np.uint8)
    w_s = rng.integers(126, 128, size=sshape).astype(np.uint8)
    return a, a_s, w, w_s


# e4m3 bit patterns with exponent field 7 (values 1 .. 1.875 in steps of 1/8),
# either sign, plus zero
_UNIT_E4M3 = np.array([0x00] + list(range(0x38, 0x40)) + list(range(0xB8, 0xC0)), dtype=np.uint8)


def lossless_fp8_gemm_inputs(rows, K, n_out, seed=0, batch=None):
    """Operands of an e4m3 x e4m3 product with float32 scales whose float32 accumulation is exact.

    Activations: codes from the set above with exponent field 7 or 8 (multiples of 1/8
    below 4), scales in {1, 2}; weights: exponent field 7 (multiples of 1/8 below 2),
    block scales in {1, 2}.  Every term is then a multiple of 2**-6 below 32, so for
    K <= 8192 every partial sum is a multiple of 2**-6 below 2**18: exact in binary32.

    returns (a_codes [rows, K] uint8, a_scales [rows, K/128] float32,
             w_codes [.., n_out, K] uint8, w_scales [.., n_out/128, K/128] float32)
    """
    rng = np.random.default_rng([seed, 78])
    a = rng.choice(_SMALL_E4M3, size=(rows, K)).astype(np.uint8)
    a_s = rng.integers(0, 2, size=(rows, K // 128)).astype(np.float32) + np.float32(1)
    wshape = (n_out, K) if batch is None else (batch, n_out, K)
    sshape = (n_out // 128, K // 128) if batch is None else (batch, n_out // 128, K // 128)
    w = rng.choice(_UNIT_E4M3, size=wshape).astype(np.uint8)
    w_s = rng.integers(0, 2, size=sshape).astype(np.float32) + np.float32(1)
    return a, a_s, w, w_s


def tie_logits(T, E, seed=0):
    """float32 logits drawn from a small set (with -0 and +0) so that many keys tie."""
    rng = np.random.default_rng([seed, 91])
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0, 2.0], dtype=np.float32)
    return rng.choice(vals, size=(T, E)).astype(np.float32)


def random_ids(T, E, k, seed=0, skew=None):
    """Distinct expert ids per token ([T, k] int32), optionally skewed towards low ids."""
    rng = np.random.default_rng([seed, 55])
    if skew is None:
        keys = rng.random((T, E))
    else:
        keys = rng.random((T, E)) * (1.0 + np.arange(E)[None, :]) ** skew
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)
