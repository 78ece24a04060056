"""Exact decoders of the storage formats, and the FP8 block quantiser.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Formats (the teardown page, "Why Are the V2.6 Files Half the Size of V2.5?",
table row "Routed experts"; the vLLM recipe, "Overview"):
  * MXFP4 expert weights: each byte holds two 4-bit codes, and each group of
    32 values shares one 8-bit scale.  The 4-bit value is OCP e2m1, the scale is OCP
    e8m0 (a bare power of two).  Which nibble holds which element is not on
    the pages; the reading used here is element 2i in bits 3:0 and element
    2i+1 in bits 7:4.
  * FP8 compute: OCP e4m3 ("FN": bias 7, no infinities, 0x7f/0xff are NaN,
    largest finite 448).
  * BF16 router weights and activations: the top 16 bits of an IEEE binary32.
  * FP8 block-scaled expert weights (the earlier V2.5 expert format, same
    table): e4m3 codes; every 128-row by 128-column tile of a matrix carries a
    float32 multiplier of its own.

Every decoder maps codes to float64 exactly; none rounds.
"""

import numpy as np

__all__ = [
    "decode_bf16",
    "decode_e2m1",
    "decode_e4m3",
    "decode_e8m0",
    "unpack_fp4",
    "decode_mxfp4",
    "encode_e4m3_rne",
    "quantize_fp8_blocks",
    "dequantize_fp8_blocks",
    "decode_fp8_block",
    "quantize_fp8_blocks_f32",
    "dequantize_fp8_blocks_f32",
    "FP8_BLOCK",
    "MX_BLOCK",
    "E4M3_MAX",
]

FP8_BLOCK = 128   # activations: one scale per token per 128 channels
MX_BLOCK = 32     # MXFP4 weights: one scale per 32 values along K
E4M3_MAX = 448.0


def decode_bf16(bits):
    """bf16 bit patterns (uint16) -> float64: the pattern is the upper half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def decode_e2m1(nibble):
    """OCP e2m1 code (0..15) -> float64.

    Sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0.  Exponent 0 is
    subnormal: value m * 0.5.  Otherwise (1 + m/2) * 2**(e-1).  The positive
    grid is therefore {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
    """
    n = np.asarray(nibble).astype(np.int64)
    s = (n >> 3) & 1
    e = (n >> 1) & 3
    m = n & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


def decode_e8m0(byte):
    """OCP e8m0 scale byte -> float64 2**(b-127); 255 is NaN."""
    b = np.asarray(byte).astype(np.int64)
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


def decode_e4m3(byte):
    """OCP e4m3 ("FN") byte -> float64.

    Sign bit 7, exponent bits 6:3 (bias 7), mantissa bits 2:0.  Exponent 0 is
    subnormal: (m/8) * 2**-6.  Exponent 15 with mantissa 7 is NaN (no infinities).
    """
    b = np.asarray(byte).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    sub = (m / 8.0) * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    mag = np.where(e == 0, sub, nrm)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


_E2M1_VALUES = decode_e2m1(np.arange(16))   # the 16 values, indexed by code


def unpack_fp4(packed):
    """[..., K/2] uint8 -> [..., K] nibbles; element 2i is the low nibble, 2i+1 the high one."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def decode_mxfp4(codes, scales):
    """MXFP4 matrix -> float64.

    codes  [R, K/2] uint8 (two e2m1 values per byte)
    scales [R, K/32] uint8 (e8m0, one per 32 consecutive K elements of a row)
    returns [R, K] float64, each element = e2m1 value * its group's scale.
    """
    vals = _E2M1_VALUES[unpack_fp4(codes)]
    sc = decode_e8m0(scales)
    return vals * np.repeat(sc, MX_BLOCK, axis=-1)


def encode_e4m3_rne(v):
    """float64 values with |v| <= 448 -> e4m3 bytes, round to nearest, ties to even.

    The sign bit is copied from v (so -0 and negative values that round to
    zero give 0x80).  Rounding is done on the exact float64 value: the grid
    spacing in the binade of |v| is 2**(floor(log2|v|) - 3) for normal values
    and 2**-9 below 2**-6; dividing by a power of two is exact, and ``np.rint``
    rounds half to even.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(~np.isfinite(a)) or np.any(a > E4M3_MAX):
        raise ValueError("encode_e4m3_rne: input outside the finite e4m3 range")
    _, ex = np.frexp(a)                # a = f * 2**ex with f in [0.5, 1)
    binade = np.maximum(ex - 1, -6)    # floor(log2 a), clamped to the subnormal binade
    quantum = np.exp2(binade - 3.0)
    mag = np.rint(a / quantum) * quantum   # may carry into the next binade: recompute fields below
    # fields of the rounded magnitude
    _, ex2 = np.frexp(mag)
    e_unb = ex2 - 1
    is_sub = (mag < 2.0 ** -6)
    e_field = np.where(is_sub, 0, e_unb + 7)
    m_field = np.where(is_sub,
                       np.rint(mag / 2.0 ** -9),
                       np.rint((mag / np.exp2(e_unb.astype(np.float64)) - 1.0) * 8.0))
    e_field = np.where(mag == 0, 0, e_field)
    m_field = np.where(mag == 0, 0, m_field)
    code = (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    if np.any(code > 0x7E):
        raise ValueError("encode_e4m3_rne: rounded past the largest finite value")
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def _block_exponent(amax, fmt_max_mant, fmt_max_exp):
    """Smallest e with amax / 2**e <= fmt_max, for fmt_max = fmt_max_mant * 2**fmt_max_exp.

    Writing amax = f * 2**q with f in [1, 2): e = q - fmt_max_exp when
    f <= fmt_max_mant, else q - fmt_max_exp + 1.  amax == 0 gives e = -127.
    The result is clamped to the e8m0 range [-127, 127].
    """
    amax = np.asarray(amax, dtype=np.float64)
    frac, ex = np.frexp(amax)          # amax = frac * 2**ex, frac in [0.5, 1)
    f = 2.0 * frac
    q = ex - 1
    e = np.where(f <= fmt_max_mant, q - fmt_max_exp, q - fmt_max_exp + 1)
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_fp8_blocks(v, block=FP8_BLOCK):
    """Dynamic FP8 quantisation of rows, one power-of-two scale per `block` channels.

    The pages fix only "FP8 (block-wise e4m3)" with "a dynamic activation
    scheme" (vLLM recipe "Overview"; devupai "Self-Hosting").  The reading used
    here: for each row and each run of 128 channels, take amax = max |v|, pick
    the smallest power of two 2**e with amax / 2**e <= 448 (written as e8m0
    byte e + 127), and store round-to-nearest-even e4m3 codes of v / 2**e.
    The scaled block maximum then lies in (224, 448], so no code saturates.

    v: [R, C] float64 with C % block == 0
    returns (codes [R, C] uint8, scales [R, C/block] uint8)
    """
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    if C % block:
        raise ValueError("channel count must be a multiple of the block")
    blocks = v.reshape(R, C // block, block)
    amax = np.abs(blocks).max(axis=-1)
    e = _block_exponent(amax, 1.75, 8)        # 448 = 1.75 * 2**8
    scaled = np.ldexp(blocks, -e[..., None])  # exact: a power-of-two scaling
    codes = encode_e4m3_rne(scaled).reshape(R, C)
    return codes, (e + 127).astype(np.uint8)


def dequantize_fp8_blocks(codes, scales, block=FP8_BLOCK):
    """Inverse of the storage mapping: e4m3 code value times its block's e8m0 scale (float64)."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, C = codes.shape
    return decode_e4m3(codes) * np.repeat(decode_e8m0(scales), block, axis=-1).reshape(R, C)


# ---------------------------------------------------------------------------
# FP8 block-scaled experts: the earlier (V2.5) storage of the routed experts in
# the teardown's table "Why Are the V2.6 Files Half the Size of V2.5?" (e4m3
# codes, each square tile of 128 rows by 128 columns sharing a single float32
# multiplier); the vLLM recipe's "Overview" has the arithmetic done in e4m3
# with that block granularity.
# ---------------------------------------------------------------------------

def decode_fp8_block(codes, scales, block=FP8_BLOCK):
    """FP8 block-scaled matrix -> float64.

    codes  [R, K] uint8 e4m3
    scales [R/128, K/128] float32, one per 128 x 128 block
    returns [R, K] float64, element (i, j) = e4m3 value * scales[i // 128, j // 128].
    """
    vals = decode_e4m3(codes)
    sc = np.asarray(scales, dtype=np.float32).astype(np.float64)
    return vals * np.repeat(np.repeat(sc, block, axis=0), block, axis=1)


def quantize_fp8_blocks_f32(v, block=FP8_BLOCK):
    """Dynamic FP8 quantisation of rows with a float32 scale per row per `block` channels.

    The activation scheme that goes with FP8 block-scaled weights.  The pages
    name the weight format only; the reading used here is the plain
    amax-over-maximum rule, evaluated in binary32 because the scale is stored
    as a binary32 and the kernel decides every code in that precision:
      amax = max |v| over the run (v rounded to binary32 first),
      s    = amax / 448 (one binary32 division),
      code = e4m3 round-to-nearest-even of (v / s) (one binary32 division;
             the quotient can exceed 448 by one binary32 rounding, and any
             such value rounds to 448).
    A run with amax == 0 stores s = 0 and the codes of v / 1 (signed zeros).

    v: [R, C] (float64 or float32) with C % block == 0
    returns (codes [R, C] uint8, scales [R, C/block] float32)
    """
    v32 = np.asarray(v).astype(np.float32)
    R, C = v32.shape
    if C % block:
        raise ValueError("channel count must be a multiple of the block")
    blocks = v32.reshape(R, C // block, block)
    amax = np.abs(blocks).max(axis=-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    div = np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)
    q = (blocks / div[..., None]).astype(np.float32)
    q = np.clip(q, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = encode_e4m3_rne(q.astype(np.float64)).reshape(R, C)
    return codes, s


def dequantize_fp8_blocks_f32(codes, scales, block=FP8_BLOCK):
    """e4m3 code value times its run's float32 scale (float64)."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, C = codes.shape
    sc = np.asarray(scales, dtype=np.float32).astype(np.float64)
    return decode_e4m3(codes) * np.repeat(sc, block, axis=-1).reshape(R, C)
