"""Pins of the oracle's format decoders and FP8 block quantiser (CPU only).

Each decoder is checked over every code against an independent source:
torch's own dtype casts (bfloat16, float8_e4m3fn, float8_e8m0fnu) or the
value table of the OCP Microscaling (MX) v1.0 specification for e2m1.
The quantiser is checked against torch's float32 -> e4m3 cast, a brute-force
nearest-grid search, and the invariants its definition implies.
"""

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import checks


def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = F.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_e4m3_decode_all_codes():
    b = np.arange(256, dtype=np.uint8)
    ours = F.decode_e4m3(b)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    assert np.nanmax(ours) == 448.0 and np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def test_e8m0_decode_all_codes():
    b = np.arange(256, dtype=np.uint8)
    ours = F.decode_e8m0(b)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


# OCP Microscaling Formats (MX) v1.0, FP4 (E2M1) value table, codes 0..15
_E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
               -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_decode_all_codes():
    ours = F.decode_e2m1(np.arange(16))
    assert np.array_equal(ours, np.array(_E2M1_TABLE))
    assert np.array_equal(np.signbit(ours), np.signbit(np.array(_E2M1_TABLE)))


def test_fp4_nibble_order():
    # reading: element 2i in the low nibble, element 2i+1 in the high nibble
    assert F.unpack_fp4(np.array([[0x21, 0xF7]], dtype=np.uint8)).tolist() == [[1, 2, 7, 15]]


def test_mxfp4_decode_matches_elementwise_definition():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, size=(3, 32), dtype=np.uint8)     # K = 64
    scales = rng.integers(120, 135, size=(3, 2), dtype=np.uint8)
    got = F.decode_mxfp4(codes, scales)
    for r in range(3):
        for c in range(64):
            byte = int(codes[r, c // 2])
            nib = (byte & 15) if c % 2 == 0 else (byte >> 4)
            want = _E2M1_TABLE[nib] * 2.0 ** (int(scales[r, c // 32]) - 127)
            assert got[r, c] == want


def _e4m3_finite_positive():
    vals = [(c, float(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).float()))
            for c in range(0x7F)]
    return vals


def test_e4m3_encode_matches_torch_cast_on_float32_values():
    rng = np.random.default_rng(2)
    mags = np.concatenate([
        rng.uniform(0, 448, 20000),
        np.exp2(rng.uniform(-12, 8.8, 20000)),
        rng.uniform(0, 2 ** -6, 5000),                     # subnormal range
    ]).astype(np.float32)
    mags = np.minimum(mags, np.float32(448))
    # exact midpoints between neighbouring codes (ties)
    grid = np.array([v for _, v in _e4m3_finite_positive()])
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    v = np.concatenate([mags, -mags, mids, -mids, grid.astype(np.float32)])
    ours = F.encode_e4m3_rne(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_bruteforce_float64():
    grid = _e4m3_finite_positive()
    codes = np.array([c for c, _ in grid])
    vals = np.array([v for _, v in grid])
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(0, 448, 3000), np.exp2(rng.uniform(-11, 8.8, 3000)),
                        (vals[1:] + vals[:-1]) / 2])
    x = np.minimum(x, 448.0)
    got = F.encode_e4m3_rne(x)
    for xi, gi in zip(x, got):
        d = np.abs(vals - xi)
        best = np.flatnonzero(d == d.min())
        want = codes[best[0]] if best.size == 1 else [c for c in codes[best] if c % 2 == 0][0]
        assert gi == want, (xi, gi, want)


def test_e4m3_encode_roundtrip_and_sign():
    b = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(F.encode_e4m3_rne(F.decode_e4m3(b)), b)
    assert F.encode_e4m3_rne(np.array([-1e-12, -0.0, 0.0]))[:].tolist() == [0x80, 0x80, 0x00]
    with pytest.raises(ValueError):
        F.encode_e4m3_rne(np.array([449.0]))


def test_fp8_block_quantiser_invariants():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((50, 512)) * np.exp2(rng.integers(-20, 20, size=(50, 1)))
    v[3, :128] = 0.0                                   # an all-zero block
    v[4, 128:256] = 448.0 * 2.0 ** 5                   # amax exactly 1.75 * 2^q
    v[5, 256:384] = 1.75000001 * 2.0 ** 3              # amax just above 1.75 * 2^q
    codes, scales = F.quantize_fp8_blocks(v)
    checks.check_fp8_blocks(codes, scales)
    e = scales.astype(np.int64) - 127
    amax = np.abs(v).reshape(50, 4, 128).max(-1)
    nz = amax > 0
    # smallest power of two: one step smaller would overflow 448
    assert np.all(amax[nz] / np.exp2(e[nz]) <= 448)
    assert np.all(amax[nz] / np.exp2(e[nz] - 1.0) > 448)
    assert scales[3, 0] == 0 and np.all(codes[3, :128] == 0)
    assert e[4, 1] == 5 and e[5, 2] == 3 - 7
    # reconstruction error <= half a code step of the scaled value
    dq = F.dequantize_fp8_blocks(codes, scales)
    s = np.repeat(np.exp2(e.astype(np.float64)), 128, axis=1)
    scaled = np.abs(v) / s
    _, ex = np.frexp(scaled)
    step = np.exp2(np.maximum(ex - 1, -6) - 3.0)
    assert np.all(np.abs(dq - v) / s <= step / 2 + 1e-300)
    # idempotent on values; on codes too wherever the rounded block maximum
    # stayed above 224 (a block whose maximum rounded down to exactly 224
    # re-quantises with a scale one step smaller and doubled codes)
    c2, s2 = F.quantize_fp8_blocks(dq)
    assert np.array_equal(F.dequantize_fp8_blocks(c2, s2), dq)
    rmax = np.abs(F.decode_e4m3(codes)).reshape(50, 4, 128).max(-1)
    keep = rmax > 224
    assert np.array_equal(s2[keep], scales[keep])
    assert np.array_equal(c2.reshape(50, 4, 128)[keep], codes.reshape(50, 4, 128)[keep])


def test_fp8_quantiser_mutations_are_caught():
    """Planted mistakes in the quantiser must fail the invariants above."""
    v = np.random.default_rng(5).standard_normal((8, 256))
    codes, scales = F.quantize_fp8_blocks(v)
    # scale one power of two too large -> block max falls to (112, 224]
    bad = F.encode_e4m3_rne(np.ldexp(v.reshape(8, 2, 128),
                                     -(scales.astype(np.int64)[..., None] - 127 + 1)).reshape(8, 256))
    with pytest.raises(AssertionError):
        checks.check_fp8_blocks(bad, scales)
