"""The seeded input generator (CPU only).

Philox4x32-10 is checked against the known-answer vectors published with the
Random123 library (Salmon et al., SC'11); the weight encoding is checked to
decode within half a grid step of the normals it encodes.
"""

import numpy as np

from oracle import formats as F


def test_philox_known_answers(syngen):
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in kat:
        assert syngen.philox4x32_10(ctr, key).tolist() == want


def test_normals_moments_and_determinism(syngen):
    z = syngen.normal_f32(0, 9, 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3 and abs((z ** 4).mean() - 3) < 0.05
    assert np.array_equal(z[:1000], syngen.normal_f32(0, 9, 1000))
    assert not np.array_equal(z[:1000], syngen.normal_f32(1, 9, 1000))


def test_mxfp4_weights_encode_their_normals(syngen):
    rows, K = 64, 512
    codes, scales = syngen.mxfp4_normal(0, 123, rows, K, 0.02)
    v = syngen.normal_f32(0, 123, rows * K, 0.02).reshape(rows, K).astype(np.float64)
    d = F.decode_mxfp4(codes, scales)
    s = np.repeat(F.decode_e8m0(scales), 32, axis=1)
    # half of the largest e2m1 step (2, between 4 and 6) in scaled units
    assert np.all(np.abs(d - v) <= s * 1.0 + 1e-30)
    amax = np.abs(v).reshape(rows, K // 32, 32).max(-1)
    assert np.all(amax / F.decode_e8m0(scales) <= 6.0) and np.all(amax / F.decode_e8m0(scales) > 3.0)


def test_make_layer_shapes_and_bias(syngen):
    lay = syngen.make_layer("tiny", bias="zipf", E=16)
    assert lay["x"].shape == (64, 256) and lay["x"].dtype == np.uint16
    assert lay["w_router"].shape == (16, 256)
    b = lay["bias"]
    assert b.shape == (16,) and b.max() == 0.0 and np.all(b <= 0)
