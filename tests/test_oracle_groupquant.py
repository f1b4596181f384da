"""Pins for the affine group quantization oracle (CPU).

The page's formulas are checked on hand-made groups whose results follow by inspection
(an exact ramp, a constant group hitting the scale floor, ties that round half to even, the
clamp), on the reconstruction bound |x - x_hat| <= scale/2 plus the float16 rounding of the
metadata, on the 2- and 4-bit byte order the page prints, and against a per-element Python
loop in float32 (numpy scalar float32 arithmetic is IEEE, like torch's).
"""

import numpy as np
import pytest

from oracle import codec, groupquant as gq


def test_exact_ramp_two_bits():
    x = np.tile(np.array([0.0, 1.0, 2.0, 3.0], dtype=np.float32), 8)[None, :]   # one group of 32
    q, s16, z16, s, z = gq.quantize(x, 2, 32)
    assert s[0, 0] == 1.0 and z[0, 0] == 0.0
    assert np.array_equal(q[0], np.tile([0, 1, 2, 3], 8))
    assert np.array_equal(gq.dequantize(q, s16, z16, 32), x)


def test_constant_group_hits_the_floor():
    x = np.full((1, 32), 2.5, dtype=np.float32)
    q, s16, z16, s, z = gq.quantize(x, 4, 32)
    assert s[0, 0] == np.float32(1e-12)
    assert np.all(q == 0)
    assert np.all(gq.dequantize(q, s16, z16, 32) == np.float32(np.float16(2.5)))


def test_ties_round_half_to_even_and_clamp():
    # one group: min 0, max 3 -> scale 1 at 2 bits; 0.5 -> 0, 1.5 -> 2, 2.5 -> 2
    vals = [0.0, 3.0, 0.5, 1.5, 2.5] + [1.0] * 27
    x = np.array(vals, dtype=np.float32)[None, :]
    q, *_ = gq.quantize(x, 2, 32)
    assert q[0, :5].tolist() == [0, 3, 0, 2, 2]
    assert q.max() <= 3


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("group", [32, 64, 128])
def test_reconstruction_bound(bits, group):
    rng = np.random.default_rng(bits * group)
    x = (rng.standard_normal((300, 128)) * rng.lognormal(size=(300, 1))).astype(np.float32)
    q, s16, z16, s, z = gq.quantize(x, bits, group)
    xh = gq.dequantize(q, s16, z16, group)
    g = x.reshape(300, -1, group)
    err = np.abs(xh.reshape(g.shape) - g)
    # half a step, plus float16 rounding of zero and of scale times the largest code, plus slack
    levels = (1 << bits) - 1
    bound = s[..., None] / 2 + np.abs(z[..., None]) * 2.0 ** -11 + levels * s[..., None] * 2.0 ** -11 + 1e-6
    assert np.all(err <= bound)


def test_codes_match_an_elementwise_float32_loop():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 64)).astype(np.float32)
    q, _, _, s, z = gq.quantize(x, 3, 32)
    for i in range(6):
        for gi in range(2):
            grp = x[i, gi * 32:(gi + 1) * 32]
            mn, mx = min(grp), max(grp)
            sc = max(np.float32(np.float32(mx - mn) / np.float32(7)), np.float32(1e-12))
            assert sc == s[i, gi] and mn == z[i, gi]
            for j, v in enumerate(grp):
                t = np.float32(np.float32(v - mn) / sc)
                r = int(np.rint(t))
                assert q[i, gi * 32 + j] == min(max(r, 0), 7)


def test_page_byte_order_two_and_four_bits():
    q = np.array([[1, 2, 3, 0] * 8], dtype=np.uint8)
    p2 = codec.pack_codes(q, 2)
    assert p2[0, 0] == (1 | 2 << 2 | 3 << 4 | 0 << 6)
    q4 = np.array([[5, 10] * 16], dtype=np.uint8)
    assert codec.pack_codes(q4, 4)[0, 0] == (5 | 10 << 4)


def test_encode_decode_round_trip_through_packing():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((10, 128)).astype(np.float32)
    for bits in (2, 3, 4, 8):
        packed, s16, z16 = gq.encode(x, bits, 32)
        assert packed.shape == (10, 128 * bits // 8)
        q, *_ = gq.quantize(x, bits, 32)
        assert np.array_equal(gq.decode(packed, s16, z16, bits, 128, 32), gq.dequantize(q, s16, z16, 32))


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        gq.quantize(np.zeros((1, 64)), 5, 32)
    with pytest.raises(ValueError):
        gq.quantize(np.zeros((1, 48)), 2, 32)
