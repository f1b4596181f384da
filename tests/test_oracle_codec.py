"""Pins for the oracle's encode, packing and decode (CPU).

  * packing: the page's own 2- and 4-bit formulas; a bit-string construction of the
    LSB-first stream at 3 bits; the dense payload size; round trips at 1..8 bits;
  * quantization: brute-force nearest centroid (first index on ties) on small inputs, and
    the decision-boundary count away from boundaries;
  * special cases: the zero vector, the identity rotation (a plain scalar quantizer);
  * statistics: the rotated-domain squared error equals the codebook's distortion integral
    within 5 standard errors; the relative error at d=128, 4 bits is the page's 0.10;
  * scale invariance: 50x inputs give the same codes and 50x norms;
  * byte accounting against the ratios the pages print.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import tq_inputs as ti
from oracle import accounting, codebook as cb, codec, rotation


def _pi(d, seed=42):
    return rotation.haar_rotation(ti.rotation_gaussian(d, seed).numpy())


# --- packing -------------------------------------------------------------------------

def test_two_and_four_bit_order_is_the_pages():
    rng = np.random.default_rng(1)
    c2 = rng.integers(0, 4, size=(5, 128))
    p2 = codec.pack_codes(c2, 2).astype(np.int64)
    q = c2.reshape(5, 32, 4)
    assert np.array_equal(p2, q[..., 0] | (q[..., 1] << 2) | (q[..., 2] << 4) | (q[..., 3] << 6))
    c4 = rng.integers(0, 16, size=(5, 128))
    p4 = codec.pack_codes(c4, 4).astype(np.int64)
    q = c4.reshape(5, 64, 2)
    assert np.array_equal(p4, q[..., 0] | (q[..., 1] << 4))


def _bitstring_pack(codes, bits):
    """Independent construction: write the codes as one string of bits, least significant
    bit of each code first, then read it 8 bits at a time, first bit = bit 0 of the byte."""
    rows = []
    for row in codes:
        s = "".join(format(int(v), "0%db" % bits)[::-1] for v in row)
        s += "0" * (-len(s) % 8)
        rows.append([int(s[i:i + 8][::-1], 2) for i in range(0, len(s), 8)])
    return np.array(rows, dtype=np.uint8)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("d", [8, 13, 64])
def test_pack_matches_bitstring_and_round_trips(bits, d):
    rng = np.random.default_rng(bits * 100 + d)
    codes = rng.integers(0, 2 ** bits, size=(7, d))
    packed = codec.pack_codes(codes, bits)
    assert packed.shape == (7, (d * bits + 7) // 8)
    assert np.array_equal(packed, _bitstring_pack(codes, bits))
    assert np.array_equal(codec.unpack_codes(packed, bits, d), codes)


def test_three_bit_codes_cross_bytes():
    codes = np.array([[7, 0, 0, 0, 0, 0, 0, 0], [0, 0, 5, 0, 0, 0, 0, 0]])
    p = codec.pack_codes(codes, 3)
    assert p.shape == (2, 3)                      # 8 codes -> 3 bytes
    assert list(p[0]) == [0b00000111, 0, 0]
    # code 2 = 0b101 fills stream bits 6, 7, 8: bit 6 of byte 0 and bit 0 of byte 1
    assert list(p[1]) == [0b01000000, 0b00000001, 0]


def test_payload_size_formula(golden_dir):
    fig = json.load(open(os.path.join(golden_dir, "page_figures.json")))["payload_bytes_formula"]
    for d in (64, 128, 256):
        for b in (2, 3, 4):
            assert codec.packed_row_bytes(d, b) == eval(fig["formula"], {"outer": 1, "dim": d, "bits": b})
    assert codec.packed_row_bytes(128, 3) == 48


# --- quantization ----------------------------------------------------------------------

@pytest.mark.parametrize("b", [2, 3, 4])
def test_nearest_centroid_by_brute_force(b):
    d = 16
    c = cb.codebook(d, b)
    x = ti.codec_check_inputs(40, d, seed=3).numpy()
    codes, n, y = codec.encode_codes(x, _pi(d, 5), c.centroids)
    for i in range(y.shape[0]):
        for j in range(d):
            best, best_k = math.inf, -1
            for k, ck in enumerate(c.centroids):
                dist = abs(y[i, j] - ck)
                if dist < best:            # strict: a tie keeps the first (lowest) index
                    best, best_k = dist, k
            assert codes[i, j] == best_k


def test_ties_go_to_the_lower_index():
    c = cb.codebook(128, 2)
    t = c.thresholds[2]
    pi = np.eye(4)
    # y = x / (n + eps): pick x so that y lands exactly on the middle boundary 0
    x = np.array([[0.0, 1.0, 0.0, 0.0]])
    codes, _, y = codec.encode_codes(x, pi, c.centroids)
    assert y[0, 0] == 0.0 and codes[0, 0] == 1          # between c_1 < 0 < c_2: lower wins
    assert t > 0


@pytest.mark.parametrize("b", [2, 3, 4])
def test_boundary_count_equals_argmin_away_from_boundaries(b):
    d = 128
    c = cb.codebook(d, b)
    x = ti.codec_check_inputs(512, d, seed=4).numpy()
    codes, _, y = codec.encode_codes(x, _pi(d), c.centroids)
    count = np.searchsorted(c.thresholds, y, side="left")   # #{k : t_k < y}
    delta = codec.boundary_distance(y, c.thresholds)
    far = delta > 1e-12
    assert np.array_equal(codes[far], count[far])


def test_zero_vector():
    for b in (2, 3, 4):
        c = cb.codebook(128, b)
        codes, n, _ = codec.encode_codes(np.zeros((1, 128)), _pi(128), c.centroids)
        assert n[0] == 0.0
        assert np.all(codes == 2 ** (b - 1) - 1)
        assert np.all(codec.decode_codes(codes, n, _pi(128), c.centroids) == 0.0)


def test_identity_rotation_is_a_scalar_quantizer():
    d, b = 64, 3
    c = cb.codebook(d, b)
    x = ti.codec_check_inputs(50, d, seed=9).numpy().astype(np.float64)
    packed, n = codec.encode(x, np.eye(d), c.centroids, b)
    xh = codec.decode(packed, n, np.eye(d), c.centroids, b, d)
    u = x / (np.linalg.norm(x, axis=1) + 1e-8)[:, None]
    idx = np.argmin(np.abs(u[..., None] - c.centroids), axis=-1)
    assert np.allclose(xh, c.centroids[idx] * n.astype(np.float64)[:, None], rtol=0, atol=1e-15)


# --- statistics --------------------------------------------------------------------------

@pytest.mark.parametrize("b", [2, 3, 4])
def test_rotated_squared_error_equals_the_distortion_integral(b):
    d = 128
    c = cb.codebook(d, b)
    x = ti.codec_check_inputs().numpy()
    codes, _, y = codec.encode_codes(x, _pi(d), c.centroids)
    err = (y - c.centroids[codes.astype(np.int64)]) ** 2
    per_vec = err.mean(axis=1)                  # vectors are independent
    se = per_vec.std(ddof=1) / math.sqrt(per_vec.size)
    assert abs(per_vec.mean() - c.mse) <= 5 * se, (per_vec.mean(), c.mse, se)


def test_relative_error_is_the_pages_ten_percent(golden_dir):
    fig = json.load(open(os.path.join(golden_dir, "page_figures.json")))["four_bit_example"]
    d, b = fig["head_dim"], fig["bits"]
    c = cb.codebook(d, b)
    expected = math.sqrt(d * c.mse)             # E||x - x_hat||^2 / ||x||^2 = d D for a Haar rotation
    assert round(expected, 2) == fig["relative_error"]
    # the page's 8-key example (its rotation is not ours, so agreement is statistical)
    x = ti.example_keys().numpy()
    packed, n = codec.encode(x, _pi(d), c.centroids, b)
    xh = codec.decode(packed, n, _pi(d), c.centroids, b, d)
    rel8 = np.linalg.norm(xh - x) / np.linalg.norm(x)
    assert abs(rel8 - expected) <= 0.015          # ~4 standard errors for 1024 coordinates
    # the 4096-vector workload rounds to the page's figure
    x = ti.codec_check_inputs().numpy()
    packed, n = codec.encode(x, _pi(d), c.centroids, b)
    xh = codec.decode(packed, n, _pi(d), c.centroids, b, d)
    rel = np.linalg.norm(xh - x) / np.linalg.norm(x)
    assert round(rel, 2) == fig["relative_error"]
    assert abs(rel - expected) <= 0.002


def test_transposed_rotation_in_decode_is_caught():
    # planted mistake, on the CPU: decoding with Pi^T instead of Pi must blow the error up
    d, b = 128, 4
    c = cb.codebook(d, b)
    x = ti.codec_check_inputs(256, d).numpy()
    pi = _pi(d)
    codes, n, _ = codec.encode_codes(x, pi, c.centroids)
    good = codec.decode_codes(codes, n, pi, c.centroids)
    bad = codec.decode_codes(codes, n, pi.T, c.centroids)
    assert np.linalg.norm(good - x) / np.linalg.norm(x) < 0.11
    assert np.linalg.norm(bad - x) / np.linalg.norm(x) > 1.0


def test_scale_invariance_of_codes_and_norms():
    d, b = 128, 3
    c = cb.codebook(d, b)
    x = ti.codec_check_inputs(512, d, seed=2).numpy()
    x50 = x.astype(np.float64) * 50               # exact in float64 (float32 x 50 needs 30 bits)
    c1, n1, y1 = codec.encode_codes(x, _pi(d), c.centroids)
    c2, n2, y2 = codec.encode_codes(x50, _pi(d), c.centroids)
    far = codec.boundary_distance(y1, c.thresholds) > 1e-9
    assert np.array_equal(c1[far], c2[far])
    ulp = np.spacing(n2.astype(np.float32))
    assert np.all(np.abs(n2.astype(np.float64) - 50.0 * n1.astype(np.float64)) <= ulp)


def test_storage_cast_rounds_to_nearest_even():
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8])    # halfway cases for bfloat16
    assert list(codec.cast(v, torch.bfloat16)) == [1.0, 1.0 + 4 * 2 ** -8]


def test_storage_cast_rounds_once():
    # just above a 16-bit halfway point by less than a float32 ulp: rounding through float32
    # first lands on the halfway point and then on the even neighbour (the wrong one)
    assert codec.cast(np.array([1.0 + 2 ** -8 + 2 ** -30]), torch.bfloat16)[0] == 1.0 + 2 ** -7
    assert codec.cast(np.array([-(1.0 + 2 ** -8 + 2 ** -30)]), torch.bfloat16)[0] == -(1.0 + 2 ** -7)
    assert codec.cast(np.array([1.0 + 2 ** -11 + 2 ** -40]), torch.float16)[0] == 1.0 + 2 ** -10


def test_storage_cast_float16_matches_numpy():
    # numpy converts float64 to float16 in one correctly rounded step (subnormals, overflow and
    # ties included): an independent implementation of the same definition
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(size=20000) * np.exp(rng.uniform(-25, 12, size=20000)),
                        [0.0, -0.0, 2.0 ** -25, 3 * 2.0 ** -25, 2.0 ** -24, 65504.0, 65519.9, 65520.0, -7e4,
                         np.inf, -np.inf]])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).astype(np.float64)
    got = codec.cast(x, torch.float16)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_storage_cast_bfloat16_is_nearest():
    # brute force: the result is a bfloat16 value (torch keeps it exactly), no other bfloat16
    # value is nearer, and exact ties go to the even significand
    rng = np.random.default_rng(6)
    x = rng.normal(size=5000) * np.exp(rng.uniform(-20, 20, size=5000))
    x = np.concatenate([x, 1.0 + (2 * np.arange(1, 200) + 1) * 2.0 ** -8])   # exact ties
    y = codec.cast(x, torch.bfloat16)
    yt = torch.from_numpy(y).to(torch.bfloat16)
    assert np.array_equal(yt.double().numpy(), y)                      # representable
    up = torch.nextafter(yt, torch.full_like(yt, float("inf"))).double().numpy()
    dn = torch.nextafter(yt, torch.full_like(yt, float("-inf"))).double().numpy()
    err = np.abs(y - x)
    assert np.all(err <= np.abs(up - x)) and np.all(err <= np.abs(dn - x))
    tie = (err == np.abs(up - x)) | (err == np.abs(dn - x))
    bits = yt.view(torch.int16).numpy()
    assert np.all(bits[tie] % 2 == 0)
    assert codec.cast(np.array([3.4e38 * 1.01]), torch.bfloat16)[0] == np.inf


# --- byte accounting -------------------------------------------------------------------

def test_ratios_the_pages_print(golden_dir):
    fig = json.load(open(os.path.join(golden_dir, "page_figures.json")))
    lo, hi = fig["compression_range_vs_fp16"]["value"]
    assert round(accounting.ratio_vs_16bit(128, 4), 1) == lo      # 256/68 = 3.76
    assert round(accounting.ratio_vs_16bit(128, 2), 1) == hi      # 256/36 = 7.11
    ex = fig["four_bit_example"]
    assert round(accounting.ratio_vs_16bit(128, 4, norm_bytes=2), 2) == ex["ratio_vs_bf16"]
    three = fig["three_bit_ratio"]["value"]
    assert round(accounting.ratio_vs_16bit(128, 3)) == three       # 4.92
    assert round(accounting.ratio_vs_16bit(128, 3, norm_bytes=2)) == three   # 5.12
    pre = fig["bit_presets"]
    assert accounting.average_bits(4, 2) == pre["K4V2"]["avg_bits"]
    assert accounting.average_bits(3, 2) == pre["K3V2"]["avg_bits"]
    assert accounting.average_bits(4, 3) == pre["K4V3"]["avg_bits"]
    assert abs(100 * accounting.saving_vs_16bit(4, 2) - pre["K4V2"]["saving_percent"]) < 1.5
    assert abs(100 * accounting.saving_vs_16bit(3, 2) - pre["K3V2"]["saving_percent"]) < 1.0


def test_ratio_table():
    table = {64: (3.56, 4.57, 6.40), 128: (3.76, 4.92, 7.11), 256: (3.88, 5.12, 7.53)}
    for d, row in table.items():
        for b, r in zip((4, 3, 2), row):
            assert round(16 * d / (b * d + 32), 2) == r
            assert round(accounting.ratio_vs_16bit(d, b), 2) == r
