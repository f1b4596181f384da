"""Pins for the oracle's QJL residual stage and asymmetric score estimator (CPU).

KV Cache API page (ginkgoq.github.io/TurboQuant/api/kv), TurboQuantCompressorV2: keys keep
max(b - 1, 1) MSE bits, the residual r = x - k_mse, its norm, and the signs of S r; the
score estimate is <q, k_mse> + ||r|| sqrt(pi/2) / m <S q, signs>. The module header on that
page calls the estimator unbiased with variance O(1/d).

The pins come from the mathematics, not from the oracle's own formula:
  * for s ~ N(0, I), E[<s, q> sign(<s, r>)] = sqrt(2/pi) <q, r> / ||r||, so the estimator's
    mean over sketch draws is <q, k> exactly (Monte Carlo over many S, within a few standard
    errors), and its variance over draws is ((pi/2) ||q||^2 ||r||^2 - <q, r>^2) / m — a
    wrong constant, a dropped ||r||, a wrong sign or m confused with d fails one of them;
  * a key that is its own MSE reconstruction has a zero residual and is scored exactly;
  * a zero projection counts as +1; signs pack one bit per coordinate, LSB-first;
  * the MSE stage is the plain codec at max(b - 1, 1) bits.
"""

import math

import numpy as np
import pytest

import tq_inputs as ti
from oracle import codebook, codec, qjl, rotation


def _pi(d, seed=3):
    return rotation.haar_rotation(ti.rotation_gaussian(d, seed).double().numpy())


@pytest.mark.parametrize("bits,expect", [(1, 1), (2, 1), (3, 2), (4, 3)])
def test_mse_bits(bits, expect):
    assert qjl.mse_bits(bits) == expect


def test_mse_stage_is_the_codec_at_b_minus_one_bits():
    d = 64
    pi = _pi(d)
    x = np.random.default_rng(1).standard_normal((50, d))
    S = ti.qjl_sketch_gaussian(d, 3).double().numpy()
    cb = codebook.codebook(d, qjl.mse_bits(3))
    codes, norms, signs, rn, y, proj = qjl.encode(x, pi, S, cb.centroids)
    c2, n2, _ = codec.encode_codes(x, pi, cb.centroids)
    assert np.array_equal(codes, c2)
    assert np.array_equal(norms, n2)
    # residual: x minus the codec's own decode at the exact norm, written out per row
    for i in range(5):
        k_mse = np.linalg.norm(x[i]) * (pi.T @ cb.centroids[codes[i].astype(int)])
        r = x[i] - k_mse
        assert abs(rn[i] - np.linalg.norm(r)) <= 1e-6 * max(1.0, np.linalg.norm(r))
        assert np.allclose(proj[i], S @ r, rtol=0, atol=1e-12)
        assert np.array_equal(signs[i], np.where(S @ r >= 0, 1, -1))


def test_zero_projection_counts_as_plus_one():
    d = 16
    pi = _pi(d)
    x = np.random.default_rng(2).standard_normal((4, d))
    S = np.random.default_rng(3).standard_normal((d, d))
    S[5] = 0.0                                   # row 5 projects every residual to 0
    cb = codebook.codebook(d, 1)
    _, _, signs, _, _, proj = qjl.encode(x, pi, S, cb.centroids)
    assert np.all(proj[:, 5] == 0.0)
    assert np.all(signs[:, 5] == 1)


def test_sign_packing_bit_order():
    signs = np.array([[1, -1, -1, 1, 1, 1, -1, 1, -1, -1, -1, -1, -1, -1, -1, 1]], dtype=np.int8)
    packed = qjl.pack_signs(signs)
    # byte 0 bits (LSB first): 1 0 0 1 1 1 0 1 -> 0b10111001; byte 1: 0000000 1 -> 0x80
    assert packed.tolist() == [[0b10111001, 0x80]]
    assert np.array_equal(qjl.unpack_signs(packed, 16), signs)


def test_zero_residual_scores_exactly():
    # With the 1-bit centroids +-1/sqrt(d), every sign vector c[idx] has unit length, so the
    # key x = n Pi^T c[idx] has y = c[idx] exactly (far from the threshold 0): the encode
    # returns idx, the residual vanishes to rounding and the estimate is <q, x>.
    d = 32
    pi = _pi(d)
    c = np.array([-1.0, 1.0]) / math.sqrt(d)
    rng = np.random.default_rng(4)
    idx = rng.integers(0, 2, size=(6, d))
    n = rng.uniform(0.5, 4.0, size=6)
    x = n[:, None] * (c[idx] @ pi)
    S = ti.qjl_sketch_gaussian(d, 9).double().numpy()
    codes, norms, signs, rn, _, _ = qjl.encode(x, pi, S, c)
    assert np.array_equal(codes, idx)
    assert np.all(rn <= 1e-13 * n)
    q = rng.standard_normal((3, d))
    s = qjl.scores(q, codes, norms, signs, rn, pi, S, c, 1.0)
    assert np.max(np.abs(s - q @ x.T)) <= 1e-6 * np.max(np.abs(q @ x.T))


def test_exact_reconstruction_gives_zero_residual():
    # one coordinate: d = 1 has y = +-1, far from the 1-bit threshold 0; k_mse = n * c * Pi
    d = 1
    pi = np.array([[1.0]])
    c = np.array([-1.0, 1.0])                   # a codebook with y itself as centroid
    x = np.array([[3.0], [-2.0]])
    S = np.array([[0.7]])
    codes, norms, signs, rn, _, _ = qjl.encode(x, pi, S, c)
    assert codes.tolist() == [[1], [0]]
    assert np.all(rn == 0.0)
    assert np.all(signs == 1)                    # projection of a zero residual is 0 -> +1
    q = np.array([[1.5], [-4.0]])
    s = qjl.scores(q, codes, norms, signs, rn, pi, S, c, 0.5)
    assert np.array_equal(s, 0.5 * (q @ x.T))


def _estimates(q, x, pi, cb, sketches):
    """Estimator of <q, x> for each sketch draw (Q = 1, T = 1)."""
    out = []
    for S in sketches:
        codes, norms, signs, rn, _, _ = qjl.encode(x[None], pi, S, cb.centroids)
        out.append(qjl.scores(q[None], codes, norms, signs, rn, pi, S, cb.centroids, 1.0)[0, 0])
    return np.array(out)


@pytest.mark.parametrize("d,m", [(16, 16), (16, 24)])
def test_unbiased_and_variance_over_sketch_draws(d, m):
    pi = _pi(d, 5)
    cb = codebook.codebook(d, 1)                 # b = 2 keys: large residual, strong signal
    rng = np.random.default_rng(6)
    x = rng.standard_normal(d)
    q = rng.standard_normal(d) + 0.8 * x         # correlated with the key
    draws = 4000
    sketches = rng.standard_normal((draws, m, d))
    est = _estimates(q, x, pi, cb, sketches)
    codes, norms, _, _, _, _ = qjl.encode(x[None], pi, sketches[0], cb.centroids)
    k_mse = (cb.centroids[codes[0]] @ pi) * float(norms[0])
    r = x - k_mse
    truth = float(q @ x)
    var = ((math.pi / 2) * (q @ q) * (r @ r) - (q @ r) ** 2) / m
    se = math.sqrt(var / draws)
    assert abs(est.mean() - truth) <= 4.0 * se
    # the MSE part alone is biased by <q, r>, far outside the Monte Carlo error
    assert abs(float(q @ k_mse) - truth) > 10.0 * se
    # sample variance of the draws: chi-square spread ~ sqrt(2 / draws) relative, 5 sigma
    assert abs(est.var(ddof=1) / var - 1.0) <= 5.0 * math.sqrt(2.0 / draws)


def test_variance_shrinks_like_one_over_m():
    d = 16
    pi = _pi(d, 7)
    cb = codebook.codebook(d, 1)
    rng = np.random.default_rng(8)
    x = rng.standard_normal(d)
    q = rng.standard_normal(d)
    v = []
    for m in (8, 64):
        est = _estimates(q, x, pi, cb, rng.standard_normal((1500, m, d)))
        v.append(est.var(ddof=1))
    assert 5.0 <= v[0] / v[1] <= 12.8            # 8 in expectation


def test_cache_attention_reduces_to_plain_attention_without_residual():
    # ||r|| = 0 removes the sketch term: QJL attention is the plain attention of the MSE keys
    from oracle import attention as oatt
    d, B, Hq, Hkv, T = 16, 2, 4, 2, 9
    rng = np.random.default_rng(11)
    pi = _pi(d, 13)
    cb = codebook.codebook(d, 2)
    codes = rng.integers(0, 4, size=(B, Hkv, T, d)).astype(np.uint8)
    norms = rng.uniform(0.5, 3.0, size=(B, Hkv, T)).astype(np.float32)
    signs = np.where(rng.random((B, Hkv, T, d)) < 0.5, -1, 1).astype(np.int8)
    S = rng.standard_normal((d, d))
    q = rng.standard_normal((B, Hq, d))
    v = rng.standard_normal((B, Hkv, T, d))
    lens = [9, 4]
    o, lse = qjl.attention(q, codes, norms, signs, np.zeros((B, Hkv, T), np.float32), pi, S, cb.centroids, v,
                           0.25, lens)
    khat = (cb.centroids[codes.astype(np.int64)] @ pi) * norms.astype(np.float64)[..., None]
    o2, lse2 = oatt.attention(q, khat, v, 0.25, seq_lens=lens)
    assert np.allclose(o, o2, rtol=0, atol=1e-12) and np.allclose(lse, lse2, rtol=0, atol=1e-12)
    # one token: the softmax weight is 1 and the output is that token's value
    o1, _ = qjl.attention(q, codes, norms, signs, norms, pi, S, cb.centroids, v, 0.25, [1, 1])
    for h in range(Hq):
        assert np.allclose(o1[:, h], v[:, h // (Hq // Hkv), 0], rtol=0, atol=1e-14)
