"""Pins for the oracle's scores and decode attention (CPU).

  * special cases: one token gives o = v_hat; equal keys give the mean of v_hat; a
    zero-length sequence gives zeros and lse = -inf;
  * the rotated-domain forms the GPU uses (s = scale n <Pi q, c[idx]>, and
    o = Pi_V^T sum_t p_t n_t c_V[idx_t]) equal the direct definitions, because Pi is
    orthogonal;
  * softmax and lse against scipy's library routines;
  * a pure-Python triple loop on a tiny GQA case;
  * paged storage under a random block permutation equals dense storage.
"""

import math

import numpy as np
import pytest
from scipy import special

import tq_inputs as ti
from oracle import attention as att, codebook as cb, codec, rotation


def _pi(d, seed):
    return rotation.haar_rotation(ti.rotation_gaussian(d, seed).numpy())


def _cache(B, H, T, d, bits, seed, pi):
    x = ti.codec_check_inputs(B * H * T, d, seed=seed).numpy()
    c = cb.codebook(d, bits)
    packed, n = codec.encode(x, pi, c.centroids, bits)
    return packed.reshape(B, H, T, -1), n.reshape(B, H, T), c


def test_single_token_returns_the_value():
    d = 64
    pk, pv = _pi(d, 42), _pi(d, 542)
    kp, kn, ck = _cache(2, 2, 1, d, 4, 1, pk)
    vp, vn, cv = _cache(2, 2, 1, d, 2, 2, pv)
    q = ti.codec_check_inputs(2 * 4, d, seed=3).numpy().reshape(2, 4, d)
    kh = att.decode_cache(kp, kn, pk, ck.centroids, 4, d)
    vh = att.decode_cache(vp, vn, pv, cv.centroids, 2, d)
    o, lse = att.attention(q, kh, vh, att.default_scale(d))
    for h in range(4):
        assert np.allclose(o[:, h], vh[:, h // 2, 0], rtol=0, atol=1e-15)
        s = att.default_scale(d) * np.einsum("bd,bd->b", q[:, h], kh[:, h // 2, 0])
        assert np.allclose(lse[:, h], s, rtol=0, atol=1e-14)


def test_equal_keys_give_the_mean_value():
    d, T = 32, 9
    vh = ti.codec_check_inputs(T, d, seed=5).numpy().astype(np.float64)[None, None]
    kh = np.repeat(ti.codec_check_inputs(1, d, seed=6).numpy().astype(np.float64)[None, None], T, axis=2)
    q = ti.codec_check_inputs(1, d, seed=7).numpy().reshape(1, 1, d)
    o, lse = att.attention(q, kh, vh, 0.3)
    assert np.allclose(o[0, 0], vh[0, 0].mean(axis=0), rtol=0, atol=1e-14)
    assert abs(lse[0, 0] - (0.3 * float(q[0, 0] @ kh[0, 0, 0]) + math.log(T))) < 1e-12


def test_empty_sequence():
    q = np.ones((2, 2, 8))
    kh = np.ones((2, 1, 4, 8))
    o, lse = att.attention(q, kh, kh, 1.0, seq_lens=[0, 4])
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


def test_rotated_domain_forms_equal_the_definition():
    d, T, bk, bv = 128, 37, 4, 2
    pk, pv = _pi(d, 42), _pi(d, 542)
    kp, kn, ck = _cache(1, 1, T, d, bk, 11, pk)
    vp, vn, cv = _cache(1, 1, T, d, bv, 12, pv)
    q = ti.codec_check_inputs(4, d, seed=13).numpy().reshape(1, 4, d).astype(np.float64)
    scale = att.default_scale(d)
    kh = att.decode_cache(kp, kn, pk, ck.centroids, bk, d)
    vh = att.decode_cache(vp, vn, pv, cv.centroids, bv, d)
    s = att.scores(q, kh, scale)
    kidx = codec.unpack_codes(kp.reshape(T, -1), bk, d).astype(np.int64)
    vidx = codec.unpack_codes(vp.reshape(T, -1), bv, d).astype(np.int64)
    for h in range(4):
        qr = pk @ q[0, h]                                         # query rotated once
        s_rot = scale * kn.reshape(T).astype(np.float64) * (ck.centroids[kidx] @ qr)
        assert np.max(np.abs(s_rot - s[0, h])) <= 1e-12 * np.max(np.abs(s[0, h]))
    o, lse = att.attention(q, kh, vh, scale)
    for h in range(4):
        p = special.softmax(s[0, h])
        acc = (p * vn.reshape(T).astype(np.float64)) @ cv.centroids[vidx]   # rotated V domain
        assert np.max(np.abs(pv.T @ acc - o[0, h])) <= 1e-12 * np.max(np.abs(o[0, h]))
        assert abs(lse[0, h] - special.logsumexp(s[0, h])) <= 1e-12


def test_tiny_gqa_by_triple_loop():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, T, d = 2, 4, 2, 5, 3
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    lens = [5, 3]
    o, _ = att.attention(q, k, v, 0.7, seq_lens=lens)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            s = [0.7 * sum(q[b, h, i] * k[b, g, t, i] for i in range(d)) for t in range(lens[b])]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            for i in range(d):
                ref = sum(w[t] / z * v[b, g, t, i] for t in range(lens[b]))
                assert abs(o[b, h, i] - ref) < 1e-13


def test_paged_equals_dense():
    rng = np.random.default_rng(8)
    S, Hkv, Hq, d, bs = 3, 2, 4, 8, 4
    lens = [5, 12, 1]
    nblk = [(L + bs - 1) // bs for L in lens]
    perm = rng.permutation(sum(nblk))
    table = np.zeros((S, max(nblk)), dtype=np.int64)
    pool = np.zeros((sum(nblk), Hkv, bs, d))
    dense = [rng.standard_normal((Hkv, L, d)) for L in lens]
    off = 0
    for s, L in enumerate(lens):
        table[s, :nblk[s]] = perm[off:off + nblk[s]]
        off += nblk[s]
        for t in range(L):
            pool[table[s, t // bs], :, t % bs] = dense[s][:, t]
    got = att.gather_paged(pool, table, lens, bs)
    for s in range(S):
        assert np.array_equal(got[s], dense[s])
    q = rng.standard_normal((S, Hq, d))
    o, lse = att.paged_attention(q, got, got, 0.5)
    for s in range(S):
        o1, l1 = att.attention(q[s:s + 1], dense[s][None], dense[s][None], 0.5)
        assert np.allclose(o[s], o1[0], rtol=0, atol=1e-15) and np.allclose(lse[s], l1[0])
