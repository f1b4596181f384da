"""QJL residual stage of keys and the asymmetric score estimator (float64 oracle; test
infrastructure only).

KV Cache API page (ginkgoq.github.io/TurboQuant/api/kv), TurboQuantCompressorV2:
  __init__: the MSE stage uses max(b - 1, 1) bits (the same Lloyd-Max codebook family); the
    sketch S is a d x d standard-normal draw from a CPU generator seeded seed + 10000.
  compress, in order: n = ||x||; codes of x / (n + 1e-8) rotated, as the MSE compressor;
    k_mse = (c[idx] Pi) * n; residual r = x - k_mse; residual norm ||r||; signs of S r,
    a zero projection counting as +1.
  asymmetric_attention_scores: <q, k> ~ <q, k_mse> + ||r|| sqrt(pi/2) / m <S q, signs>, m the
    number of sketch rows (d); the attention scale multiplies the sum (TurboQuantKVCache).
The module's header on the same page states the estimator is unbiased with variance O(1/d).
Decode attention over QJL keys takes the softmax of these scores and the weighted sum of the
decompressed values, as TurboQuantKVCache.attend does with its scores.

Readings: norms and residual norms are kept in float32 (the page stores float16; the MSE
codec here keeps float32 norms, reading 1 of the codec); k_mse uses the exact norm, as the
page's compress does (it multiplies by the unrounded norm).
"""

from __future__ import annotations

import math

import numpy as np

from . import attention as _att
from . import codec


def mse_bits(bits: int) -> int:
    return max(bits - 1, 1)


def encode(x, pi, S, centroids_mse):
    """Returns (codes uint8 [N, d], norms float32 [N], signs int8 [N, d] in {-1, +1},
    residual norms float32 [N], y float64 [N, d], projections float64 [N, d])."""
    x = np.asarray(x, dtype=np.float64)
    pi = np.asarray(pi, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    codes, _, y = codec.encode_codes(x, pi, centroids_mse)
    n = np.sqrt(np.sum(x * x, axis=1))
    c = np.asarray(centroids_mse, dtype=np.float64)
    k_mse = (c[codes.astype(np.int64)] @ pi) * n[:, None]
    r = x - k_mse
    rn = np.sqrt(np.sum(r * r, axis=1))
    proj = r @ S.T
    signs = np.where(proj >= 0, 1, -1).astype(np.int8)
    return codes, n.astype(np.float32), signs, rn.astype(np.float32), y, proj


def pack_signs(signs):
    """1 bit per coordinate, LSB-first (bit i of the stream = coordinate i), 1 = +1."""
    return codec.pack_codes((np.asarray(signs) > 0).astype(np.uint8), 1)


def unpack_signs(packed, d: int):
    return np.where(codec.unpack_codes(packed, 1, d) > 0, 1, -1).astype(np.int8)


def key_estimate(codes, norms, signs, rnorms, pi, S, centroids_mse):
    """Each key as the estimator sees it, [T, d]: the MSE reconstruction n_t (c[idx_t] Pi) plus
    the sketch's reconstruction of the residual, ||r_t|| sqrt(pi/2) / rows * S^T z_t, where z_t
    are the stored signs and rows is the number of sketch rows. The page's estimator
    <q, k_mse> + ||r|| sqrt(pi/2)/rows <S q, z> is the inner product of q with this vector
    (<S q, z> = <q, S^T z>)."""
    S = np.asarray(S, dtype=np.float64)
    rows = S.shape[0]
    c = np.asarray(centroids_mse, dtype=np.float64)
    recon = (c[np.asarray(codes).astype(np.int64)] @ np.asarray(pi, dtype=np.float64))
    recon *= np.asarray(norms, dtype=np.float64)[:, None]
    z = np.asarray(signs, dtype=np.float64)
    gain = np.asarray(rnorms, dtype=np.float64) * (math.sqrt(math.pi / 2) / rows)
    return recon + gain[:, None] * (z @ S)


def scores(q, codes, norms, signs, rnorms, pi, S, centroids_mse, scale: float):
    """s[i, t] = scale * <q_i, key_estimate_t> = scale * (<q_i, k_mse_t> + ||r_t|| sqrt(pi/2)/m
    <S q_i, signs_t>), m sketch rows. q [Q, d]; per-key arrays over T keys. Returns [Q, T]."""
    q = np.asarray(q, dtype=np.float64)
    return scale * (q @ key_estimate(codes, norms, signs, rnorms, pi, S, centroids_mse).T)


def cache_scores(q, codes, norms, signs, rnorms, pi, S, centroids_mse, scale: float, seq_lens=None):
    """QJL scores over a cache: q [B, Hq, d]; codes / signs [B, Hkv, T, d], norms / rnorms
    [B, Hkv, T]; query head h reads KV head h // (Hq / Hkv). Returns [B, Hq, T], -inf past len_b."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, T = np.asarray(norms).shape[1:3]
    G = Hq // Hkv
    out = np.full((B, Hq, T), -np.inf)
    for b in range(B):
        L = T if seq_lens is None else int(seq_lens[b])
        if L == 0:
            continue
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            out[b, hs, :L] = scores(q[b, hs], codes[b, g, :L], norms[b, g, :L], signs[b, g, :L],
                                    rnorms[b, g, :L], pi, S, centroids_mse, scale)
    return out


def attention(q, codes, norms, signs, rnorms, pi, S, centroids_mse, v_hat, scale: float, seq_lens=None):
    """Decode attention with QJL keys: softmax of cache_scores, then the weighted sum of v_hat
    [B, Hkv, T, d] (the plain attention's second half). Returns (o [B, Hq, d], lse [B, Hq])."""
    s = cache_scores(q, codes, norms, signs, rnorms, pi, S, centroids_mse, scale, seq_lens)
    return _att.attend(s, v_hat, seq_lens)
