"""Attention scores and decode attention over a compressed cache, float64 (oracle).

KV Cache API page (ginkgoq.github.io/TurboQuant/api/kv), TurboQuantKVCache.attention_scores:
scores are scale * <q, k_hat> with scale = 1/sqrt(head_dim) unless given, where k_hat is the
decompressed key; TurboQuantKVCache.attend: out = softmax(scores) @ v_hat, with v_hat the
decompressed values. The oracle is that definition written out: decode every cached vector
(codec.decode), take the dot products, a max-subtracted softmax, and the weighted sum.

Readings:
  * Grouped-query attention: query head h reads KV head floor(h / (Hq / Hkv)) (contiguous
    groups). The pages do not show the mapping.
  * A sequence of length 0 gives an output of zeros and lse = -inf.
  * Paged cache: a pool [num_blocks, Hkv, block_size, ...]; token t of sequence s lives in
    block block_table[s, t // block_size] at offset t % block_size. The pages name a paged
    layout but print none; this is the common one.
"""

from __future__ import annotations

import math

import numpy as np

from . import codec


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def decode_cache(packed, norms, pi, centroids, bits: int, d: int):
    """Decode a cache of any leading shape: packed [..., row], norms [...] -> [..., d] float64."""
    packed = np.asarray(packed)
    lead = packed.shape[:-1]
    flat = codec.decode(packed.reshape(-1, packed.shape[-1]), np.asarray(norms).reshape(-1),
                        pi, centroids, bits, d)
    return flat.reshape(*lead, d)


def _group(hq: int, hkv: int) -> int:
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    return hq // hkv


def scores(q, k_hat, scale: float, seq_lens=None):
    """s[b, h, t] = scale * <q[b, h], k_hat[b, h // G, t]> for t < len_b; -inf beyond."""
    q = np.asarray(q, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    B, Hq, d = q.shape
    _, Hkv, T, _ = k_hat.shape
    G = _group(Hq, Hkv)
    out = np.full((B, Hq, T), -np.inf)
    for b in range(B):
        L = T if seq_lens is None else int(seq_lens[b])
        for h in range(Hq):
            out[b, h, :L] = scale * (k_hat[b, h // G, :L] @ q[b, h])
    return out


def attend(s, v_hat, seq_lens=None):
    """o[b, h] = sum_t softmax(s[b, h, :L])_t v_hat[b, h // G, t]; lse = log sum_t exp(s[b, h, :L])."""
    s = np.asarray(s, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    B, Hq, T = s.shape
    Hkv, d = v_hat.shape[1], v_hat.shape[3]
    G = _group(Hq, Hkv)
    o = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = T if seq_lens is None else int(seq_lens[b])
        if L == 0:
            continue
        for h in range(Hq):
            row = s[b, h, :L]
            m = np.max(row)
            e = np.exp(row - m)
            tot = np.sum(e)
            o[b, h] = (e / tot) @ v_hat[b, h // G, :L]
            lse[b, h] = m + math.log(tot)
    return o, lse


def attention(q, k_hat, v_hat, scale: float, seq_lens=None):
    """o[b, h] = sum_t softmax(s[b, h])_t v_hat[b, h // G, t]; also lse = log sum_t exp(s)."""
    return attend(scores(q, k_hat, scale, seq_lens), v_hat, seq_lens)


def gather_paged(pool, block_table, seq_lens, block_size: int):
    """Per-sequence dense views of a paged pool [num_blocks, Hkv, block_size, ...].

    Returns a list with one array [Hkv, len_s, ...] per sequence.
    """
    pool = np.asarray(pool)
    out = []
    for s, L in enumerate(np.asarray(seq_lens)):
        L = int(L)
        t = np.arange(L)
        blocks = np.asarray(block_table)[s, t // block_size]
        out.append(pool[blocks, :, t % block_size].swapaxes(0, 1))
    return out


def paged_attention(q, k_seqs, v_seqs, scale: float):
    """Decode attention over ragged sequences given as lists of [Hkv, len, d] float64 arrays."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    o = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        kb = np.asarray(k_seqs[b])[None]
        vb = np.asarray(v_seqs[b])[None]
        ob, lb = attention(q[b:b + 1], kb, vb, scale)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse
