"""Pins for the recent-token window oracle (CPU).

The split of a sequence into compressed and window tokens is pinned against the page's
buffer rule replayed token by token (prefill keeps the newest R, append flushes the oldest
beyond R), including chunked appends. The attention over [compressed; window] is pinned by
its two special cases — a window at least as long as the sequence gives exact attention on
the full-precision tokens (an independent softmax written with torch), a zero window gives
the compressed-cache oracle — and by a pure-Python loop on a tiny case.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as oatt, window as ow


@pytest.mark.parametrize("R", [0, 1, 5, 128])
@pytest.mark.parametrize("chunks", [[1] * 300, [200, 1, 1, 50, 3], [7], [128, 1], [129], [3, 400, 2]])
def test_split_follows_the_buffer_rule(R, chunks):
    L = sum(chunks)
    assert ow.stream_split(chunks, R) == ow.split(L, R)


def test_split_values():
    assert ow.split(100, 128) == (0, 100)
    assert ow.split(128, 128) == (0, 128)
    assert ow.split(129, 128) == (1, 128)
    assert ow.split(5000, 128) == (4872, 128)
    assert ow.split(7, 0) == (7, 0)
    with pytest.raises(ValueError):
        ow.split(-1, 3)


def _rand(B, Hq, Hkv, T, R, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, d))
    kh = rng.standard_normal((B, Hkv, T, d))
    vh = rng.standard_normal((B, Hkv, T, d))
    kw = rng.standard_normal((B, Hkv, max(R, 1), d))
    vw = rng.standard_normal((B, Hkv, max(R, 1), d))
    return q, kh, vh, kw, vw


def test_window_covering_the_sequence_is_exact_attention():
    B, Hq, Hkv, T, R, d = 2, 4, 2, 40, 64, 16
    q, kh, vh, kw, vw = _rand(B, Hq, Hkv, T, R, d, 1)
    lens = [40, 17]
    o, lse = ow.attention(q, kh, vh, kw, vw, lens, R, 1 / math.sqrt(d))
    for b, L in enumerate(lens):
        for h in range(Hq):
            g = h // 2
            K = torch.tensor(np.stack([kw[b, g, t % R] for t in range(L)]))
            V = torch.tensor(np.stack([vw[b, g, t % R] for t in range(L)]))
            s = (K @ torch.tensor(q[b, h])) / math.sqrt(d)
            ref = torch.softmax(s, 0) @ V
            assert np.allclose(o[b, h], ref.numpy(), atol=1e-12)
            assert abs(lse[b, h] - torch.logsumexp(s, 0).item()) < 1e-12


def test_zero_window_is_the_compressed_oracle():
    B, Hq, Hkv, T, d = 3, 6, 3, 50, 8
    q, kh, vh, kw, vw = _rand(B, Hq, Hkv, T, 0, d, 2)
    lens = [50, 0, 9]
    o, lse = ow.attention(q, kh, vh, kw, vw, lens, 0, 0.3)
    o2, lse2 = oatt.attention(q, kh, vh, 0.3, seq_lens=lens)
    assert np.allclose(o, o2, atol=1e-12)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse2))
    assert np.allclose(lse[~np.isneginf(lse)], lse2[~np.isneginf(lse2)], atol=1e-12)


def test_mixed_case_by_a_python_loop():
    B, Hq, Hkv, T, R, d = 1, 2, 1, 12, 4, 3
    q, kh, vh, kw, vw = _rand(B, Hq, Hkv, T, R, d, 3)
    L = 10   # positions 0..5 compressed, 6..9 in ring slots 2, 3, 0, 1
    o, lse = ow.attention(q, kh, vh, kw, vw, [L], R, 0.5)
    for h in range(Hq):
        toks = [(kh[0, 0, t], vh[0, 0, t]) for t in range(6)] + [(kw[0, 0, s], vw[0, 0, s]) for s in (2, 3, 0, 1)]
        sc = [0.5 * sum(k[i] * q[0, h][i] for i in range(d)) for k, _ in toks]
        m = max(sc)
        ex = [math.exp(x - m) for x in sc]
        tot = sum(ex)
        ref = [sum(ex[j] / tot * toks[j][1][i] for j in range(L)) for i in range(d)]
        assert np.allclose(o[0, h], ref, atol=1e-12)
        assert abs(lse[0, h] - (m + math.log(tot))) < 1e-12
