"""Recent-token window: the newest tokens kept in full precision beside the compressed cache
(float64 oracle; test infrastructure only).

KV Cache API page (ginkgoq.github.io/TurboQuant/api/kv):
  * TurboQuantKVCache.prefill: a sequence no longer than the buffer stays whole in the
    buffer; otherwise all but the newest buffer_size tokens are compressed and the newest
    buffer_size stay in full precision.
  * TurboQuantKVCache.append: a decode token joins the buffer; once the buffer holds more
    than buffer_size tokens its oldest ones are flushed into the compressed store.
  * TurboQuantKVCache.attention_scores / attend: the scores are those of the compressed
    tokens followed by the exact dot products with the buffered keys, and the output is the
    weighted sum of the decompressed values plus that of the buffered values.
  TurboQuantV3.compress_kv on the same page splits a sequence the same way (the newest
  residual_window tokens stay in 16-bit form).

Readings (the flush body is not printed): a flush moves exactly the tokens beyond the
window, so after any sequence of appends a sequence of L tokens has positions
[0, L - min(L, R)) compressed and [L - min(L, R), L) in the window — the same split a prefill
of those L tokens makes. The softmax runs over all L tokens at once (the page applies one
softmax to the concatenated scores). Window tokens are held at the cache's own precision
(bf16/fp16 inputs are exact in float64).
"""

from __future__ import annotations

import numpy as np


def split(length: int, window: int):
    """(compressed count, window count) of a sequence of `length` tokens with window R."""
    if length < 0 or window < 0:
        raise ValueError("length and window must be >= 0")
    w = min(length, window)
    return length - w, w


def stream_split(lengths_appended, window: int):
    """Replay the page's buffer rule token by token: start empty, append chunks of the given
    sizes, flush the buffer down to `window` tokens after each append. Returns the final
    (compressed count, window count). Used to pin `split` against the streaming rule."""
    comp, buf = 0, 0
    for n in lengths_appended:
        if comp == 0 and buf == 0:
            # prefill of the first chunk: keep the newest `window` whole, compress the rest
            buf = min(n, window)
            comp = n - buf
            continue
        for _ in range(n):
            buf += 1
            if buf > window:
                comp += buf - window
                buf = window
    return comp, buf


def attention(q, k_hat, v_hat, k_win, v_win, lengths, window: int, scale: float):
    """o[b, h] = softmax over the L_b tokens of [compressed; window] scores, applied to
    [v_hat; v_win]; also lse. q [B, Hq, d]; k_hat / v_hat [B, Hkv, T, d] decoded compressed
    cache indexed by absolute position; k_win / v_win [B, Hkv, R, d] ring buffers, token at
    absolute position t held at slot t mod R. Query head h reads KV head h // (Hq / Hkv)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k_hat.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    o = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = int(lengths[b])
        c, w = split(L, window)
        if L == 0:
            continue
        for h in range(Hq):
            g = h // G
            keys = [np.asarray(k_hat[b, g, t], dtype=np.float64) for t in range(c)]
            vals = [np.asarray(v_hat[b, g, t], dtype=np.float64) for t in range(c)]
            for t in range(c, L):
                keys.append(np.asarray(k_win[b, g, t % window], dtype=np.float64))
                vals.append(np.asarray(v_win[b, g, t % window], dtype=np.float64))
            s = scale * (np.stack(keys) @ q[b, h])
            m = np.max(s)
            e = np.exp(s - m)
            o[b, h] = (e / np.sum(e)) @ np.stack(vals)
            lse[b, h] = m + np.log(np.sum(e))
    return o, lse
