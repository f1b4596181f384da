"""Encode and decode of KV vectors, float64 (oracle; test infrastructure only).

Encode follows KV Cache API page (ginkgoq.github.io/TurboQuant/api/kv),
TurboQuantCompressorMSE.compress / MSECompressor.compress, in its order:
  1. work in floating point (float64 here; exact for float32/bfloat16/float16 inputs);
  2. n = ||x||_2 per vector;
  3. u = x / (n + 1e-8);
  4. y = u Pi^T (rows are vectors), i.e. y = Pi u;
  5. idx_i = argmin_k |y_i - c_k|, ties to the lowest k (torch argmin keeps the first);
  6. pack the codes.
Decode follows the same page, TurboQuantCompressorMSE.decompress: x_hat = (c[idx] Pi) * n,
cast to the output dtype.

Readings (the pages disagree or are silent):
  * Norm format: float32, rounded to nearest even (aitherkvcache landing page shows
    "[...] f32" norms; the KV Cache API page uses float16 and turbo-attn bfloat16).
  * Packing: an LSB-first bitstream. Code j occupies stream bits [j*b, j*b + b) and stream
    bit s is bit (s mod 8) of byte floor(s / 8). This is the order of the page's 2- and
    4-bit value packing (quantize_value_chunk: v0 | v1<<2 | v2<<4 | v3<<6 and v0 | v1<<4)
    and, at 3 bits, the dense bitstream whose size is (d*b + 7) // 8 bytes per vector
    (value_formula_nbytes). MSECompressor's MSB-first, 8//b-codes-per-byte layout is not
    used: it contradicts the former and cannot hold 3-bit codes densely.
  * A zero vector gives y = 0, which ties between the two middle centroids; the lower
    one wins, so every code is 2^(b-1) - 1 and the decode is 0.
"""

from __future__ import annotations

import numpy as np
import torch

EPS = 1e-8


def encode_codes(x, pi, centroids):
    """Steps 1-5. Returns (codes [N,d] uint8, norms float32 [N], y float64 [N,d])."""
    x = np.asarray(x, dtype=np.float64)
    pi = np.asarray(pi, dtype=np.float64)
    c = np.asarray(centroids, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=1))
    u = x / (n + EPS)[:, None]
    y = u @ pi.T
    codes = np.empty(y.shape, dtype=np.uint8)
    step = 2048   # bound the [rows, d, 2^b] distance array to a few hundred MB
    for s in range(0, y.shape[0], step):
        dist = np.abs(y[s:s + step, :, None] - c[None, None, :])
        codes[s:s + step] = np.argmin(dist, axis=-1)
    return codes, n.astype(np.float32), y


def encode_codes_norm_corrected(x, pi, centroids):
    """Encode with key-side norm correction: the stored norm is n / ||c[idx]||, so the decoded
    vector n / ||c[idx]|| * Pi^T c[idx] has the input's length n.

    Turbo Attention PyPI page, "The codec" table, "Norms" row (key-side norm correction keeps
    the decoded key's length). Reading: the codes are those of the plain encode; only the
    stored scalar changes, to n / ||c[idx]||_2 (float32, round to nearest even), which makes
    decode, scores and attention need no change. A zero vector keeps norm 0.
    Returns (codes, corrected norms float32, y).
    """
    codes, _, y = encode_codes(x, pi, centroids)
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=1))
    c = np.asarray(centroids, dtype=np.float64)
    cn = np.sqrt(np.sum(c[codes.astype(np.int64)] ** 2, axis=1))
    return codes, (n / cn).astype(np.float32), y


def boundary_distance(y, thresholds):
    """min_k |y_i - t_k|: how far each rotated coordinate is from a decision boundary."""
    y = np.asarray(y, dtype=np.float64)
    t = np.asarray(thresholds, dtype=np.float64)
    out = np.empty(y.shape)
    step = 4096
    for s in range(0, y.shape[0], step):
        out[s:s + step] = np.min(np.abs(y[s:s + step, :, None] - t[None, None, :]), axis=-1)
    return out


def packed_row_bytes(d: int, bits: int) -> int:
    """Bytes of one packed vector: (d*b + 7) // 8."""
    return (d * bits + 7) // 8


def pack_codes(codes, bits: int):
    """LSB-first bitstream packing of [N, d] codes into [N, (d*b+7)//8] bytes."""
    codes = np.asarray(codes, dtype=np.int64)
    n, d = codes.shape
    out = np.zeros((n, packed_row_bytes(d, bits)), dtype=np.int64)
    for j in range(d):
        for k in range(bits):
            s = j * bits + k
            out[:, s // 8] |= ((codes[:, j] >> k) & 1) << (s % 8)
    return out.astype(np.uint8)


def unpack_codes(packed, bits: int, d: int):
    """Inverse of pack_codes: [N, (d*b+7)//8] bytes -> [N, d] codes."""
    p = np.asarray(packed, dtype=np.int64)
    codes = np.zeros((p.shape[0], d), dtype=np.int64)
    for j in range(d):
        for k in range(bits):
            s = j * bits + k
            codes[:, j] |= ((p[:, s // 8] >> (s % 8)) & 1) << k
    return codes.astype(np.uint8)


def encode(x, pi, centroids, bits: int):
    """Full encode: returns (packed uint8 [N, d*b/8], norms float32 [N])."""
    codes, norms, _ = encode_codes(x, pi, centroids)
    return pack_codes(codes, bits), norms


def decode_codes(codes, norms, pi, centroids):
    """x_hat = (c[idx] Pi) * n in float64, from unpacked codes and float32 norms."""
    c = np.asarray(centroids, dtype=np.float64)
    chat = c[np.asarray(codes, dtype=np.int64)]
    return (chat @ np.asarray(pi, dtype=np.float64)) * np.asarray(norms, dtype=np.float64)[:, None]


def decode(packed, norms, pi, centroids, bits: int, d: int):
    """Full decode in float64 (cast with `cast` for a storage dtype)."""
    return decode_codes(unpack_codes(packed, bits, d), norms, pi, centroids)


# (significant bits, frexp exponent of the smallest normal, largest finite value) per format
_FORMATS = {
    torch.bfloat16: (8, -125, (2.0 - 2.0 ** -7) * 2.0 ** 127),
    torch.float16: (11, -13, 65504.0),
    torch.float32: (24, -125, float(np.finfo(np.float32).max)),
}


def cast(x, dtype: torch.dtype):
    """Round float64 values to a storage dtype and return them as float64.

    The decode's last step casts to the input's dtype (KV Cache API page,
    TurboQuantCompressorMSE.decompress); read as IEEE round-to-nearest-even of the exact value.
    Written from that definition: with x = m 2^e (frexp, m in [0.5, 1)), the spacing of the
    format's values near x is q = 2^(max(e, e_min) - p) for p significant bits (the max covers
    the subnormal range), and x rounds to rint(x / q) * q (rint breaks ties to even); a result
    beyond the largest finite value is infinite. One rounding step: converting float64 to float32
    first and then to the 16-bit format rounds twice and can land on the other neighbour.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == torch.float64:
        return x.copy()
    p, emin, big = _FORMATS[dtype]
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e, emin) - p)
    with np.errstate(invalid="ignore", over="ignore"):
        y = np.rint(x / q) * q
        y = np.where(np.abs(y) > big, np.copysign(np.inf, x), y)
    return np.where(np.isfinite(x), y, x)
