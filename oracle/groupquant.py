"""Affine group quantization of value vectors (oracle; test infrastructure only).

KV Cache API page (ginkgoq.github.io/TurboQuant/api/kv), quantize_values / dequantize_values
(also quantize_value_chunk / dequantize_value_chunk), in their order:
  1. work in float32 (the page casts the values to float32 first);
  2. split each vector into groups of `group_size` consecutive elements;
  3. per group: zero = min, scale = max((max - min) / (2^b - 1), floor) with floor 1e-12;
  4. q = clamp(round((x - zero) / scale), 0, 2^b - 1), round half to even (torch.round);
  5. pack the q's; keep scale and zero per group, stored in float16 (the page's default
     scale dtype);
  dequantize: x_hat = q * float(scale16) + float(zero16) in float32 (a product, then a sum).
Every step is an IEEE float32 operation, so the codes follow from the float32 data exactly;
numpy's float32 arithmetic is IEEE with round to nearest even, as the kernels must be.

Readings:
  * bits in {2, 3, 4, 8} (quantize_values); packing is the same LSB-first bitstream as the
    key codes (codec.pack_codes: the page's 2- and 4-bit order, dense at 3 bits; 8 bits = one
    byte per value). pack_unsigned itself is not printed.
  * The clamp floor is 1e-12 (quantize_values; quantize_value_chunk uses 1e-10).
  * Group sizes that divide d (d in {64, 128, 256}) need no padding.
"""

from __future__ import annotations

import numpy as np

from . import codec

FLOOR = np.float32(1e-12)


def quantize(x, bits: int, group: int = 32):
    """x [N, d] (any float; cast to float32). Returns (q uint8 [N, d], scale16, zero16 [N, d/group])
    plus the float32 scale and zero used for the codes."""
    if bits not in (2, 3, 4, 8):
        raise ValueError("bits must be 2, 3, 4 or 8")
    x = np.asarray(x, dtype=np.float32)
    N, d = x.shape
    if d % group:
        raise ValueError("group size must divide d")
    g = x.reshape(N, d // group, group)
    vmin = g.min(axis=-1)
    vmax = g.max(axis=-1)
    levels = np.float32((1 << bits) - 1)
    scale = np.maximum((vmax - vmin) / levels, FLOOR).astype(np.float32)
    zero = vmin
    t = (g - zero[..., None]) / scale[..., None]          # float32 subtract, float32 divide
    q = np.clip(np.rint(t), 0, levels).astype(np.uint8)   # rint: round half to even
    return q.reshape(N, d), scale.astype(np.float16), zero.astype(np.float16), scale, zero


def dequantize(q, scale16, zero16, group: int = 32):
    """x_hat = q * float32(scale16) + float32(zero16), float32."""
    q = np.asarray(q)
    N, d = q.shape
    s = np.asarray(scale16, dtype=np.float16).astype(np.float32)
    z = np.asarray(zero16, dtype=np.float16).astype(np.float32)
    qg = q.reshape(N, d // group, group).astype(np.float32)
    prod = (qg * s[..., None]).astype(np.float32)
    return (prod + z[..., None]).astype(np.float32).reshape(N, d)


def encode(x, bits: int, group: int = 32):
    """Packed rows (d*bits/8 bytes, LSB-first) and float16 scales / zeros [N, d/group]."""
    q, s16, z16, _, _ = quantize(x, bits, group)
    return codec.pack_codes(q, bits), s16, z16


def decode(packed, scale16, zero16, bits: int, d: int, group: int = 32):
    return dequantize(codec.unpack_codes(packed, bits, d), scale16, zero16, group)
