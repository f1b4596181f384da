"""Byte accounting of the compressed format (oracle; test infrastructure only).

A vector of head dimension d at b bits is stored as (d*b + 7)//8 code bytes (the dense
bitstream size of value_formula_nbytes, KV Cache API page, ginkgoq.github.io/TurboQuant/api/kv)
plus one norm (4 bytes here: float32, per the aitherkvcache landing page's "[...] f32").
The pages quote ratios against 16-bit storage: 3.8-7.1x at 2-4 bits (aitherkvcache landing
page), 3.88x at 4 bits with a 2-byte norm (Turbo Attention PyPI page, "Install and try it"),
5x at 3 bits (turboquant-pytorch index page), 80% and 84% memory saved for K4/V2 and K3/V2
(TurboQuant forum article, zingnex.cn, bit settings).
"""

from __future__ import annotations


def code_bytes(d: int, bits: int) -> int:
    return (d * bits + 7) // 8


def vector_bytes(d: int, bits: int, norm_bytes: int = 4) -> int:
    return code_bytes(d, bits) + norm_bytes


def ratio_vs_16bit(d: int, bits: int, norm_bytes: int = 4) -> float:
    """Compression ratio against 2-byte elements: 2d / (code bytes + norm bytes)."""
    return (2 * d) / vector_bytes(d, bits, norm_bytes)


def average_bits(key_bits: int, value_bits: int) -> float:
    return (key_bits + value_bits) / 2.0


def saving_vs_16bit(key_bits: int, value_bits: int) -> float:
    """Fraction of 16-bit K+V memory saved by the codes alone (norms ignored)."""
    return 1.0 - average_bits(key_bits, value_bits) / 16.0


def encode_bytes(d: int, bits: int, in_elem_bytes: int) -> int:
    """Algorithmic HBM bytes of encoding one vector: read d inputs, write codes and norm."""
    return d * in_elem_bytes + vector_bytes(d, bits)


def decode_bytes(d: int, bits: int, out_elem_bytes: int) -> int:
    """Algorithmic HBM bytes of decoding one vector: read codes and norm, write d outputs."""
    return vector_bytes(d, bits) + d * out_elem_bytes
