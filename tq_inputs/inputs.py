"""Seeded input recipes for the five workloads (random draws and shapes only).

Every function returns plain torch tensors. Large workloads are drawn on the device
that the caller names (a CUDA generator on the GPU); the parity tests copy sampled
rows to the host for the oracle. Nothing here computes any part of the codec.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "key_seed", "value_seed", "rotation_gaussian", "rotation_gaussians", "qjl_sketch_gaussian",
    "example_keys", "codec_check_inputs", "LlamaCacheShape", "llama_layer_kv",
    "LongCacheShape", "long_cache_layer_kv", "AttnShape", "attn_inputs",
    "PagedShape", "paged_layout", "paged_layer_bits", "paged_layer_tokens", "paged_queries",
    "generator", "random_bytes", "random_norms", "normal", "random_signs",
]


def generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


# --- rotation draws -----------------------------------------------------------------

def key_seed(layer: int) -> int:
    """Seed of a layer's key rotation: 42 + 7*layer."""
    return 42 + 7 * int(layer)


def value_seed(layer: int) -> int:
    """Seed of a layer's value rotation: the key seed plus 500."""
    return key_seed(layer) + 500


def rotation_gaussian(d: int, seed: int) -> torch.Tensor:
    """The float32 d x d standard-normal draw a Haar rotation is built from (CPU generator)."""
    return torch.randn(d, d, generator=generator("cpu", seed), dtype=torch.float32)


def rotation_gaussians(d: int, seeds) -> torch.Tensor:
    """Stack of draws, one per seed: [len(seeds), d, d] float32."""
    return torch.stack([rotation_gaussian(d, s) for s in seeds])


def random_signs(n_rot: int, d: int, seed: int) -> np.ndarray:
    """The random +-1 diagonal of a Hadamard rotation (Turbo Attention PyPI page, "The codec"):
    int8 [n_rot, d], each sign a fair coin from a CPU generator."""
    g = generator("cpu", seed)
    return (torch.randint(0, 2, (n_rot, d), generator=g) * 2 - 1).to(torch.int8).numpy()


def qjl_sketch_gaussian(d: int, seed: int) -> torch.Tensor:
    """The float32 d x d standard-normal sketch matrix of the QJL stage for a key compressor
    seeded `seed`: a CPU generator seeded seed + 10000 (the key compressor's second draw)."""
    return torch.randn(d, d, generator=generator("cpu", seed + 10000), dtype=torch.float32)


# --- small codec workloads ----------------------------------------------------------

def normal(shape, seed: int, scale: float = 1.0, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """scale * N(0, 1) of the given shape from a CPU generator, rounded to dtype, on device."""
    z = torch.randn(tuple(shape), generator=generator("cpu", seed), dtype=torch.float32)
    return (z * scale).to(dtype).to(device)


def example_keys() -> torch.Tensor:
    """8 key vectors of dimension 128, N(0,1), drawn as torch.randn(8, 128) after manual_seed(0)."""
    return torch.randn(8, 128, generator=generator("cpu", 0), dtype=torch.float32)


def codec_check_inputs(n: int = 4096, d: int = 128, seed: int = 0) -> torch.Tensor:
    """The codec-correctness workload: n x d float32 N(0,1) from a CPU generator (default seed 0)."""
    return torch.randn(n, d, generator=generator("cpu", seed), dtype=torch.float32)


# --- Llama-3-8B-shaped cache (K4/V2, one shared rotation per layer) ------------------

@dataclass(frozen=True)
class LlamaCacheShape:
    layers: int = 32
    kv_heads: int = 8
    tokens: int = 8192
    head_dim: int = 128
    key_bits: int = 4
    value_bits: int = 2
    outlier_channels: int = 4
    outlier_scale: float = 10.0

    @property
    def vectors_per_layer(self) -> int:
        return self.kv_heads * self.tokens


def llama_outlier_channels(shape: LlamaCacheShape, layer: int) -> torch.Tensor:
    """Indices of the key channels scaled up in this layer (shared by heads and tokens)."""
    perm = torch.randperm(shape.head_dim, generator=generator("cpu", 3000 + layer))
    return perm[: shape.outlier_channels].sort().values


def llama_layer_kv(shape: LlamaCacheShape, layer: int, device="cpu", dtype=torch.bfloat16,
                   tokens: int | None = None, out_k=None, out_v=None):
    """Keys and values of one layer as [kv_heads, tokens, head_dim].

    Keys: N(0,1) with `outlier_channels` channels multiplied by `outlier_scale`.
    Values: N(0,1). Seeds: keys 1000+layer, values 2000+layer.
    """
    T = shape.tokens if tokens is None else tokens
    sz = (shape.kv_heads, T, shape.head_dim)
    k = torch.randn(sz, generator=generator(device, 1000 + layer), device=device, dtype=torch.float32)
    ch = llama_outlier_channels(shape, layer).to(device)
    k[..., ch] *= shape.outlier_scale
    v = torch.randn(sz, generator=generator(device, 2000 + layer), device=device, dtype=torch.float32)
    if out_k is not None:
        out_k.copy_(k)
        out_v.copy_(v)
        return out_k, out_v
    return k.to(dtype), v.to(dtype)


# --- 70B-class cache at 128K context (3-bit K and V, streamed per layer) ------------

@dataclass(frozen=True)
class LongCacheShape:
    layers: int = 80
    kv_heads: int = 8
    tokens: int = 131072
    head_dim: int = 128
    key_bits: int = 3
    value_bits: int = 3

    @property
    def vectors_per_layer(self) -> int:
        return self.kv_heads * self.tokens


def long_cache_channel_std(shape: LongCacheShape, layer: int) -> torch.Tensor:
    """Per-channel standard deviations exp(0.5 z), z ~ N(0,1), as [2 (K,V), kv_heads, head_dim]."""
    z = torch.randn(2, shape.kv_heads, shape.head_dim, generator=generator("cpu", 4000 + layer))
    return torch.exp(0.5 * z)


def long_cache_layer_kv(shape: LongCacheShape, layer: int, device="cpu", dtype=torch.bfloat16,
                        tokens: int | None = None, out_k=None, out_v=None):
    """Keys and values of one layer as [kv_heads, tokens, head_dim]: sigma (per channel) * N(0,1).

    Seeds: keys 5000+layer, values 6000+layer; sigma from 4000+layer.
    """
    T = shape.tokens if tokens is None else tokens
    sz = (shape.kv_heads, T, shape.head_dim)
    std = long_cache_channel_std(shape, layer).to(device)
    k = torch.randn(sz, generator=generator(device, 5000 + layer), device=device, dtype=torch.float32)
    k *= std[0][:, None, :]
    v = torch.randn(sz, generator=generator(device, 6000 + layer), device=device, dtype=torch.float32)
    v *= std[1][:, None, :]
    if out_k is not None:
        out_k.copy_(k)
        out_v.copy_(v)
        return out_k, out_v
    return k.to(dtype), v.to(dtype)


# --- fused decode attention workload --------------------------------------------------

@dataclass(frozen=True)
class AttnShape:
    batch: int = 32
    q_heads: int = 32
    kv_heads: int = 8
    tokens: int = 32768
    head_dim: int = 128
    key_bits: int = 4
    value_bits: int = 2


def attn_inputs(shape: AttnShape, device="cpu", dtype=torch.bfloat16, seed: int = 11):
    """q [B, Hq, d], K and V [B, Hkv, T, d]; all N(0,1) (seeds seed, seed+1, seed+2)."""
    B, Hq, Hkv, T, d = shape.batch, shape.q_heads, shape.kv_heads, shape.tokens, shape.head_dim
    q = torch.randn(B, Hq, d, generator=generator(device, seed), device=device).to(dtype)
    k = torch.randn(B, Hkv, T, d, generator=generator(device, seed + 1), device=device).to(dtype)
    v = torch.randn(B, Hkv, T, d, generator=generator(device, seed + 2), device=device).to(dtype)
    return q, k, v


# --- paged ragged cache -----------------------------------------------------------------

@dataclass(frozen=True)
class PagedShape:
    sequences: int = 256
    max_len: int = 16384
    block_size: int = 16
    kv_heads: int = 8
    q_heads: int = 32
    head_dims: tuple = (64, 128, 256)
    layers_per_dim: int = 9
    spike_fraction: float = 0.01
    spike_scale: float = 50.0


@dataclass
class PagedLayout:
    seq_lens: torch.Tensor          # [S] int32
    block_table: torch.Tensor       # [S, max_blocks] int32 (unused entries 0)
    num_blocks: int
    token_slots: torch.Tensor       # [total_tokens] int64: physical (block*bs + offset) of each token,
                                    # tokens ordered sequence by sequence
    seq_starts: torch.Tensor        # [S+1] int64 prefix sums of seq_lens
    extra: dict = field(default_factory=dict)


def paged_layout(shape: PagedShape, sequences: int | None = None, max_len: int | None = None,
                 seed: int = 7) -> PagedLayout:
    """Sequence lengths ~ U[1, max_len] (seed 7) and a seeded random permutation of physical blocks."""
    S = shape.sequences if sequences is None else sequences
    ML = shape.max_len if max_len is None else max_len
    bs = shape.block_size
    lens = torch.randint(1, ML + 1, (S,), generator=generator("cpu", seed), dtype=torch.int64)
    nblk = (lens + bs - 1) // bs
    total_blocks = int(nblk.sum())
    perm = torch.randperm(total_blocks, generator=generator("cpu", seed + 1))
    max_blocks = int(nblk.max())
    table = torch.zeros(S, max_blocks, dtype=torch.int32)
    starts = torch.zeros(S + 1, dtype=torch.int64)
    starts[1:] = torch.cumsum(lens, 0)
    slots = torch.empty(int(starts[-1]), dtype=torch.int64)
    off = 0
    for s in range(S):
        blocks = perm[off: off + int(nblk[s])]
        off += int(nblk[s])
        table[s, : blocks.numel()] = blocks.to(torch.int32)
        t = torch.arange(int(lens[s]))
        slots[starts[s]: starts[s + 1]] = blocks[t // bs].to(torch.int64) * bs + t % bs
    return PagedLayout(seq_lens=lens.to(torch.int32), block_table=table, num_blocks=total_blocks,
                       token_slots=slots, seq_starts=starts)


def paged_layer_bits(layer: int):
    """(key_bits, value_bits) of layer `layer`: the nine pairs of {2,3,4}^2 in order."""
    widths = (2, 3, 4)
    j = layer % 9
    return widths[j // 3], widths[j % 3]


def paged_layer_tokens(shape: PagedShape, total_tokens: int, head_dim: int, layer: int,
                       device="cpu", dtype=torch.bfloat16):
    """K and V of one layer, token-major [total_tokens, kv_heads, head_dim], N(0,1), with a
    Bernoulli(spike_fraction) set of tokens (all heads, K and V) multiplied by spike_scale."""
    base = 100000 + 1000 * head_dim + 10 * layer
    sz = (total_tokens, shape.kv_heads, head_dim)
    k = torch.randn(sz, generator=generator(device, base), device=device)
    v = torch.randn(sz, generator=generator(device, base + 1), device=device)
    spikes = torch.rand(total_tokens, generator=generator(device, base + 2), device=device) < shape.spike_fraction
    factor = torch.where(spikes, torch.tensor(shape.spike_scale, device=device),
                         torch.tensor(1.0, device=device))
    k *= factor[:, None, None]
    v *= factor[:, None, None]
    return k.to(dtype), v.to(dtype), spikes


def paged_queries(shape: PagedShape, sequences: int, head_dim: int, layer: int,
                  device="cpu", dtype=torch.bfloat16):
    """One decode query per sequence: [sequences, q_heads, head_dim] N(0,1)."""
    base = 200000 + 1000 * head_dim + 10 * layer
    return torch.randn(sequences, shape.q_heads, head_dim, generator=generator(device, base),
                       device=device).to(dtype)


# --- compressed-cache stand-ins ----------------------------------------------------------
# A packed code row is any byte string (every bit pattern decodes to valid codes), so uniform
# random bytes stand in for a compressed cache; norms are log-normal around a typical key norm.

def random_bytes(shape, seed: int, device="cpu") -> torch.Tensor:
    """Uniform random uint8 tensor of the given shape."""
    g = generator("cpu", seed)
    return torch.randint(0, 256, tuple(shape), generator=g, dtype=torch.uint8).to(device)


def random_norms(shape, seed: int, median: float = 16.0, sigma: float = 0.4, device="cpu") -> torch.Tensor:
    """Positive float32 tensor: median * exp(sigma * N(0, 1))."""
    g = generator("cpu", seed)
    z = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    return (median * torch.exp(sigma * z)).to(device)
