"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module draws random numbers and builds workload shapes. It holds none of the
codec's arithmetic: no norms, rotations, codebooks, quantization or packing. The
Gaussian matrix that a Haar rotation is made from is a random draw of the method, so
it is produced here and handed to both the oracle and the library as an input.

Sources for the recipes:
  * Rotation draw: a d x d float32 standard-normal matrix from a CPU torch generator
    seeded with the layer's seed (KV Cache API page, ginkgoq.github.io/TurboQuant/api/kv,
    TurboQuantCompressorV2.__init__ / TurboQuantCompressorMSE.__init__).
  * Per-layer seeds: keys 42 + 7*layer, values that plus 500 (same page,
    CompressedKVStore.__init__).
  * QJL sketch draw: d x d float32 standard normal from a CPU generator seeded seed + 10000
    (same page, TurboQuantCompressorV2.__init__).
  * The 8-key example: torch.randn(8, 128) under manual_seed(0) (Turbo Attention
    (turbo-attn) PyPI page, "Install and try it").
"""

from .inputs import *  # noqa: F401,F403
