"""Float64 CPU oracle of the TurboQuant KV-cache codec hot path.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check in __graft_entry__ and the
bench's CPU-baseline leg may import or run anything in this package. The product path
(the HIP library and its Python binding) never calls it, and this package imports
nothing from the product: the two share no code. Inputs come from `tq_inputs`, which
holds only seeded random draws.

Sources (pages are cited by title and section; see each function's docstring):
  * KV Cache API page (ginkgoq.github.io/TurboQuant/api/kv): the compressor classes
    TurboQuantCompressorV2 / TurboQuantCompressorMSE / MSECompressor (__init__,
    compress, decompress), TurboQuantKVCache.attention_scores / attend, the value
    packing helpers (2- and 4-bit packing order) and value_formula_nbytes (dense
    bitstream size).
  * TurboQuant forum article (zingnex.cn, "TurboQuant: A KV Cache Compression
    Technique ..."): the three steps, data-independent codebooks, bit presets, the
    ~2.7x distance from the information-theoretic bound.
  * aitherkvcache landing page: encode(x) -> (packed uint8, float32 norms), 3.8-7.1x.
  * Turbo Attention (turbo-attn) PyPI page: the 8-key example (3.88x, error 0.10);
    its codec table, whose rotation row applies the key rotation to the queries too.

Modules: rotation (Haar rotation by QR), codebook (Lloyd-Max for the sphere-coordinate
density), codec (norm, rotate, quantize, pack, unpack, decode), attention (scores and
decode attention, dense and paged), accounting (bytes per vector, ratios).

Parity status: every function here is pinned by tests/test_oracle_*.py against values
the pages print, closed forms, special cases, independent high-precision quadrature or
brute force. No function is "parity unpinned".
"""

from . import accounting, attention, codebook, codec, rotation  # noqa: F401
