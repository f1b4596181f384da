"""Parity helpers for the GPU tests: compare libtq's outputs with the float64 oracle.

Bars:
  * codes: bit-exact, except coordinates whose oracle rotated value lies within 1e-5 of a
    decision boundary (counted and reported as flips);
  * norms: |n_gpu - n| <= (d/4 + 4) * 2^-24 * n, the rounding bound of the kernel's float32
    sum of squares (two chains of d/4 fused multiply-adds per lane, two adds, a square root);
  * decode: x_ref = float64 oracle decode of the same codes and norms, cast to the output
    dtype by round-to-nearest-even as the pages' decompress does. Element by element x_gpu
    must be what the cast gives for some value within DEC_W[dtype] * ||x_ref|| of x_ref:
    bit-exact where that interval holds one representable value, either neighbour where the
    float64 value sits that close to a rounding midpoint (a rounding flip, counted like a code
    flip: a decision both sides take in different precision). Per vector, over the elements
    the interval determines, ||x_gpu - x_ref_cast|| <= 2e-3 ||x_ref||. DEC_W bounds the
    kernel's unrounded error; float32 outputs take the same interval plus one float32 rounding
    and ||x_gpu - x_ref|| <= 2e-3 ||x_ref||;
  * scores: |s_gpu - s_ref| <= 2e-3 * scale * n_t * ||q|| * ||c[idx_t]|| (Cauchy-Schwarz scale);
  * attention: ||o_gpu - o_ref|| <= 2e-3 * sum_t p_t ||v_hat_t||; |lse_gpu - lse_ref| <= the
    largest score bound of the row.

Provenance: the oracle never takes a GPU output as input. A decode, score or attention test
feeds the GPU a compressed cache made by the oracle's own encode of seeded inputs
(oracle_encoded) or by tq_inputs' random bytes and norms, and gives the oracle the same bytes.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

from oracle import attention as oatt, codebook as ocb, codec as occ, rotation as orot

WINDOW = 1e-5
REL = 2e-3
# decode: bound on the kernel's unrounded error per element, relative to the vector norm, by
# output dtype. fp16 and float32 outputs: the fp16 hi/lo splits of both operands give ~1.2e-7 in
# a float emulation of the kernel's arithmetic. bfloat16 outputs: one fp16 operand per centroid
# (a scaled table within 2.5e-5 relative of the centroids) bounds the error by 2.5e-5 of the norm
# (Cauchy-Schwarz over a unit row of the rotation), a fifth of a bfloat16 half-ulp at a
# coordinate of typical size ||x|| / sqrt(d), so the window stays far inside the output's
# own rounding.
DEC_W = {torch.bfloat16: 3e-5, torch.float16: 1e-6, torch.float32: 1e-6}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype != torch.float64 else t.cpu().numpy()


def check_encode(x: np.ndarray, packed: np.ndarray, norms: np.ndarray, pi: np.ndarray, d: int, bits: int,
                 what: str = ""):
    """x float64 [N, d] (the exact input values), packed/norms from the GPU. Returns flip count."""
    cb = ocb.codebook(d, bits)
    codes_ref, n_ref, y = occ.encode_codes(x, pi, cb.centroids)
    codes = unpack(packed, bits, d)
    delta = occ.boundary_distance(y, cb.thresholds)
    diff = codes != codes_ref
    bad = diff & (delta >= WINDOW)
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError("%s: %d codes differ outside the %.0e window (first at vector %d coord %d: "
                             "gpu %d ref %d, y=%.9g, delta=%.3g)" % (what, int(bad.sum()), WINDOW, i, j,
                                                                     codes[i, j], codes_ref[i, j], y[i, j],
                                                                     delta[i, j]))
    nr = np.sqrt(np.sum(x * x, axis=1))
    ng = norms.astype(np.float64)
    tol = (d / 4 + 4) * 2.0 ** -24 * nr
    assert np.all(np.abs(ng - nr) <= tol), "%s: norm error %.3g > bound" % (what, np.max(np.abs(ng - nr) / np.maximum(nr, 1e-300)))
    flips = int(diff.sum())
    inside = int((delta < WINDOW).sum())
    log("%s: %d vectors, %d flips among %d coordinates inside the window" % (what, x.shape[0], flips, inside))
    return flips


def unpack(packed: np.ndarray, bits: int, d: int) -> np.ndarray:
    """Codes of GPU-written rows for comparison (LSB-first bitstream, code j in stream bits
    [j*bits, (j+1)*bits)); the tests' own vectorized reader, so no GPU output enters the oracle."""
    p = np.asarray(packed, dtype=np.uint8).reshape(-1, np.asarray(packed).shape[-1])
    stream = np.unpackbits(p, axis=1, bitorder="little")[:, : d * bits].reshape(-1, d, bits).astype(np.int64)
    return (stream << np.arange(bits)).sum(axis=2).astype(np.uint8)


def oracle_encoded(x64: np.ndarray, pi: np.ndarray, bits: int):
    """The oracle's encode of x [..., d] (float64 values of a seeded input): packed uint8
    [..., (d*bits)/8] and norms float32 [...], to be uploaded as a GPU test input."""
    d = x64.shape[-1]
    lead = x64.shape[:-1]
    cb = ocb.codebook(d, bits)
    packed, norms = occ.encode(x64.reshape(-1, d), pi, cb.centroids, bits)
    return packed.reshape(*lead, -1), norms.reshape(lead)


def upload(a: np.ndarray, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def decode_bar(got: np.ndarray, ref: np.ndarray, dtype: torch.dtype):
    """The decode bar for outputs `got` (float64 values of a `dtype` tensor) against the float64
    decode `ref`, both [N, d]. Returns (ok per vector, rounding flips, worst normwise error
    against the cast reference / ||ref||, rounding flips included)."""
    rn = np.linalg.norm(ref, axis=1)
    w = DEC_W[dtype] * rn[:, None]
    if dtype == torch.float32:
        inside = np.abs(got - ref) <= w + 2.0 ** -24 * np.abs(ref)
        cast, determined, flips = ref, np.ones(ref.shape, bool), 0
    else:
        lo = occ.cast(ref - w, dtype)
        hi = occ.cast(ref + w, dtype)
        inside = (got >= lo) & (got <= hi)
        cast = occ.cast(ref, dtype)
        determined = lo == hi
        flips = int(np.sum(got != cast))
    diff = got - cast
    num = np.linalg.norm(np.where(determined, diff, 0.0), axis=1)
    ok = inside.all(axis=1) & ((num <= REL * rn) | ((rn == 0) & (num == 0)))
    worst = float(np.max(np.linalg.norm(diff, axis=1) / np.maximum(rn, 1e-300))) if len(rn) else 0.0
    return ok, flips, worst


def check_decode(out: torch.Tensor, packed: np.ndarray, norms: np.ndarray, pi: np.ndarray, d: int, bits: int,
                 what: str = ""):
    cb = ocb.codebook(d, bits)
    ref = occ.decode(packed, norms, pi, cb.centroids, bits, d)
    got = to64(out)
    ok, flips, worst = decode_bar(got, ref, out.dtype)
    if not ok.all():
        i = int(np.argmin(ok))
        j = int(np.argmax(np.abs(got[i] - ref[i])))
        raise AssertionError("%s: %d of %d vectors miss the decode bar (vector %d coord %d: gpu %.9g ref %.12g, "
                             "|ref| %.6g)" % (what, int((~ok).sum()), len(ok), i, j, got[i, j], ref[i, j],
                                              float(np.linalg.norm(ref[i]))))
    # against the unrounded float64 decode, the output's error next to the cast's own
    rn = np.maximum(np.linalg.norm(ref, axis=1), 1e-300)
    e_gpu = float(np.max(np.linalg.norm(got - ref, axis=1) / rn)) if len(rn) else 0.0
    e_cast = float(np.max(np.linalg.norm(occ.cast(ref, out.dtype) - ref, axis=1) / rn)) if len(rn) else 0.0
    log("%s: decode %s, worst normwise error vs the cast reference %.3g, %d rounding flips; "
        "vs the float64 decode %.3g (the cast itself: %.3g)" % (what, str(out.dtype)[6:], worst, flips, e_gpu, e_cast))


def rotation_pair(d: int, seeds):
    """(device Rotation stack, list of oracle float64 rotations) from the same Gaussian draws."""
    import kv_cache_vector_encode_amd as tq
    import tq_inputs as ti
    g = ti.rotation_gaussians(d, seeds)
    rot = tq.Rotation.from_gaussian(g)
    return rot, [orot.haar_rotation(gi.numpy()) for gi in g]


def score_bounds(q64: np.ndarray, k_norms: np.ndarray, k_codes: np.ndarray, cb, scale: float):
    """2e-3 * scale * n_t * ||q|| * ||c[idx_t]||, shapes [B, Hq, T] (q [B,Hq,d], k [B,Hkv,T,...])."""
    B, Hq, d = q64.shape
    Hkv = k_norms.shape[1]
    G = Hq // Hkv
    cnorm = np.linalg.norm(cb.centroids[k_codes.astype(np.int64)], axis=-1)   # [B,Hkv,T]
    qn = np.linalg.norm(q64, axis=-1)                                         # [B,Hq]
    kv = np.repeat(k_norms.astype(np.float64) * cnorm, G, axis=1)             # [B,Hq,T]
    return REL * scale * kv * qn[:, :, None]


def check_attention(o_gpu: np.ndarray, lse_gpu, q64, khat, vhat, scale, lens, what=""):
    """khat/vhat float64 [B, Hkv, T, d] decoded from the GPU's codes."""
    o_ref, lse_ref = oatt.attention(q64, khat, vhat, scale, seq_lens=lens)
    s_ref = oatt.scores(q64, khat, scale, seq_lens=lens)
    B, Hq, d = q64.shape
    G = Hq // khat.shape[1]
    worst = 0.0
    for b in range(B):
        L = int(lens[b]) if lens is not None else khat.shape[2]
        for h in range(Hq):
            if L == 0:
                assert np.all(o_gpu[b, h] == 0), (what, b, h)
                if lse_gpu is not None:
                    assert np.isneginf(lse_gpu[b, h])
                continue
            p = np.exp(s_ref[b, h, :L] - lse_ref[b, h])
            bound = REL * float(p @ np.linalg.norm(vhat[b, h // G, :L], axis=1))
            err = float(np.linalg.norm(o_gpu[b, h] - o_ref[b, h]))
            if bound > 0:                      # all-zero values: the bar is exact zero
                worst = max(worst, err / bound)
            assert err <= bound, "%s: b=%d h=%d attention error %.3g > bound %.3g" % (what, b, h, err, bound)
            if lse_gpu is not None:
                kn = np.linalg.norm(khat[b, h // G, :L], axis=1)
                lb = REL * scale * float(np.max(kn)) * float(np.linalg.norm(q64[b, h]))
                assert abs(lse_gpu[b, h] - lse_ref[b, h]) <= lb + 1e-6, (what, b, h, lse_gpu[b, h], lse_ref[b, h])
    log("%s: attention worst error / bound = %.3g" % (what, worst))
    return worst
