"""The decode parity bar (tests/parity.py decode_bar) on CPU: what it accepts and what it refuses.

The bar compares a 16-bit decode with the float64 oracle decode cast to that dtype by
round-to-nearest-even, element by element, allowing a neighbour only where the float64 value
lies within DEC_W[dtype] * ||x|| of a rounding midpoint, and takes the 2e-3 normwise bound over the
elements that window determines. These checks run it on the oracle's own
decode of seeded codes, so they need no GPU.
"""

import numpy as np
import pytest
import torch

import tq_inputs as ti
from oracle import codebook as ocb, codec as occ, rotation as orot
from parity import DEC_W, decode_bar


def _ref(d=64, bits=3, n=3000, seed=3):
    cb = ocb.codebook(d, bits)
    pi = orot.haar_rotation(ti.rotation_gaussian(d, 42).numpy())
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 2 ** bits, size=(n, d))
    norms = np.exp(rng.normal(size=n)).astype(np.float32)
    return occ.decode_codes(codes, norms, pi, cb.centroids)


def _trunc_bf16(x):
    # drop the low 16 bits of the float32 pattern: rounding toward zero
    f = np.asarray(x, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return f.view(np.float32).astype(np.float64)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_the_cast_reference_passes(dtype):
    ref = _ref()
    ok, flips, worst = decode_bar(occ.cast(ref, dtype), ref, dtype)
    assert ok.all() and flips == 0 and worst <= 2e-3


def test_small_errors_pass():
    # an unrounded result within the window's error bound, then rounded: always accepted
    ref = _ref(d=128, bits=4)
    rng = np.random.default_rng(1)
    rn = np.linalg.norm(ref, axis=1, keepdims=True)
    for dt in (torch.bfloat16, torch.float16):
        noisy = ref + rng.uniform(-0.5, 0.5, size=ref.shape) * DEC_W[dt] * rn
        ok, flips, _ = decode_bar(occ.cast(noisy, dt), ref, dt)
        assert ok.all()


def test_truncating_bfloat16_fails():
    ref = _ref()
    ok, _, _ = decode_bar(_trunc_bf16(ref), ref, torch.bfloat16)
    assert not ok.any()         # every vector has elements truncated away from the nearest value


def _ref_codes(d, bits, n=3000, seed=3):
    cb = ocb.codebook(d, bits).centroids
    pi = orot.haar_rotation(ti.rotation_gaussian(d, 42).numpy())
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 2 ** bits, size=(n, d))
    norms = np.exp(rng.normal(size=n)).astype(np.float32)
    return codes, norms, pi, cb


@pytest.mark.parametrize("d,bits", [(64, 2), (64, 3), (128, 2), (128, 3), (256, 2), (256, 3)])
def test_centroids_within_the_table_bound_pass(d, bits):
    # bfloat16 decodes take one fp16 operand per centroid, within 2.5e-5 (relative) of it: the
    # exact decode with every centroid moved by that much, either way, then rounded, is accepted
    codes, norms, pi, cb = _ref_codes(d, bits)
    ref = occ.decode_codes(codes, norms, pi, cb)
    signs = np.where(np.random.default_rng(d + bits).random(len(cb)) < 0.5, -1.0, 1.0)
    moved = occ.decode_codes(codes, norms, pi, cb * (1.0 + 2.5e-5 * signs))
    ok, flips, _ = decode_bar(occ.cast(moved, torch.bfloat16), ref, torch.bfloat16)
    assert ok.all() and flips > 0


@pytest.mark.parametrize("d,bits", [(64, 3), (128, 2), (128, 3), (128, 4), (256, 3)])
def test_unscaled_fp16_centroids_fail(d, bits):
    # centroids simply rounded to fp16 (2^-12 relative, with no scale chosen for the table)
    # change the rounding of elements outside the window
    codes, norms, pi, cb = _ref_codes(d, bits)
    ref = occ.decode_codes(codes, norms, pi, cb)
    plain = occ.decode_codes(codes, norms, pi, cb.astype(np.float16).astype(np.float64))
    ok, _, _ = decode_bar(occ.cast(plain, torch.bfloat16), ref, torch.bfloat16)
    assert not ok.all()


def test_single_fp16_operand_error_fails_for_fp16_and_float32():
    # an unrounded error of 3e-4 of the norm (single fp16 operands, no scaled table) changes
    # many fp16 roundings and exceeds the float32 window
    ref = _ref(d=128, bits=4)
    rng = np.random.default_rng(2)
    rn = np.linalg.norm(ref, axis=1, keepdims=True)
    noisy = ref + rng.normal(size=ref.shape) * 3e-4 * rn / np.sqrt(ref.shape[1])
    ok16, _, _ = decode_bar(occ.cast(noisy, torch.float16), ref, torch.float16)
    assert not ok16.any()
    ok32, _, _ = decode_bar(noisy, ref, torch.float32)
    assert not ok32.any()


def test_wrong_vector_fails_normwise():
    ref = _ref()
    bad = ref.copy()
    bad[7] *= 1.01
    ok, _, _ = decode_bar(occ.cast(bad, torch.bfloat16), ref, torch.bfloat16)
    assert not ok[7] and ok[:7].all()
