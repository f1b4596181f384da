"""Pins for the oracle's Hadamard rotation and the norm-corrected encode (CPU).

Hadamard rotation (Turbo Attention PyPI page, "The codec", Hadamard rotation row): the
oracle builds Pi = H_d diag(s) / sqrt(d) from Sylvester's doubling. It is pinned against the
closed form H[i, j] = (-1)^popcount(i & j), scipy's construction, the 2x2 case written out,
orthogonality, and a fast Walsh-Hadamard butterfly written here (a different algorithm).

Norm correction (same table, Norms row: key-side norm correction keeps the decoded key's
length): pinned by that property itself — the decode of the corrected norm has the input's
length — plus the codes being the plain encode's and a per-vector loop.
"""

import numpy as np
import pytest
import scipy.linalg

import tq_inputs as ti
from oracle import codebook, codec, rotation


def fwht(x):
    """Unnormalized fast Walsh-Hadamard transform of the last axis (butterflies)."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :], y[..., 1, :] = a + b, a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


def test_two_by_two_written_out():
    s2 = 1.0 / np.sqrt(2.0)
    assert np.array_equal(rotation.hadamard_rotation(2), np.array([[s2, s2], [s2, -s2]]))


@pytest.mark.parametrize("d", [1, 2, 4, 8, 64, 128, 256])
def test_entries_are_the_popcount_closed_form(d):
    i = np.arange(d)[:, None]
    j = np.arange(d)[None, :]
    pop = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    assert np.array_equal(rotation.hadamard_matrix(d), (-1.0) ** pop)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_matches_scipy_and_is_orthogonal(d):
    assert np.array_equal(rotation.hadamard_matrix(d), scipy.linalg.hadamard(d).astype(np.float64))
    s = np.where(np.random.default_rng(d).random(d) < 0.5, -1.0, 1.0)
    pi = rotation.hadamard_rotation(d, s)
    assert np.max(np.abs(pi @ pi.T - np.eye(d))) <= 1e-14
    assert np.max(np.abs(pi.T @ pi - np.eye(d))) <= 1e-14


@pytest.mark.parametrize("d", [64, 128, 256])
def test_pi_x_is_the_butterfly_of_the_sign_flipped_input(d):
    rng = np.random.default_rng(5)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    x = rng.standard_normal((7, d))
    pi = rotation.hadamard_rotation(d, s)
    assert np.max(np.abs(x @ pi.T - fwht(x * s) / np.sqrt(d))) <= 1e-12
    # the transposed orientation is a different map once signs are random: a swapped
    # operand would be caught
    assert np.max(np.abs(x @ pi - fwht(x * s) / np.sqrt(d))) > 1e-3


def test_rejects_bad_sizes_and_signs():
    with pytest.raises(ValueError):
        rotation.hadamard_matrix(96)
    with pytest.raises(ValueError):
        rotation.hadamard_rotation(4, [1, -1, 0.5, 1])


@pytest.mark.parametrize("b", [2, 3, 4])
def test_norm_correction_keeps_the_decoded_length(b):
    d = 128
    x = ti.codec_check_inputs(n=512, d=d, seed=3).numpy().astype(np.float64)
    pi = rotation.haar_rotation(ti.rotation_gaussian(d, 42).numpy())
    c = codebook.codebook(d, b).centroids
    codes, nc, _ = codec.encode_codes_norm_corrected(x, pi, c)
    codes0, n0, _ = codec.encode_codes(x, pi, c)
    assert np.array_equal(codes, codes0)
    xh = codec.decode_codes(codes, nc, pi, c)
    n = np.linalg.norm(x, axis=1)
    # float32 storage of the corrected norm is the only rounding: <= 2^-24 relative
    assert np.max(np.abs(np.linalg.norm(xh, axis=1) / n - 1.0)) <= 2.0 ** -23
    # the uncorrected decode is shorter on average (||c[idx]|| < 1 in expectation)
    assert np.mean(np.linalg.norm(codec.decode_codes(codes0, n0, pi, c), axis=1) / n) < 1.0


def test_norm_correction_per_vector_loop_and_zero_vector():
    d = 64
    rng = np.random.default_rng(9)
    x = rng.standard_normal((20, d))
    x[3] = 0.0
    pi = rotation.hadamard_rotation(d, np.where(rng.random(d) < 0.5, -1.0, 1.0))
    c = codebook.codebook(d, 3).centroids
    codes, nc, _ = codec.encode_codes_norm_corrected(x, pi, c)
    for i in range(x.shape[0]):
        n = np.sqrt(sum(v * v for v in x[i]))
        cn = np.sqrt(sum(c[int(k)] ** 2 for k in codes[i]))
        assert nc[i] == np.float32(n / cn)
    assert nc[3] == 0.0
