"""Pins for the oracle's Haar rotation (CPU).

The rotation is defined as the Q factor of a seeded Gaussian draw with the signs fixed so
R has a positive diagonal (KV Cache API page, TurboQuantCompressorV2.__init__). QR with a
positive-diagonal R is unique, so the oracle's own Householder QR must agree with LAPACK's
and must satisfy the definition G = Pi R' with R' upper triangular and positive on the
diagonal. The sign fix is what makes Q Haar-distributed; a test on the law of one entry
catches a missing or inverted fix.
"""

import math

import numpy as np
import pytest
from scipy import special, stats

import tq_inputs as ti
from oracle import rotation


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("seed", [42, 49, 542])
def test_orthogonal_to_1e12(d, seed):
    pi = rotation.haar_rotation(ti.rotation_gaussian(d, seed).numpy())
    assert np.max(np.abs(pi.T @ pi - np.eye(d))) <= 1e-12
    assert np.max(np.abs(pi @ pi.T - np.eye(d))) <= 1e-12


@pytest.mark.parametrize("d", [64, 128])
def test_is_the_qr_factor_with_positive_diagonal(d):
    g = ti.rotation_gaussian(d, 7).numpy().astype(np.float64)
    pi = rotation.haar_rotation(g)
    r = pi.T @ g
    scale = np.max(np.abs(r))
    assert np.max(np.abs(np.tril(r, -1))) <= 1e-12 * scale
    assert np.all(np.diag(r) > 0)
    assert np.max(np.abs(pi @ np.triu(r) - g)) <= 1e-12 * scale


@pytest.mark.parametrize("d", [64, 128, 256])
def test_matches_lapack_after_sign_fix(d):
    g = ti.rotation_gaussian(d, 42).numpy().astype(np.float64)
    q, r = np.linalg.qr(g)
    s = np.sign(np.diag(r))
    s[s == 0] = 1
    assert np.max(np.abs(rotation.haar_rotation(g) - q * s[None, :])) <= 1e-12


def test_zero_sign_counts_as_plus():
    # a draw whose first column is e_2 gives R[0,0] = 1 > 0; a zero column gives R[0,0] = 0,
    # whose sign must be taken as +1 (the column of Q stays as Householder made it)
    g = np.eye(4)
    g[:, 0] = 0.0
    pi = rotation.haar_rotation(g)
    q, r = rotation.householder_qr(g)
    assert r[0, 0] == 0.0
    assert np.array_equal(pi[:, 0], q[:, 0])


def test_entries_follow_the_haar_law():
    # For a Haar rotation every entry is distributed as one coordinate of a uniform unit
    # vector: (x + 1)/2 ~ Beta((d-1)/2, (d-1)/2). Without the sign fix Householder's Q[0,0]
    # is always negative, which this rejects at once.
    d = 8
    vals = np.array([rotation.haar_rotation(ti.rotation_gaussian(d, 10_000 + s).numpy())[0, 0]
                     for s in range(1500)])
    a = (d - 1) / 2
    p = stats.kstest((vals + 1) / 2, lambda u: special.betainc(a, a, u)).pvalue
    assert p > 1e-3


def test_deterministic_in_the_seed():
    a = rotation.haar_rotation(ti.rotation_gaussian(128, 42).numpy())
    b = rotation.haar_rotation(ti.rotation_gaussian(128, 42).numpy())
    c = rotation.haar_rotation(ti.rotation_gaussian(128, 49).numpy())
    assert np.array_equal(a, b)
    assert not np.allclose(a, c)


def test_layer_seed_convention(golden_dir):
    import json, os
    fig = json.load(open(os.path.join(golden_dir, "page_figures.json")))["layer_seeds"]
    for layer in (0, 1, 31, 79):
        assert ti.key_seed(layer) == eval(fig["key"], {"layer": layer})
        assert ti.value_seed(layer) == eval(fig["value"], {"layer": layer})
    assert math.isclose(ti.key_seed(0), 42)
