"""Pins for the oracle's Lloyd-Max codebook (CPU).

Independent of the solver's closed-form cell integrals:
  * exact special cases: b = 1 (c = +-E|X|), d = 3 (uniform density -> uniform quantizer);
  * the textbook Gaussian quantizers (Max 1960), reached by the same solver on N(0,1);
  * the d -> infinity limit sqrt(d) c(d) -> Gaussian levels at rate 1/d;
  * the fixed-point conditions re-checked with 30-digit mpmath quadrature;
  * the distortion re-integrated numerically (scipy quad) over the density;
  * the information-theoretic bracket 4^-b <= d D <= (sqrt(3) pi / 2) 4^-b (the ~2.7x
    factor of the TurboQuant forum article).
"""

import json
import math
import os

import mpmath
import numpy as np
import pytest
from scipy import integrate

from oracle import codebook as cb

DIMS = (64, 128, 256)
BITS = (2, 3, 4)


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("b", (1, 2, 3, 4))
def test_symmetric_and_midpoint_thresholds(d, b):
    c = cb.codebook(d, b)
    L = 2 ** b
    assert c.centroids.shape == (L,) and c.thresholds.shape == (L - 1,)
    assert np.all(np.diff(c.centroids) > 0)
    assert np.array_equal(c.centroids[::-1], -c.centroids)
    assert c.thresholds[L // 2 - 1] == 0.0
    assert np.allclose(c.thresholds, 0.5 * (c.centroids[1:] + c.centroids[:-1]), rtol=0, atol=1e-17)


@pytest.mark.parametrize("d", (3, 5, 64, 128, 256))
def test_one_bit_closed_form(d):
    # c = E|X| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)); at d = 3 that is 1/2
    c = cb.lloyd_max(cb.SphereCoordinate(d), 1)
    expect = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    assert abs(c.centroids[1] - expect) <= 1e-13 * expect
    assert abs(c.mse - (1.0 / d - expect ** 2)) <= 1e-12 / d   # cancellation is relative to E[X^2]
    if d == 3:
        assert abs(expect - 0.5) <= 1e-15


@pytest.mark.parametrize("b", (1, 2, 3, 4))
def test_uniform_density_at_d3(b):
    # d = 3: f is uniform on [-1, 1], Lloyd-Max is the uniform quantizer, D = 1/(3 L^2)
    L = 2 ** b
    c = cb.lloyd_max(cb.SphereCoordinate(3), b)
    expect = np.array([-1 + (2 * k + 1) / L for k in range(L)])
    assert np.max(np.abs(c.centroids - expect)) <= 1e-13
    assert abs(c.mse - 1.0 / (3 * L * L)) <= 1e-13


def test_gaussian_matches_max_1960(golden_dir):
    table = json.load(open(os.path.join(golden_dir, "max1960_gaussian.json")))["levels"]
    for b_str, row in table.items():
        b = int(b_str)
        g = cb.lloyd_max(cb.Gaussian(), b)
        h = 2 ** (b - 1)
        # the table has 4 significant digits
        for mine, ref in zip(g.centroids[h:], row["outputs"]):
            assert abs(mine - ref) <= 6e-4 * max(1.0, abs(ref)), (b, mine, ref)
        for mine, ref in zip(g.thresholds[h:], row["thresholds"]):
            assert abs(mine - ref) <= 6e-4 * max(1.0, abs(ref)), (b, mine, ref)
        assert abs(g.mse - row["mse"]) <= 1e-3 * row["mse"], (b, g.mse, row["mse"])


@pytest.mark.parametrize("b", (2, 3))
def test_large_d_tends_to_gaussian_at_rate_one_over_d(b):
    g = cb.lloyd_max(cb.Gaussian(), b).centroids
    gaps = {}
    for d in (256, 4096):
        c = cb.lloyd_max(cb.SphereCoordinate(d), b).centroids * math.sqrt(d)
        gaps[d] = np.max(np.abs(c - g))
    # the scaled gap shrinks as 1/d: d * gap is the same constant at both sizes
    assert gaps[4096] < gaps[256] / 10
    assert abs(4096 * gaps[4096] / (256 * gaps[256]) - 1.0) < 0.05


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("b", BITS)
def test_mse_identity_at_fixed_point(d, b):
    # at a Lloyd-Max fixed point D = E[X^2] - sum_k p_k c_k^2 with E[X^2] = 1/d
    c = cb.codebook(d, b)
    p = cb.cell_masses(cb.SphereCoordinate(d), c.thresholds)
    assert abs(p.sum() - 1.0) <= 1e-14
    assert abs(c.mse - (1.0 / d - np.sum(p * c.centroids ** 2))) <= 1e-12 / d


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("b", BITS)
def test_mse_equals_numerical_integral(d, b):
    c = cb.codebook(d, b)
    f = cb.SphereCoordinate(d)
    edges = np.concatenate(([-1.0], c.thresholds, [1.0]))
    total = 0.0
    for k, ck in enumerate(c.centroids):
        val, err = integrate.quad(lambda x: (x - ck) ** 2 * float(f.pdf(x)), edges[k], edges[k + 1],
                                  epsabs=0, epsrel=1e-13, limit=200)
        total += val
    assert abs(total - c.mse) <= 1e-10 * c.mse


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("b", BITS)
def test_fixed_point_in_30_digits(d, b):
    c = cb.codebook(d, b)
    mpmath.mp.dps = 30
    m = mpmath.mpf(d - 3) / 2
    f = lambda x: (1 - x * x) ** m   # the constant C_d cancels in a conditional mean
    edges = [mpmath.mpf(-1)] + [mpmath.mpf(float(t)) for t in c.thresholds] + [mpmath.mpf(1)]
    h = 2 ** (b - 1)
    for k in range(h, 2 ** b):   # positive half; the negative half is the mirror image
        a, e = edges[k], edges[k + 1]
        num = mpmath.quad(lambda x: x * f(x), [a, e])
        den = mpmath.quad(f, [a, e])
        assert abs(float(num / den) - c.centroids[k]) <= 1e-13, (k, float(num / den), c.centroids[k])


@pytest.mark.parametrize("d", DIMS)
def test_distortion_within_the_bound_factor(d, golden_dir):
    factor = json.load(open(os.path.join(golden_dir, "page_figures.json")))["distortion_vs_lower_bound"]["factor"]
    hi_res_constant = math.sqrt(3) * math.pi / 2   # 2.7207: the "~2.7x"
    assert abs(hi_res_constant - factor) < 0.05
    prev = None
    for b in (1, 2, 3, 4):
        dd = d * cb.codebook(d, b).mse
        lower = 4.0 ** (-b)   # Shannon D(R) for unit total variance at b bits per coordinate
        assert lower < dd <= hi_res_constant * lower, (b, dd / lower)
        if prev is not None:
            assert dd / lower > prev   # the ratio climbs toward the high-resolution constant
        prev = dd / lower


def test_codebook_depends_only_on_d_and_b():
    a = cb.lloyd_max(cb.SphereCoordinate(128), 3)
    b = cb.lloyd_max(cb.SphereCoordinate(128), 3)
    assert np.array_equal(a.centroids, b.centroids)
    assert not np.allclose(cb.codebook(64, 3).centroids, cb.codebook(128, 3).centroids)
