"""Lloyd-Max scalar codebook for one coordinate of a rotated unit vector (oracle, float64).

What the pages fix: the codebook is the optimal (Lloyd-Max) scalar quantizer with 2^b
levels, precomputed from mathematics alone, with no data or calibration (TurboQuant
forum article, zingnex.cn, "two core steps" list item 2; aitherkvcache landing page,
"no calibration pass"); each rotated coordinate is rounded to its nearest centroid
(KV Cache API page, ginkgoq.github.io/TurboQuant/api/kv, TurboQuantCompressorMSE.compress);
the pages call the coordinate distribution a predictable bell curve (turboquant-pytorch
index page, "The Core: Random Rotation + Lloyd-Max Quantization").

Readings where the pages are silent (the solver body is not printed):
  * Density: after a Haar rotation a unit vector is uniform on the sphere S^{d-1}; one
    coordinate X has density f_d(x) = C_d (1 - x^2)^((d-3)/2) on [-1, 1] with
    C_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)); (X + 1)/2 ~ Beta((d-1)/2, (d-1)/2);
    E[X^2] = 1/d.
  * Solver: Lloyd's iteration (boundaries at midpoints of neighbouring centroids,
    centroids at the conditional mean of their cell) run to a fixed point. f_d is
    log-concave for d >= 3, so the fixed point is unique and start and stop rules do not
    change the answer beyond rounding.
  * Symmetry: f_d is even, so the codebook is odd-symmetric and the middle boundary is 0;
    only the positive half is iterated.

Cell integrals in closed form:
  mass        P(a < X < b) from the regularized incomplete beta function;
  1st moment  int_a^b x f_d = C_d [(1-a^2)^((d-1)/2) - (1-b^2)^((d-1)/2)] / (d-1);
  2nd moment  int_a^b x^2 f_d = P_d(a,b) - ((d-1)/d) P_{d+2}(a,b)
              (from x^2 (1-x^2)^m = (1-x^2)^m - (1-x^2)^(m+1) and C_d / C_{d+2} = (d-1)/d).
The same solver also runs on N(0, sigma^2), which is the d -> infinity limit of
sqrt(d) X and the textbook case (Max 1960) used to pin it.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
from scipy import special


class SphereCoordinate:
    """Density of one coordinate of a uniform random unit vector in R^d (d >= 3)."""

    def __init__(self, d: int):
        if d < 3:
            raise ValueError("the sphere-coordinate density needs d >= 3")
        self.d = int(d)
        self.alpha = (d - 1) / 2.0
        self.m = (d - 3) / 2.0
        self.log_c = math.lgamma(d / 2.0) - 0.5 * math.log(math.pi) - math.lgamma((d - 1) / 2.0)
        self.variance = 1.0 / d
        self.upper = 1.0

    def pdf(self, x):
        x = np.asarray(x, dtype=np.float64)
        inside = np.abs(x) < 1.0
        xs = np.where(inside, x, 0.0)
        val = np.exp(self.log_c + self.m * np.log1p(-xs * xs))
        return np.where(inside, val, 0.0)

    def upper_tail(self, x: float) -> float:
        """P(X > x)."""
        if x >= 1.0:
            return 0.0
        if x <= -1.0:
            return 1.0
        return float(special.betainc(self.alpha, self.alpha, (1.0 - x) / 2.0))

    def mass(self, a: float, b: float) -> float:
        return _mass_from_tail(self.upper_tail, a, b)

    def _g(self, x: float) -> float:
        # antiderivative (up to sign) of x f_d(x): C_d (1-x^2)^((d-1)/2) / (d-1)
        if abs(x) >= 1.0:
            return 0.0
        k = self.m + 1.0
        return math.exp(self.log_c + k * math.log1p(-x * x)) / (2.0 * k)

    def first_moment(self, a: float, b: float) -> float:
        return self._g(a) - self._g(b)

    def second_moment(self, a: float, b: float) -> float:
        wider = SphereCoordinate(self.d + 2)
        return self.mass(a, b) - (self.d - 1) / self.d * wider.mass(a, b)


class Gaussian:
    """N(0, sigma^2), the d -> infinity limit of sqrt(d) times a sphere coordinate."""

    def __init__(self, sigma: float = 1.0):
        self.sigma = float(sigma)
        self.variance = self.sigma ** 2
        self.upper = math.inf

    def pdf(self, x):
        z = np.asarray(x, dtype=np.float64) / self.sigma
        return np.exp(-0.5 * z * z) / (self.sigma * math.sqrt(2.0 * math.pi))

    def upper_tail(self, x: float) -> float:
        return 0.5 * math.erfc(x / (self.sigma * math.sqrt(2.0)))

    def mass(self, a: float, b: float) -> float:
        return _mass_from_tail(self.upper_tail, a, b)

    def _phi(self, x: float) -> float:
        if math.isinf(x):
            return 0.0
        return float(self.pdf(x))

    def first_moment(self, a: float, b: float) -> float:
        return self.variance * (self._phi(a) - self._phi(b))

    def second_moment(self, a: float, b: float) -> float:
        def xphi(x):
            return 0.0 if math.isinf(x) else x * self._phi(x)
        return self.variance * (self.mass(a, b) + xphi(a) - xphi(b))


def _mass_from_tail(tail, a: float, b: float) -> float:
    """P(a < X < b) for an even density, taken from the nearer tail to avoid cancellation."""
    if a >= 0.0:
        return tail(a) - tail(b)
    if b <= 0.0:
        return tail(-b) - tail(-a)
    return 1.0 - tail(b) - tail(-a)


@dataclass
class Codebook:
    bits: int
    centroids: np.ndarray    # [2^b] ascending
    thresholds: np.ndarray   # [2^b - 1] ascending, midpoints of neighbouring centroids
    mse: float               # expected squared error of one coordinate
    iterations: int


def lloyd_max(density, bits: int, tol: float = 0.0, max_iter: int = 1_000_000) -> Codebook:
    """Symmetric Lloyd-Max quantizer with 2^bits levels for an even density.

    Iterates on the positive half: boundaries 0 = t_0 < t_1 < ... < t_{h-1} < t_h = upper,
    interior boundaries at centroid midpoints, centroid k at E[X | t_k < X < t_{k+1}].
    Stops when an iteration no longer changes any centroid by more than `tol` (0: until
    the iterates stop moving in float64, i.e. the fixed point to rounding).
    """
    if bits < 1:
        raise ValueError("bits must be >= 1")
    h = 2 ** (bits - 1)
    sd = math.sqrt(density.variance)
    upper = density.upper
    # start: evenly spaced positive levels inside +-3 sd (any start reaches the same point)
    span = min(3.0 * sd, 0.9 * upper)
    c = np.array([(k + 0.5) * span / h for k in range(h)])
    it = 0
    prev_step = math.inf
    stall = 0
    for it in range(1, max_iter + 1):
        t = np.concatenate(([0.0], 0.5 * (c[:-1] + c[1:]), [upper]))
        new = np.array([density.first_moment(t[k], t[k + 1]) / density.mass(t[k], t[k + 1])
                        for k in range(h)])
        step = float(np.max(np.abs(new - c)))
        c = new
        if step <= tol:
            break
        # float64 fixed point: the step stops shrinking once it is at rounding level
        if step >= prev_step and step < 1e-14 * sd:
            stall += 1
            if stall >= 3:
                break
        prev_step = step
    centroids = np.concatenate((-c[::-1], c))
    thresholds = 0.5 * (centroids[:-1] + centroids[1:])
    thresholds[h - 1] = 0.0
    return Codebook(bits=bits, centroids=centroids, thresholds=thresholds,
                    mse=distortion(density, centroids, thresholds), iterations=it)


def distortion(density, centroids, thresholds) -> float:
    """E[(X - Q(X))^2] = sum over cells of int (x - c_k)^2 f, from the closed-form cell moments."""
    lo = -density.upper
    edges = np.concatenate(([lo], thresholds, [density.upper]))
    total = 0.0
    for k, ck in enumerate(centroids):
        a, b = edges[k], edges[k + 1]
        total += (density.second_moment(a, b) - 2.0 * ck * density.first_moment(a, b)
                  + ck * ck * density.mass(a, b))
    return total


def cell_masses(density, thresholds) -> np.ndarray:
    edges = np.concatenate(([-density.upper], thresholds, [density.upper]))
    return np.array([density.mass(edges[k], edges[k + 1]) for k in range(len(edges) - 1)])


_CACHE: dict = {}


def codebook(d: int, bits: int) -> Codebook:
    """The codebook for head dimension d and b bits (sphere-coordinate density, cached)."""
    key = (int(d), int(bits))
    if key not in _CACHE:
        _CACHE[key] = lloyd_max(SphereCoordinate(d), bits)
    return _CACHE[key]
