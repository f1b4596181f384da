"""Haar-random orthogonal rotation, float64 (oracle; test infrastructure only).

KV Cache API page (ginkgoq.github.io/TurboQuant/api/kv), TurboQuantCompressorV2.__init__
(also TurboQuantCompressorMSE.__init__, MSECompressor.__init__): a seeded CPU generator
draws a d x d standard-normal matrix G; G is QR-factored; the rotation is Q with each
column j multiplied by the sign of R[j, j], a zero sign counting as +1.

Reading: the page factors in float32, which is orthogonal only to ~1e-6. The oracle
keeps the page's float32 draw (the input) and factors it in float64, so the result is
orthogonal to ~1e-15 and is the unique QR factor whose R has a positive diagonal.
"""

from __future__ import annotations

import numpy as np


def householder_qr(g):
    """Plain Householder QR of a square matrix in float64: returns (Q, R) with G = Q R."""
    r = np.array(g, dtype=np.float64, copy=True)
    d = r.shape[0]
    if r.shape != (d, d):
        raise ValueError("householder_qr expects a square matrix")
    q = np.eye(d)
    for k in range(d - 1):
        col = r[k:, k]
        norm = np.sqrt(np.dot(col, col))
        if norm == 0.0:
            continue
        alpha = -norm if col[0] >= 0 else norm
        v = col.copy()
        v[0] -= alpha
        vn = np.sqrt(np.dot(v, v))
        if vn == 0.0:
            continue
        v /= vn
        # reflect the trailing rows of R and accumulate Q = H_0 H_1 ... H_k
        r[k:, :] -= 2.0 * np.outer(v, v @ r[k:, :])
        q[:, k:] -= 2.0 * np.outer(q[:, k:] @ v, v)
    return q, r


def haar_rotation(gaussian):
    """Rotation Pi from a Gaussian draw: Q * sign(diag R) column-wise (sign 0 -> +1)."""
    q, r = householder_qr(gaussian)
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return q * s[None, :]


def haar_rotations(gaussians):
    """Stack version: [n, d, d] draws -> [n, d, d] rotations."""
    g = np.asarray(gaussians, dtype=np.float64)
    return np.stack([haar_rotation(gi) for gi in g])


def hadamard_matrix(d: int):
    """Walsh-Hadamard matrix of order d (a power of two), Sylvester's doubling:
    H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]]. Entries are +-1 and H H^T = d I."""
    if d < 1 or d & (d - 1):
        raise ValueError("hadamard_matrix: d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_rotation(d: int, signs=None):
    """Hadamard rotation: Pi = H_d diag(s) / sqrt(d), s in {+1, -1}^d (all +1 if None).

    Turbo Attention PyPI page, "The codec" table, "Hadamard rotation" row: the rotation is a
    Walsh-Hadamard transform, whose purpose there is to smear large channels over all
    coordinates; the query side uses it too. Reading: the orthonormal Sylvester-ordered transform, optionally preceded by a sign
    flip per input channel (a randomized Hadamard transform when the signs are drawn at
    random); y = Pi x means y = H (s * x) / sqrt(d).
    """
    s = np.ones(d) if signs is None else np.asarray(signs, dtype=np.float64).reshape(d)
    if not np.all(np.abs(s) == 1.0):
        raise ValueError("hadamard_rotation: signs must be +1 or -1")
    return hadamard_matrix(d) * s[None, :] / np.sqrt(d)
