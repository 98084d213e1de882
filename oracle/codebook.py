"""Scalar codebooks for the post-rotation coordinate law N(0, 1/d).

After a norm is taken out and a random orthogonal rotation is applied, each
coordinate of a d-dimensional unit vector is close to N(0, 1/d) ("turbo4
post-mortem", section 5: the rotated coordinate law, sigma = 1/sqrt(128) for
d = 128).  Two constructions are provided:

``quantile_mean``
    The conditional expectation of N(0, sigma^2) inside each of K
    equal-probability intervals ("turbo4 post-mortem", section 5: each
    centroid is the conditional mean of its quantile interval).  This is one
    Lloyd centroid update applied to the quantile partition, and it is the
    construction whose d = 128, K = 16 values the page prints.

``lloyd_max``
    The fixed point of Lloyd's two alternating conditions (boundaries at
    midpoints, centroids at conditional means) for the same Gaussian law
    ("turbo4 post-mortem", section 5, on the Python reference's Gaussian
    Lloyd iteration; "TurboQuant Triton deep dive", write path: Lloyd-Max
    codebook per (d, bits); "PolarQuant-KV", section 2.2).

Both return float64 centroids; ``tables`` rounds them and their midpoints to
fp32, the precision in which the quantization decision is taken.
"""

from dataclasses import dataclass

import numpy as np
from scipy.special import ndtr, ndtri

QUANTILE_MEAN = 0
LLOYD_MAX = 1


def _pdf(z):
    """Standard normal density, zero at +-inf."""
    z = np.asarray(z, dtype=np.float64)
    out = np.zeros_like(z)
    fin = np.isfinite(z)
    out[fin] = np.exp(-0.5 * z[fin] ** 2) / np.sqrt(2.0 * np.pi)
    return out


def _conditional_means(edges_std):
    """E[Z | a < Z < b] for Z ~ N(0, 1), for consecutive standardized edges."""
    a, b = edges_std[:-1], edges_std[1:]
    mass = ndtr(b) - ndtr(a)
    return (_pdf(a) - _pdf(b)) / mass


def quantile_mean(d, bits):
    """Conditional means of the 2**bits equal-probability bins of N(0, 1/d)."""
    k = 1 << bits
    sigma = 1.0 / np.sqrt(d)
    edges = ndtri(np.arange(k + 1) / k)  # -inf ... +inf
    # every bin holds probability 1/k, so the conditional mean is
    # sigma * k * (pdf(left) - pdf(right)); the table is made exactly
    # odd-symmetric so that zero sits on the middle boundary
    c = k * (_pdf(edges[:-1]) - _pdf(edges[1:]))
    return sigma * 0.5 * (c - c[::-1])


def lloyd_max(d, bits, tol=1e-13, max_iter=200000):
    """Fixed point of the Lloyd conditions for N(0, 1/d) with 2**bits levels."""
    k = 1 << bits
    sigma = 1.0 / np.sqrt(d)
    c = quantile_mean(1, bits)  # standardized start
    for _ in range(max_iter):
        edges = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        c_new = _conditional_means(edges)
        c_new = 0.5 * (c_new - c_new[::-1])  # keep the table exactly odd-symmetric
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta < tol:
            break
    else:  # pragma: no cover - convergence is fast for these sizes
        raise RuntimeError("Lloyd iteration did not converge")
    assert c.shape == (k,)
    return sigma * c


@dataclass(frozen=True)
class Tables:
    """fp32 centroids and fp32 decision boundaries of one codebook."""

    d: int
    bits: int
    kind: int
    centroids: np.ndarray  # float32 [K]
    bounds: np.ndarray  # float32 [K-1], boundary k separates code k and k+1
    centroids64: np.ndarray  # float64 [K], before rounding


def tables(d, bits, kind=QUANTILE_MEAN):
    """Centroids and midpoints, each rounded once to fp32."""
    if kind == QUANTILE_MEAN:
        c = quantile_mean(d, bits)
    elif kind == LLOYD_MAX:
        c = lloyd_max(d, bits)
    else:
        raise ValueError(f"unknown codebook kind {kind}")
    mid = 0.5 * (c[:-1] + c[1:])
    return Tables(d, bits, kind, c.astype(np.float32), mid.astype(np.float32), c)


def quantize(y32, bounds32):
    """Code of each fp32 coordinate: the number of boundaries strictly below it.

    The comparison is done on fp32 values; a coordinate equal to a boundary
    takes the lower code.  With boundaries at midpoints this is the nearest
    centroid ("turbo4 post-mortem", section 1: nearest-centroid encoding).
    """
    y32 = np.asarray(y32, dtype=np.float32)
    return np.searchsorted(bounds32, y32, side="left").astype(np.int64)
