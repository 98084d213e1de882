"""Pins of the oracle's codebooks against printed values and independent maths."""

import numpy as np
import pytest
from scipy import integrate
from scipy.stats import norm

from oracle import codebook as cb


def _page_table(golden):
    return np.array([float(x) for x in golden("page_centroids_d128_4bit.txt")])


def test_quantile_mean_reproduces_page_table(golden):
    page = _page_table(golden)
    c = cb.quantile_mean(128, 4)
    # tolerance 5e-4 on every printed value; the construction actually lands
    # within 5e-5 of the 4-decimal print
    assert np.max(np.abs(c - page)) < 5e-4
    assert np.max(np.abs(c - page)) < 5e-5


def test_page_outer_value_is_197_sigma(golden):
    page = _page_table(golden)
    sigma = 1 / np.sqrt(128)
    assert abs(page[-1] / sigma - 1.97) < 0.005
    assert abs(cb.quantile_mean(128, 4)[-1] / sigma - 1.97) < 0.005


def _max_table(golden):
    rows = {}
    for ln in golden("max1960_gaussian_quantizer.txt"):
        k, vals = ln.split(":")
        rows[int(k)] = np.array([float(v) for v in vals.split()])
    return rows


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_matches_max_1960(golden, bits):
    ref = _max_table(golden)[bits]
    c = cb.lloyd_max(1, bits)
    half = c[len(c) // 2:]
    assert np.max(np.abs(half - ref)) < 1.5e-4
    # odd symmetry
    assert np.allclose(c, -c[::-1], atol=1e-14)


def test_lloyd_max_outer_matches_page_quote():
    # the page quotes the N(0,1)-scaled 16-level table's outer value as
    # 2.73 sigma = 0.2416 at d = 128
    c = cb.lloyd_max(128, 4)
    assert abs(c[-1] - 0.2416) < 1e-4
    assert abs(c[-1] * np.sqrt(128) - 2.73) < 0.005


def test_one_bit_constructions_coincide_with_closed_form():
    for d in (64, 128, 256):
        ref = np.sqrt(2 / np.pi) / np.sqrt(d)
        assert np.allclose(cb.quantile_mean(d, 1), [-ref, ref], rtol=1e-12)
        assert np.allclose(cb.lloyd_max(d, 1), [-ref, ref], rtol=1e-10)


@pytest.mark.parametrize("d,bits", [(128, 4), (128, 3), (256, 4), (128, 2)])
def test_quantile_mean_is_conditional_mean_by_quadrature(d, bits):
    """Numerical integration of x p(x) over each equal-mass bin."""
    K = 1 << bits
    sigma = 1 / np.sqrt(d)
    edges = norm.ppf(np.arange(K + 1) / K, scale=sigma)
    c = cb.quantile_mean(d, bits)
    for k in range(K):
        a, b = edges[k], edges[k + 1]
        num, _ = integrate.quad(lambda x: x * norm.pdf(x, scale=sigma), a, b, epsabs=1e-14)
        assert abs(num * K - c[k]) < 1e-9


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_max_is_a_fixed_point_by_quadrature(bits):
    d = 128
    sigma = 1 / np.sqrt(d)
    c = cb.lloyd_max(d, bits)
    edges = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
    for k in range(len(c)):
        a, b = edges[k], edges[k + 1]
        num, _ = integrate.quad(lambda x: x * norm.pdf(x, scale=sigma), a, b, epsabs=1e-15)
        den, _ = integrate.quad(lambda x: norm.pdf(x, scale=sigma), a, b, epsabs=1e-15)
        assert abs(num / den - c[k]) < 1e-9


def _mse_by_quadrature(c, sigma):
    edges = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
    tot = 0.0
    for k in range(len(c)):
        v, _ = integrate.quad(lambda x: (x - c[k]) ** 2 * norm.pdf(x, scale=sigma),
                              edges[k], edges[k + 1], epsabs=1e-16)
        tot += v
    return tot


@pytest.mark.parametrize("kind", [cb.QUANTILE_MEAN, cb.LLOYD_MAX])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantizer_mse_monte_carlo_matches_quadrature(kind, bits):
    d = 128
    sigma = 1 / np.sqrt(d)
    t = cb.tables(d, bits, kind)
    x = np.random.default_rng(11).normal(scale=sigma, size=400_000)
    err = (x - t.centroids.astype(np.float64)[cb.quantize(x.astype(np.float32), t.bounds)]) ** 2
    ref = _mse_by_quadrature(t.centroids64, sigma)
    se = err.std() / np.sqrt(err.size)
    assert abs(err.mean() - ref) < 4 * se
    # Lloyd-Max must beat the quantile construction (it minimizes the MSE)
    if kind == cb.LLOYD_MAX:
        assert ref < _mse_by_quadrature(cb.quantile_mean(d, bits), sigma)


def test_lloyd_max_4bit_mse_vs_quantile_mean():
    # closed-form ratios of the two constructions' per-coordinate MSE in
    # units of sigma^2 (quadrature; the Lloyd-Max figure is Max's 0.009497)
    s2 = 1.0 / 128
    lm = _mse_by_quadrature(cb.lloyd_max(128, 4), np.sqrt(s2)) / s2
    assert abs(lm - 0.0095) < 1e-4


@pytest.mark.parametrize("kind", [cb.QUANTILE_MEAN, cb.LLOYD_MAX])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_decision_rule_ties_and_monotonicity(kind, bits):
    t = cb.tables(128, bits, kind)
    # every centroid maps to its own code
    assert np.array_equal(cb.quantize(t.centroids, t.bounds), np.arange(1 << bits))
    # a value equal to a boundary takes the lower code; the next fp32 above takes the upper
    up = np.nextafter(t.bounds, np.float32(np.inf), dtype=np.float32)
    assert np.array_equal(cb.quantize(t.bounds, t.bounds), np.arange((1 << bits) - 1))
    assert np.array_equal(cb.quantize(up, t.bounds), np.arange(1, 1 << bits))
    # monotone non-decreasing in the input
    y = np.sort(np.random.default_rng(3).normal(scale=0.2, size=10_000).astype(np.float32))
    assert np.all(np.diff(cb.quantize(y, t.bounds)) >= 0)
    # zero is the symmetric midpoint and lands on the lower middle code
    assert cb.quantize(np.float32(0.0), t.bounds) == (1 << bits) // 2 - 1


def test_tables_round_once_to_fp32():
    t = cb.tables(128, 4, cb.QUANTILE_MEAN)
    assert t.centroids.dtype == np.float32 and t.bounds.dtype == np.float32
    mid64 = 0.5 * (t.centroids64[:-1] + t.centroids64[1:])
    assert np.array_equal(t.bounds, mid64.astype(np.float32))
    assert np.all(np.diff(t.bounds) > 0)
