"""Pins of the oracle's random state and rotation."""

import numpy as np
import pytest
import scipy.linalg
from scipy import stats

from oracle import prng, rotation


def test_splitmix64_published_outputs(golden):
    ref = [int(x, 16) for x in golden("splitmix64_seed0.txt")]
    assert prng.splitmix64(0, 3) == ref


def test_splitmix64_is_counter_based():
    # output i depends only on seed + (i + 1) * gamma: a stream seeded at
    # seed + gamma is the first stream shifted by one
    a = prng.splitmix64(12345, 6)
    b = prng.splitmix64((12345 + prng.GOLDEN_GAMMA) & prng.MASK64, 5)
    assert a[1:] == b


def test_rotation_signs_balanced_and_seeded():
    s = prng.rotation_signs(7, 4096)
    assert set(np.unique(s)) == {-1.0, 1.0}
    assert abs(s.mean()) < 4 / np.sqrt(4096)
    assert not np.array_equal(prng.rotation_signs(7, 128), prng.rotation_signs(8, 128))
    assert np.array_equal(prng.rotation_signs(7, 128), s[:128])


def test_qjl_matrix_is_standard_normal():
    S = prng.qjl_matrix(99, 128).astype(np.float64).ravel()
    n = S.size
    assert abs(S.mean()) < 5 / np.sqrt(n)
    assert abs(S.var() - 1.0) < 5 * np.sqrt(2.0 / n)
    assert stats.kstest(S, "norm").pvalue > 1e-3
    # consecutive Box-Muller pairs are uncorrelated
    assert abs(np.corrcoef(S[0::2], S[1::2])[0, 1]) < 5 / np.sqrt(n / 2)


def test_qjl_matrix_independent_of_rotation_stream():
    a = prng.qjl_matrix(1, 64)
    b = prng.qjl_matrix(2, 64)
    assert abs(np.corrcoef(a.ravel(), b.ravel())[0, 1]) < 0.05


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_matches_scipy(d):
    assert np.array_equal(rotation.hadamard(d), scipy.linalg.hadamard(d))


@pytest.mark.parametrize("d", [16, 128, 256])
def test_rotation_is_orthogonal(d):
    s = prng.rotation_signs(3, d)
    P = rotation.rotation_matrix(s)
    assert np.max(np.abs(P @ P.T - np.eye(d))) < 1e-12
    P32 = P.astype(np.float32).astype(np.float64)
    assert np.max(np.abs(P32 @ P32.T - np.eye(d))) < 1e-6
    x = np.random.default_rng(0).normal(size=(50, d))
    y = rotation.rotate(x, s)
    assert np.max(np.abs(np.linalg.norm(y, axis=1) / np.linalg.norm(x, axis=1) - 1)) < 1e-12
    assert np.max(np.abs(rotation.unrotate(y, s) - x)) < 1e-12


@pytest.mark.parametrize("d", [8, 128])
def test_basis_vector_maps_to_signed_hadamard_column(d):
    # Pi e_m = s_m * H[:, m] / sqrt(d): signs act before the transform
    s = prng.rotation_signs(5, d)
    H = scipy.linalg.hadamard(d)
    for m in (0, 1, d - 1):
        e = np.zeros(d)
        e[m] = 1
        assert np.allclose(rotation.rotate(e[None], s)[0], s[m] * H[:, m] / np.sqrt(d), atol=1e-15)


def test_rotated_unit_vector_coordinates_have_variance_one_over_d():
    d = 128
    s = prng.rotation_signs(17, d)
    x = np.random.default_rng(1).normal(size=(4000, d))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    y = rotation.rotate(u, s).ravel()
    assert abs(y.var() * d - 1) < 0.02
    assert abs(y.mean()) < 5 / np.sqrt(y.size * d)
