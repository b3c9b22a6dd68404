"""Pins of the oracle's random streams and rotations.

SplitMix64 reference outputs come from the published generator (Steele, Lea &
Flood 2014; Vigna's reference implementation seeded with 0). The rotation facts
are the defining properties of a Haar orthogonal matrix and of the
Sylvester Hadamard matrix ("TurboQuant" blog, "Couche 1").
"""
import numpy as np
import pytest
from scipy import stats
from scipy.linalg import hadamard

from oracle import rng, rotation


def test_splitmix64_reference_outputs():
    # first three outputs of the reference generator started from state 0
    assert rng.splitmix64(0, 0) == 0xE220A8397B1DCDAF
    assert rng.splitmix64(0, 1) == 0x6E789E6AA1B965F4
    assert rng.splitmix64(0, 2) == 0x06C45D188009454F


def test_uniform_and_gaussian_streams():
    u = np.array([rng.uniform(7, i) for i in range(20000)])
    assert u.min() > 0 and u.max() < 1
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    g = rng.gaussian(7, 20001)
    assert g.shape == (20001,)
    assert stats.kstest(g, "norm").pvalue > 1e-3
    # Box-Muller pair structure: g[0], g[1] share the radius sqrt(-2 ln u0)
    r2 = -2.0 * np.log(rng.uniform(7, 0))
    assert abs(g[0] ** 2 + g[1] ** 2 - r2) < 1e-12
    s = rng.signs(7, 4000)
    assert set(np.unique(s)) == {-1.0, 1.0}
    assert abs(s.mean()) < 4 / np.sqrt(4000)


@pytest.mark.parametrize("d", [16, 128])
def test_haar_is_orthogonal(d):
    pi = rotation.haar_rotation(1, d)
    assert np.max(np.abs(pi @ pi.T - np.eye(d))) < 1e-12
    pi32 = rotation.stored(pi)
    assert np.max(np.abs(pi32 @ pi32.T - np.eye(d))) < 1e-6
    x = np.random.default_rng(0).standard_normal((50, d))
    assert np.allclose(np.linalg.norm(x @ pi.T, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)


def test_haar_distribution_first_moments():
    """Over many seeds, Pi[0,0] and the trace have mean 0 and Pi[i,j] variance 1/d.

    QR without the sign fix is orthogonal but not Haar: its diagonal is biased,
    which this test detects."""
    d, n = 8, 3000
    p00, tr = np.empty(n), np.empty(n)
    for s in range(n):
        pi = rotation.haar_rotation(1000 + s, d)
        p00[s] = pi[0, 0]
        tr[s] = np.trace(pi)
    se = np.sqrt(1.0 / d / n)
    assert abs(p00.mean()) < 4 * se
    assert abs(p00.var() - 1.0 / d) < 0.1 / d
    assert abs(tr.mean()) < 4 * np.sqrt(1.0 / n)  # Var(trace) = 1 for Haar O(d)


def test_rotated_unit_coordinates_have_variance_one_over_d():
    d = 128
    x = np.random.default_rng(3).standard_normal(d)
    u = x / np.linalg.norm(x)
    ys = np.array([rotation.haar_rotation(50 + s, d) @ u for s in range(60)])
    assert abs(np.mean(ys ** 2) - 1.0 / d) < 0.1 / d


@pytest.mark.parametrize("d", [8, 128])
def test_fwht_equals_dense_sylvester(d):
    s = rotation.wht_signs(5, d)
    h = hadamard(d).astype(np.float64)
    assert np.array_equal(h @ h, d * np.eye(d))
    dense = h @ np.diag(s) / np.sqrt(d)
    assert np.allclose(rotation.wht_matrix(s), dense, atol=1e-15)
    x = np.random.default_rng(1).standard_normal((10, d))
    assert np.allclose(rotation.fwht_rotate(x, s), x @ dense.T, atol=1e-13)
    pw = rotation.wht_matrix(s)
    assert np.max(np.abs(pw @ pw.T - np.eye(d))) < 1e-14


def test_qjl_matrix_is_standard_gaussian():
    s = rotation.qjl_matrix(2, 128, 128)
    assert s.shape == (128, 128)
    assert stats.kstest(s.ravel(), "norm").pvalue > 1e-3
    assert np.array_equal(s.ravel(), rng.gaussian(2, 128 * 128))
