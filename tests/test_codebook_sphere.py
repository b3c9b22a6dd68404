"""CPU pins of the spherical-marginal codebook ("TurboQuant" blog, "Étape 2" and
"Couche 2": a rotated coordinate follows the spherical Beta law, quantized with its
Lloyd-Max codebook) in the oracle, and the host builder fq_build_levels against it.

The oracle is pinned by things other than itself:
* d = 3: the law is uniform on (-1, 1), whose Lloyd-Max quantizer is the uniform one
  (levels -1 + (2i + 1) / L);
* the density's normalization and its second moment E[X^2] = 1/d (a coordinate of a
  unit vector), and the closed-form first moments against numerical quadrature;
* the centroid condition at the fixed point by quadrature;
* d -> infinity: sqrt(d) X tends to N(0, 1), so sqrt(d) * levels tends to the Gaussian
  Lloyd-Max levels, at rate 1/d;
* Monte Carlo: first coordinates of normalized Gaussian vectors, conditional means
  per cell;
* optimality: lower mean squared error under the spherical law than the Gaussian
  codebook scaled by 1/sqrt(d), and any single-level perturbation raises it.
"""
import numpy as np
import pytest
from scipy import integrate
from scipy.special import betaln

from kv_cache_vector_tq4_amd import fq
from oracle import codebook as cb


def _density(d):
    p = (d - 1) / 2.0
    log_z = (2.0 * p - 1.0) * np.log(2.0) + betaln(p, p)
    return lambda x: np.exp((p - 1.0) * np.log1p(-x * x) - log_z) if abs(x) < 1 else 0.0


def _cells(bnd):
    return np.concatenate([[-1.0], bnd]), np.concatenate([bnd, [1.0]])


@pytest.mark.parametrize("bits", [2, 4])
def test_d3_is_the_uniform_quantizer(bits):
    lev, bnd, _, resid = cb.lloyd_max_sphere(bits, 3)
    L = 1 << bits
    assert resid < 1e-15
    assert np.allclose(lev, -1.0 + (2 * np.arange(L) + 1.0) / L, rtol=0, atol=1e-15)
    assert np.allclose(bnd, -1.0 + 2.0 * np.arange(1, L) / L, rtol=0, atol=1e-15)


@pytest.mark.parametrize("d", [3, 16, 128])
def test_density_normalization_and_second_moment(d):
    f = _density(d)
    mass, _ = integrate.quad(f, -1, 1, epsabs=1e-14, epsrel=1e-13, limit=200)
    m2, _ = integrate.quad(lambda x: x * x * f(x), -1, 1, epsabs=1e-15, epsrel=1e-12, limit=200)
    assert abs(mass - 1.0) < 1e-12
    assert abs(m2 - 1.0 / d) < 1e-12
    p = (d - 1) / 2.0
    assert abs(float(cb._sphere_mass(-1.0, 1.0, p)) - 1.0) < 1e-14
    # closed-form cell masses and first moments against quadrature
    for a, b in [(-1.0, -0.3), (-0.2, 0.05), (0.0, 0.1), (0.4, 1.0)]:
        m0, _ = integrate.quad(f, a, b, epsabs=1e-16, epsrel=1e-12, limit=200)
        m1, _ = integrate.quad(lambda x: x * f(x), a, b, epsabs=1e-16, epsrel=1e-12, limit=200)
        assert abs(float(cb._sphere_mass(a, b, p)) - m0) < 1e-12
        assert abs(float(cb._sphere_m1(a, b, p)) - m1) < 1e-12


@pytest.mark.parametrize("bits", [2, 4])
def test_centroid_condition_at_d128(bits):
    d = 128
    lev, bnd, it, resid = cb.lloyd_max_sphere(bits, d)
    assert resid < 1e-15 and it < 10000
    assert np.array_equal(lev, -lev[::-1])
    assert np.array_equal(bnd, 0.5 * (lev[:-1] + lev[1:]))
    f = _density(d)
    for c, a, b in zip(lev, *_cells(bnd)):
        m0, _ = integrate.quad(f, a, b, epsabs=1e-16, epsrel=1e-13, limit=200)
        m1, _ = integrate.quad(lambda x: x * f(x), a, b, epsabs=1e-17, epsrel=1e-13, limit=200)
        assert abs(c - m1 / m0) < 1e-12


def test_large_d_tends_to_the_gaussian_codebook_at_rate_1_over_d():
    g, _, _, _ = cb.lloyd_max_gaussian(4)
    diff = {}
    for d in (1000, 1000000):
        lev, _, _, _ = cb.lloyd_max_sphere(4, d)
        diff[d] = float(np.max(np.abs(lev * np.sqrt(d) - g)))
    assert diff[1000000] < 1e-5
    assert 900 < diff[1000] / diff[1000000] < 1100


@pytest.mark.parametrize("bits", [2, 4])
def test_monte_carlo_conditional_means(bits):
    d = 128
    lev, bnd, _, _ = cb.lloyd_max_sphere(bits, d)
    rng = np.random.default_rng(11)
    xs = []
    for _ in range(4):
        g = rng.standard_normal((100000, d))
        xs.append(g[:, 0] / np.linalg.norm(g, axis=1))
    x = np.concatenate(xs)
    cell = np.searchsorted(bnd, x)
    for i, c in enumerate(lev):
        xi = x[cell == i]
        se = xi.std() / np.sqrt(len(xi))
        assert abs(xi.mean() - c) < 5 * se + 1e-12, (i, xi.mean(), c, se)


def _mse(lev, bnd, d):
    f = _density(d)
    tot = 0.0
    for c, a, b in zip(lev, *_cells(bnd)):
        v, _ = integrate.quad(lambda x: (x - c) ** 2 * f(x), a, b, epsabs=1e-17, epsrel=1e-12, limit=200)
        tot += v
    return tot


@pytest.mark.parametrize("bits", [2, 4])
def test_lower_mse_than_the_scaled_gaussian_codebook_and_locally_optimal(bits):
    d = 128
    lev, bnd, _, _ = cb.lloyd_max_sphere(bits, d)
    g, gb, _, _ = cb.lloyd_max_gaussian(bits)
    best = _mse(lev, bnd, d)
    assert best < _mse(g / np.sqrt(d), gb / np.sqrt(d), d)
    for i in range(len(lev)):
        for eps in (-1e-3, 1e-3):
            l2 = lev.copy()
            l2[i] += eps
            assert _mse(l2, 0.5 * (l2[:-1] + l2[1:]), d) > best


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [3, 16, 128, 256])
def test_host_builder_matches_the_oracle(bits, d):
    lev, bnd = fq.build_levels(bits, d, fq.CB_SPHERE)
    ol, ob = cb.sphere_codebook(bits, d)
    assert np.array_equal(lev, ol) and np.array_equal(bnd, ob)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_host_gaussian_kind_is_the_quantizer_codebook(bits):
    lev, bnd = fq.build_levels(bits, 128, fq.CB_GAUSSIAN)
    h = fq.build_codebook(bits)
    assert np.array_equal(lev, h["levels"]) and np.array_equal(bnd, h["boundaries"])
    ol, ob = cb.scaled_codebook(bits, 128)
    assert np.array_equal(lev, ol) and np.array_equal(bnd, ob)


def test_host_builder_argument_checks():
    import ctypes

    lib = fq.lib()
    lev = np.zeros(16, np.float32)
    bnd = np.zeros(15, np.float32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert lib.fq_build_levels(4, 128, 7, p(lev), p(bnd)) == 1  # bad kind
    assert lib.fq_build_levels(4, 128, fq.CB_SPHERE, None, p(bnd)) == 1
    assert lib.fq_build_levels(5, 128, fq.CB_SPHERE, p(lev), p(bnd)) == 2
    assert lib.fq_build_levels(4, 2, fq.CB_SPHERE, p(lev), p(bnd)) == 2
    assert lib.fq_build_levels(4, 257, fq.CB_SPHERE, p(lev), p(bnd)) == 2
