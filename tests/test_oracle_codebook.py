"""Pins of the oracle's Lloyd-Max codebook against facts outside the oracle.

The pages ("FlashQuant" page, section "TurboQuant") state the MSE bound
(sqrt(3) pi / 2) / 4^b and that the Gaussian Lloyd-Max quantizer has a closed
form; the rest are textbook facts (Lloyd 1957 / Max 1960 optimality conditions,
the 1-bit closed form, the 2-bit table).
"""
import json
import os

import numpy as np
import pytest
from scipy import integrate
from scipy.stats import norm

from oracle import codebook

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lloyd_max_gaussian.json")


def test_one_bit_closed_form():
    lev, bnd, _, _ = codebook.lloyd_max_gaussian(1)
    assert np.allclose(lev, [-np.sqrt(2 / np.pi), np.sqrt(2 / np.pi)], atol=1e-14)
    assert bnd[0] == 0.0
    assert abs(codebook.gaussian_mse(lev, bnd) - (1 - 2 / np.pi)) < 1e-14


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_centroid_condition_by_quadrature(bits):
    """Each level is the conditional mean of N(0,1) on its cell, computed by numerical
    integration of the density (an independent route from the closed-form update)."""
    lev, bnd, _, _ = codebook.lloyd_max_gaussian(bits)
    edges = np.concatenate([[-np.inf], bnd, [np.inf]])
    for i, c in enumerate(lev):
        a, b = edges[i], edges[i + 1]
        num = integrate.quad(lambda z: z * norm.pdf(z), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        den = integrate.quad(norm.pdf, a, b, epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(num / den - c) < 1e-9, (i, num / den, c)
    # nearest-neighbour condition: boundaries are midpoints
    assert np.allclose(bnd, 0.5 * (lev[:-1] + lev[1:]), atol=0)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mse_by_quadrature_and_page_bound(bits):
    lev, bnd, _, _ = codebook.lloyd_max_gaussian(bits)
    edges = np.concatenate([[-np.inf], bnd, [np.inf]])
    mse_q = sum(
        integrate.quad(lambda z: (z - c) ** 2 * norm.pdf(z), edges[i], edges[i + 1],
                       epsabs=1e-15, epsrel=1e-12)[0]
        for i, c in enumerate(lev)
    )
    mse = codebook.gaussian_mse(lev, bnd)
    assert abs(mse - mse_q) < 1e-10
    bound = np.sqrt(3) * np.pi / 2 / 4 ** bits
    assert mse <= bound


def test_panter_dite_ratio_rises_toward_one():
    """MSE * 4^b / (sqrt(3) pi / 2) rises toward 1 (high-resolution limit of the bound)."""
    r = [codebook.gaussian_mse(*codebook.lloyd_max_gaussian(b)[:2]) * 4 ** b / (np.sqrt(3) * np.pi / 2)
         for b in range(1, 6)]
    assert all(x < y for x, y in zip(r, r[1:]))
    assert 0.85 < r[3] < 0.95 and r[4] < 1.0


def test_textbook_table():
    """Published Gaussian Lloyd-Max values (Max 1960), stored with their source."""
    with open(GOLDEN) as f:
        g = json.load(f)
    for key, entry in g["tables"].items():
        bits = int(key)
        lev, bnd, _, _ = codebook.lloyd_max_gaussian(bits)
        half = len(lev) // 2
        assert np.allclose(lev[half:], entry["positive_levels"], atol=entry["atol"])
        assert np.allclose(bnd[half - 1:], entry["nonnegative_boundaries"], atol=entry["atol"])
        assert abs(codebook.gaussian_mse(lev, bnd) - entry["mse"]) < entry.get("mse_atol", entry["atol"])


@pytest.mark.parametrize("bits", [2, 4])
def test_fixed_point_and_symmetry(bits):
    lev, bnd, it, resid = codebook.lloyd_max_gaussian(bits)
    assert resid < 1e-13
    assert np.array_equal(lev, -lev[::-1])
    assert bnd[len(bnd) // 2] == 0.0
    assert np.all(np.diff(lev) > 0)
    # 50 Lloyd steps from the quantile start are far from the fixed point at 4 bits
    if bits == 4:
        lev50, _, _, _ = codebook.lloyd_max_gaussian(4, tol=0, max_iter=50)
        assert np.max(np.abs(lev50 - lev)) > 1e-2


def test_scaled_codebook_rounding():
    lev32, bnd32 = codebook.scaled_codebook(4, 128)
    lev, bnd, _, _ = codebook.lloyd_max_gaussian(4)
    assert lev32.dtype == np.float32 and bnd32.dtype == np.float32
    assert np.array_equal(lev32, (lev / np.sqrt(128.0)).astype(np.float32))
    assert np.array_equal(bnd32, (bnd / np.sqrt(128.0)).astype(np.float32))
    assert bnd32[7] == 0.0
