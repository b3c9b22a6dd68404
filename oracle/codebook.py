"""Lloyd-Max scalar codebook for the rotated coordinates (oracle).

"FlashQuant" page, section "TurboQuant", step 3: after the random rotation
each coordinate is quantized with a Lloyd-Max scalar quantizer; for a Gaussian
the centroid update has a closed form. Section "架构设计" lists the codebook
(Lloyd-Max, closed form) as a core component. The "TurboQuant" blog, "Couche
2", describes the search over the 2^b - 1 boundaries.

Readings taken where the pages are silent or disagree:
* distribution: N(0, 1) levels scaled by 1/sqrt(d) (the blog's spherical-Beta
  codebook is not used);
* the codebook is the Lloyd fixed point in float64 (iterate until the largest
  level change is below 1e-15, a few ulps), not a fixed iteration count;
* levels are made exactly antisymmetric (l[L-1-i] = -l[i]) so the middle
  boundary is exactly 0;
* stored values: level_i = fp32(l_i / sqrt(d)), boundary_i = fp32(b_i / sqrt(d)),
  each rounded once from float64.
"""
import numpy as np
from scipy.special import ndtr, ndtri


def _phi(x):
    """Standard normal density; 0 at +-inf."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    fin = np.isfinite(x)
    out[fin] = np.exp(-0.5 * x[fin] ** 2) / np.sqrt(2.0 * np.pi)
    return out


def _mass(a, b):
    """P(a < Z <= b) for Z ~ N(0,1), computed on the side of 0 where it is accurate."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    upper = a >= 0
    return np.where(upper, ndtr(-a) - ndtr(-b), ndtr(b) - ndtr(a))


def lloyd_max_gaussian(bits: int, tol: float = 1e-15, max_iter: int = 200000):
    """Fixed point of the Lloyd iteration for N(0,1) with 2**bits cells (float64).

    Returns (levels, boundaries, iterations, residual), levels ascending,
    boundaries = midpoints of adjacent levels. Start: the cell quantiles
    Phi^{-1}((i + 1/2) / L). Update: boundaries to midpoints, then each level to
    the conditional mean of N(0,1) on its cell, (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
    """
    L = 1 << bits
    lev = ndtri((np.arange(L) + 0.5) / L)
    it = 0
    resid = np.inf
    while it < max_iter:
        bnd = 0.5 * (lev[:-1] + lev[1:])
        lo = np.concatenate([[-np.inf], bnd])
        hi = np.concatenate([bnd, [np.inf]])
        new = (_phi(lo) - _phi(hi)) / _mass(lo, hi)
        resid = float(np.max(np.abs(new - lev)))
        lev = new
        it += 1
        if resid < tol:
            break
    lev = 0.5 * (lev - lev[::-1])
    bnd = 0.5 * (lev[:-1] + lev[1:])
    return lev, bnd, it, resid


def gaussian_mse(levels, boundaries) -> float:
    """E[(Z - Q(Z))^2] for Z ~ N(0,1) under the given levels/boundaries, in closed form.

    On a cell (a, b] with level c: E[(Z-c)^2 1{a<Z<=b}] = m2 - 2 c m1 + c^2 m0 with
    m0 = Phi(b)-Phi(a), m1 = phi(a)-phi(b), m2 = m0 + a phi(a) - b phi(b).
    """
    lev = np.asarray(levels, dtype=np.float64)
    bnd = np.asarray(boundaries, dtype=np.float64)
    lo = np.concatenate([[-np.inf], bnd])
    hi = np.concatenate([bnd, [np.inf]])
    m0 = _mass(lo, hi)
    m1 = _phi(lo) - _phi(hi)
    alo = np.zeros_like(lo)
    ahi = np.zeros_like(hi)
    flo, fhi = np.isfinite(lo), np.isfinite(hi)
    alo[flo] = lo[flo] * _phi(lo[flo])
    ahi[fhi] = hi[fhi] * _phi(hi[fhi])
    m2 = m0 + alo - ahi
    return float(np.sum(m2 - 2.0 * lev * m1 + lev * lev * m0))


def scaled_codebook(bits: int, head_dim: int):
    """The stored codebook: (levels fp32 [2^b], boundaries fp32 [2^b - 1]).

    Coordinates of a rotated unit vector in dimension d have variance 1/d, so the
    N(0,1) codebook is scaled by 1/sqrt(d) ("FlashQuant" page, "TurboQuant" step 3).
    """
    lev, bnd, _, _ = lloyd_max_gaussian(bits)
    s = np.sqrt(float(head_dim))
    return (lev / s).astype(np.float32), (bnd / s).astype(np.float32)


# ---------------------------------------------------------------------------
# Exact spherical marginal ("TurboQuant" blog, "Étape 2" and "Couche 2": after the
# rotation a coordinate follows the spherical Beta law; its Lloyd-Max codebook).
#
# A coordinate X of a uniform point on the unit sphere in R^d has density
# proportional to (1 - x^2)^((d-3)/2) on (-1, 1): (1 + X) / 2 ~ Beta(p, p) with
# p = (d - 1) / 2. On a cell (a, b]:
#   mass  P(a < X <= b) = I_{(1+b)/2}(p, p) - I_{(1+a)/2}(p, p)   (regularized
#         incomplete beta; for a >= 0 taken from the upper tail by symmetry);
#   first moment E[X 1{a<X<=b}] = ((1 - a^2)^p - (1 - b^2)^p) / (2 p Z),
#         Z = 2^(2p-1) B(p, p) the normalizer of (1 - x^2)^(p-1).
# Readings: the same float64 fixed point as the Gaussian codebook (not the blog's
# 50 iterations), started from the cell quantiles of the Beta law, made exactly
# antisymmetric; the levels are already in the unit-vector scale (no 1/sqrt(d)).
# ---------------------------------------------------------------------------
from scipy.special import betainc, betaincinv, betaln  # noqa: E402


def _sphere_mass(a, b, p):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    upper = a >= 0
    lower_form = betainc(p, p, (1.0 + b) / 2.0) - betainc(p, p, (1.0 + a) / 2.0)
    upper_form = betainc(p, p, (1.0 - a) / 2.0) - betainc(p, p, (1.0 - b) / 2.0)
    return np.where(upper, upper_form, lower_form)


def _sphere_m1(a, b, p):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    log_z = (2.0 * p - 1.0) * np.log(2.0) + betaln(p, p)
    with np.errstate(divide="ignore"):  # log(0) at x = +-1: the term is 0
        ta = np.exp(p * np.log1p(-np.minimum(a * a, 1.0)) - log_z)
        tb = np.exp(p * np.log1p(-np.minimum(b * b, 1.0)) - log_z)
    return (ta - tb) / (2.0 * p)


def lloyd_max_sphere(bits: int, d: int, tol: float = 1e-15, max_iter: int = 2000000):
    """Fixed point of the Lloyd iteration for the spherical marginal in R^d (float64).

    Returns (levels, boundaries, iterations, residual), levels ascending in (-1, 1).
    Start: the cell quantiles 2 I^{-1}((i + 1/2) / L; p, p) - 1. Update: boundaries to
    midpoints, then each level to the conditional mean on its cell.
    """
    if d < 3:
        raise ValueError("the spherical marginal needs d >= 3")
    p = (d - 1) / 2.0
    L = 1 << bits
    lev = 2.0 * betaincinv(p, p, (np.arange(L) + 0.5) / L) - 1.0
    it = 0
    resid = np.inf
    while it < max_iter:
        bnd = 0.5 * (lev[:-1] + lev[1:])
        lo = np.concatenate([[-1.0], bnd])
        hi = np.concatenate([bnd, [1.0]])
        new = _sphere_m1(lo, hi, p) / _sphere_mass(lo, hi, p)
        resid = float(np.max(np.abs(new - lev)))
        lev = new
        it += 1
        if resid < tol:
            break
    lev = 0.5 * (lev - lev[::-1])
    bnd = 0.5 * (lev[:-1] + lev[1:])
    return lev, bnd, it, resid


def sphere_codebook(bits: int, head_dim: int):
    """Stored spherical codebook: (levels fp32 [2^b], boundaries fp32 [2^b - 1]),
    each rounded once from float64."""
    lev, bnd, _, _ = lloyd_max_sphere(bits, head_dim)
    return lev.astype(np.float32), bnd.astype(np.float32)
