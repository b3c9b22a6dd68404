"""Random orthogonal rotations (oracle).

* Haar rotation: "FlashQuant" page, "TurboQuant" step 2 (a Haar-distributed
  orthogonal matrix) and "架构设计" (Rotation: Haar QR matrix). Reading: draw
  G with i.i.d. N(0,1) entries, take the QR factorisation G = QR and set
  Pi = Q diag(sign(diag R)), which makes Pi Haar-distributed. The page applies
  R^T; since a Haar matrix and its transpose have the same law, the rotation is
  defined directly as y = Pi u.
* Randomized Walsh-Hadamard: "TurboQuant" blog, "Couche 1": multiply by a
  random sign vector, run the in-place butterflies (a+b, a-b) with doubling
  stride, divide by sqrt(n). As a matrix this is Pi_W = H diag(s) / sqrt(d)
  with H the Sylvester-ordered Hadamard matrix.

Both are returned as the fp32 matrix that the method stores; the rest of the
oracle uses that fp32 operator (promoted to float64).
"""
import numpy as np

from . import rng


def haar_rotation(seed: int, d: int) -> np.ndarray:
    """Pi (d x d, float64, exactly orthogonal up to fp64 rounding) from stream ``seed``.

    G[i, j] is Gaussian number i*d + j of the stream.
    """
    g = rng.gaussian(seed, d * d).reshape(d, d)
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def wht_signs(seed: int, d: int) -> np.ndarray:
    """The random sign vector s (d entries of +-1.0)."""
    return rng.signs(seed, d)


def fwht_rotate(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Randomized Walsh-Hadamard transform of the rows of x, by butterflies.

    x: [..., d] with d a power of two. Returns H (s * x) / sqrt(d) per row.
    """
    y = np.array(x, dtype=np.float64) * signs
    n = y.shape[-1]
    h = 1
    while h < n:
        y = y.reshape(y.shape[:-1] + (n // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (n,))
        h *= 2
    return y / np.sqrt(float(n))


def wht_matrix(signs: np.ndarray) -> np.ndarray:
    """Dense Pi_W = H diag(s) / sqrt(d), built by transforming the unit vectors."""
    d = signs.shape[0]
    return fwht_rotate(np.eye(d), signs).T


def qjl_matrix(seed: int, m: int, d: int) -> np.ndarray:
    """The QJL projection S (m x d), i.i.d. N(0,1), from stream ``seed``.

    "FlashQuant" page, section "QJL". The page calls S a random sign matrix but
    also states the estimator is unbiased, which holds exactly for Gaussian S;
    the Gaussian reading is taken. S[i, j] is Gaussian number i*d + j.
    """
    return rng.gaussian(seed, m * d).reshape(m, d)


def stored(mat: np.ndarray) -> np.ndarray:
    """The fp32 value the method stores, promoted back to float64 for arithmetic."""
    return np.asarray(mat, dtype=np.float32).astype(np.float64)
