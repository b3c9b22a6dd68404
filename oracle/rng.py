"""Counter-based random streams the method draws from (oracle copy).

The pages say the rotation is a random Haar orthogonal matrix, the QJL matrix S
is random, and the Walsh-Hadamard variant uses a random sign vector
("FlashQuant" page, sections "TurboQuant" step 2 and "QJL"; "TurboQuant"
blog, "Couche 1"), but fix no generator. To let the library's own builder and
this oracle draw the same numbers without sharing code, both implement the same
published generators independently:

* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): output i of stream ``seed`` is
  mix64(seed + (i + 1) * 0x9E3779B97F4A7C15) with the variant-13 finaliser
  (shifts 30/27/31, multipliers 0xBF58476D1CE4E5B9, 0x94D049BB133111EB).
* uniform(i) = ((out_i >> 11) + 0.5) * 2**-53, which lies in (0, 1).
* Box & Muller (1958): pair p uses u1 = uniform(2p), u2 = uniform(2p+1);
  r = sqrt(-2 ln u1); g[2p] = r cos(2 pi u2), g[2p+1] = r sin(2 pi u2).
* sign(j) = -1 if the top bit of out_j is set, else +1.

Pure-Python scalar math (``math.log`` etc.) is used so the values are the C
library's, like the builder's.
"""
import math

import numpy as np

_MASK = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed: int, i: int) -> int:
    """Output ``i`` (0-based) of the SplitMix64 stream that starts at ``seed``."""
    z = (seed + (i + 1) * _GAMMA) & _MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def uniform(seed: int, i: int) -> float:
    """The i-th uniform in (0, 1) of the stream: 53 top bits plus one half ulp."""
    return ((splitmix64(seed, i) >> 11) + 0.5) * (2.0 ** -53)


def gaussian(seed: int, n: int) -> np.ndarray:
    """n standard normals (float64) by Box-Muller, both outputs of each pair used."""
    out = np.empty(n, dtype=np.float64)
    for p in range((n + 1) // 2):
        u1 = uniform(seed, 2 * p)
        u2 = uniform(seed, 2 * p + 1)
        r = math.sqrt(-2.0 * math.log(u1))
        out[2 * p] = r * math.cos(2.0 * math.pi * u2)
        if 2 * p + 1 < n:
            out[2 * p + 1] = r * math.sin(2.0 * math.pi * u2)
    return out


def signs(seed: int, n: int) -> np.ndarray:
    """n random signs (+1.0 / -1.0) from the top bit of each stream output."""
    return np.array([-1.0 if (splitmix64(seed, j) >> 63) else 1.0 for j in range(n)])
