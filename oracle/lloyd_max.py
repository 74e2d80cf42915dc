"""Lloyd-Max optimal scalar quantizer for the standard normal, in float64.

Test infrastructure (see the package docstring).

eliza quantization README, PolarQuant, "Algorithm in one paragraph": after the rotation each
coordinate is quantized against the Lloyd-Max optimal centroids for N(0,1),
precomputed with the iterative conditional-expectation algorithm.  The
turbopress 0.4.2 README ("Package layout", codebooks.py) computes the same codebooks to
a fixed point in float64.

The two Lloyd conditions, iterated until nothing moves:
  * boundaries are midpoints of adjacent centroids,
        beta_k = (c_k + c_{k+1}) / 2;
  * centroids are the conditional means of N(0,1) on their cells,
        c_k = (phi(beta_{k-1}) - phi(beta_k)) / (Phi(beta_k) - Phi(beta_{k-1})),
    with beta_{-1} = -inf and beta_{L-1} = +inf.
The distortion of the fixed point is E[(X - Q(X))^2] = 1 - sum_k p_k c_k^2 with
p_k = Phi(beta_k) - Phi(beta_{k-1}) (the centroid condition makes the cross
term vanish).
"""

import math
from functools import lru_cache

import numpy as np

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def phi(x):
    """Standard normal density."""
    x = np.asarray(x, dtype=np.float64)
    return _INV_SQRT_2PI * np.exp(-0.5 * x * x)


def Phi(x):
    """Standard normal CDF, via erfc so that both tails keep full relative accuracy."""
    x = np.asarray(x, dtype=np.float64)
    from scipy.special import erfc
    return 0.5 * erfc(-x / _SQRT2)


def _cell_masses_and_means(boundaries):
    edges = np.concatenate(([-np.inf], boundaries, [np.inf]))
    lo, hi = edges[:-1], edges[1:]
    # mass of each cell; the upper tail is computed as Phi(-lo) - Phi(-hi) for
    # cells on the positive side so that small differences are not lost
    mass = np.where(lo >= 0, Phi(-lo) - Phi(-hi), Phi(hi) - Phi(lo))
    num = phi(lo) - phi(hi)
    return mass, num / mass


@lru_cache(maxsize=None)
def codebook(bits, tol=1e-13, max_iter=2_000_000):
    """Return (centroids[2^b], boundaries[2^b - 1], mse) as float64 arrays.

    Starts from centroids at the midpoints of equal-probability cells and
    alternates the two Lloyd conditions until the largest centroid move is
    below ``tol`` (the float64 tail masses put a noise floor near 1e-14 on
    the move for 6-8 bits, so the default stops just above it).
    """
    if not 1 <= bits <= 8:
        raise ValueError("bits must be in 1..8")
    L = 1 << bits
    from scipy.special import ndtri
    q = (np.arange(L, dtype=np.float64) + 0.5) / L
    c = ndtri(q)
    for _ in range(max_iter):
        beta = 0.5 * (c[:-1] + c[1:])
        _, c_new = _cell_masses_and_means(beta)
        step = np.max(np.abs(c_new - c))
        c = c_new
        if step < tol:
            break
    else:
        raise RuntimeError("Lloyd-Max iteration did not converge")
    # the N(0,1) fixed point is symmetric; remove the last rounding asymmetry
    c = 0.5 * (c - c[::-1])
    beta = 0.5 * (c[:-1] + c[1:])
    mass, _ = _cell_masses_and_means(beta)
    mse = 1.0 - float(np.sum(mass * c * c))
    c.setflags(write=False)
    beta.setflags(write=False)
    return c, beta, mse
