"""Dense random rotation with the Beta-distribution codebook, plain float64.

Test infrastructure (see the package docstring).

eliza quantization README, TurboQuant, "Algorithm in one paragraph": the norm of each cached
vector is stored, the unit vector is rotated by a fixed random orthogonal matrix Pi drawn via a
QR decomposition with a sign fix, after which each coordinate follows the Beta-type law of one
coordinate of a uniform point on the sphere (close to N(0, 1/d) for large d); each coordinate is
bucketed against the Lloyd-Max centroids of that law, and the vector comes back as
||x|| . Pi^T c[code].

Readings where the pages leave a step open:
  * Pi = Q . diag(sign(diag(R))) for G = Q R, G the seeded d x d Gaussian matrix (the sign fix
    makes Pi Haar-distributed); the matrix is an input of the codec, like the sign mask D;
  * the law of one coordinate t of a uniform unit vector in R^d has density
        f(t) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) . (1 - t^2)^((d-3)/2),  -1 < t < 1,
    its distribution function is I_{(1+t)/2}((d-1)/2, (d-1)/2) (regularized incomplete beta)
    and int t f(t) dt = -K (1 - t^2)^((d-1)/2) / (d - 1) with K the constant above;
  * the Lloyd-Max conditions as for the Gaussian codebook: centroids are the conditional means
    of their cells, boundaries the midpoints of neighbouring centroids, iterated to a fixed point;
  * the norm is stored as fp16 (as the rest of the codec; the page names bf16), codes are
    decided in float64 against the float64 boundaries, ties to the lower code.
"""

import functools
import math

import numpy as np
from scipy import special

from .numerics import round_fp16


def haar_rotation(G):
    """Pi = Q diag(sign(diag(R))) from the QR decomposition of the d x d matrix G."""
    Q, R = np.linalg.qr(np.asarray(G, dtype=np.float64))
    s = np.sign(np.diag(R))
    s[s == 0] = 1.0
    return Q * s[None, :]


def _const(d):
    return math.exp(math.lgamma(d / 2.0) - math.lgamma((d - 1) / 2.0)) / math.sqrt(math.pi)


def beta_density(t, d):
    t = np.asarray(t, dtype=np.float64)
    return _const(d) * np.power(np.clip(1.0 - t * t, 0.0, None), (d - 3) / 2.0)


def beta_cdf(t, d):
    a = (d - 1) / 2.0
    return special.betainc(a, a, (1.0 + np.clip(np.asarray(t, dtype=np.float64), -1.0, 1.0)) / 2.0)


def _moment(t, d):
    """Antiderivative of t f(t): -K (1 - t^2)^((d-1)/2) / (d - 1)."""
    t = np.clip(np.asarray(t, dtype=np.float64), -1.0, 1.0)
    return -_const(d) * np.power(1.0 - t * t, (d - 1) / 2.0) / (d - 1)


@functools.lru_cache(maxsize=None)
def beta_codebook(bits, d, tol=1e-13, max_iter=200000):
    """Lloyd-Max quantizer of one sphere coordinate in R^d at `bits` bits.

    Returns (centroids (2^b,), boundaries (2^b - 1,), mse) on the coordinate's own scale."""
    L = 1 << bits
    # start from equal-mass cells
    qs = (np.arange(1, L) / L)
    lo, hi = -1.0, 1.0
    beta = np.empty(L - 1)
    for i, q in enumerate(qs):                          # bisection on the distribution function
        a, b = lo, hi
        for _ in range(200):
            mid = 0.5 * (a + b)
            if beta_cdf(mid, d) < q:
                a = mid
            else:
                b = mid
        beta[i] = 0.5 * (a + b)
    for _ in range(max_iter):
        edges = np.concatenate([[-1.0], beta, [1.0]])
        mass = beta_cdf(edges[1:], d) - beta_cdf(edges[:-1], d)
        mom = _moment(edges[1:], d) - _moment(edges[:-1], d)
        c = mom / mass
        nb = 0.5 * (c[1:] + c[:-1])
        if np.max(np.abs(nb - beta)) < tol:
            beta = nb
            break
        beta = nb
    # the law is symmetric, so the fixed point is antisymmetric: impose it exactly (the middle
    # boundary of an odd count is then exactly 0, as for the Gaussian codebook)
    beta = 0.5 * (beta - beta[::-1])
    edges = np.concatenate([[-1.0], beta, [1.0]])
    mass = beta_cdf(edges[1:], d) - beta_cdf(edges[:-1], d)
    mom = _moment(edges[1:], d) - _moment(edges[:-1], d)
    c = mom / mass
    c = 0.5 * (c - c[::-1])
    # E[t^2] = 1/d; MSE = E[t^2] - sum_k mass_k c_k^2 for the conditional-mean centroids
    mse = 1.0 / d - float(np.sum(mass * c * c))
    return c, beta, mse


def quantize(x, bits, Pi):
    """Blocks x (n, d) -> dict(norm, n16, y = Pi u (n, d), codes uint8)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[1]
    c, beta, _ = beta_codebook(bits, d)
    norm = np.sqrt(np.sum(x * x, axis=1))
    safe = np.where(norm > 0, norm, 1.0)
    y = np.where(norm[:, None] > 0, (x @ np.asarray(Pi, dtype=np.float64).T) / safe[:, None], 0.0)
    codes = np.zeros(y.shape, dtype=np.int64)
    for bj in beta:
        codes += (y > bj)
    return {"norm": norm, "n16": round_fp16(norm), "y": y, "codes": codes.astype(np.uint8), "beta": beta}


def dequantize(codes, n16, bits, Pi):
    """xhat = n16 . Pi^T c[code] for every block (n, d)."""
    codes = np.asarray(codes)
    d = codes.shape[1]
    c, _, _ = beta_codebook(bits, d)
    return np.asarray(n16, dtype=np.float64)[:, None] * (c[codes.astype(np.int64)] @ np.asarray(Pi, dtype=np.float64))
