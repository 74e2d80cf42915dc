"""Block quantize / dequantize and the QJL residual stage, plain float64.

Test infrastructure (see the package docstring).

eliza quantization README, PolarQuant, "Algorithm in one paragraph", step by step for one block x
of d = 2^k values:
  1. the L2 norm n = ||x|| is taken and stored as fp16 (n16);
  2. the block is normalised to the unit sphere, u = x / n;
  3. it is rotated by the randomized Walsh-Hadamard transform and scaled by
     sqrt(d), so each coordinate is close to N(0, 1):
        y = sqrt(d) . R u = H (D * u) = H (D * x) / n,   R = H . diag(D) / sqrt(d);
  4. each coordinate takes the index of its nearest Lloyd-Max N(0,1) centroid,
     stored as a byte: code_i = #{ j : y_i > beta_j } (beta ascending);
  5. (optional) a 1-bit QJL sketch of the residual is appended.
Dequantize undoes the steps: centroid lookup, divide by sqrt(d), inverse
rotation, multiply by the stored norm:
        xhat = n16 . R^T c[code] / sqrt(d) = (n16 / d) . D * (H c[code]).
For a d that is not a power of two R is block diagonal (see ``hadamard``):
sqrt(d) R = diag(w) H_b diag(D) with H_b = blockdiag(H_{d_k}) and w = sqrt(d / d_k) on
block k, so y = w * H_b (D * x) / n and xhat = (n16 / d) . D * (H_b (w * c[code])).

Readings where the pages leave a step open:
  * normalisation uses the unrounded norm n; dequantize and the residual use n16;
  * a zero block has u = 0, hence y = 0 and code 2^(b-1) - 1, n16 = 0;
  * ties y_i == beta_j take the lower code (strict >);
  * the code decision is taken in float64: the float64 y_i is compared with the
    float64 boundaries beta_j.  ``boundary_distance`` gives the float64 distance
    to the nearest boundary and the code on its far side for the parity rule;
  * QJL residual: r = x - xhat in the block's own coordinates, rnorm16 =
    fp16(||r||), bits = [S r > 0] packed LSB-first, where S is the seeded
    m x d Gaussian matrix itself (stored as bf16 values), applied to r without
    any rotation.
"""

import math

import numpy as np

from . import lloyd_max
from .hadamard import block_sylvester, block_weights
from .numerics import round_fp16, pack_bits_lsb

BAND = 1e-4   # coordinates this close to a boundary may take either side (parity rule)


def block_view(x, d):
    """Flat or 2-D array -> (n_blocks, d) float64 view of consecutive d-element runs."""
    x = np.asarray(x, dtype=np.float64)
    if x.size % d:
        raise ValueError("size must be a multiple of d")
    return x.reshape(-1, d)


def quantize(x, bits, D):
    """Steps 1-4 for every block.  x: (n, d) float64; D: +-1 vector of length d.

    Returns a dict with
      norm   (n,)    float64 unrounded block norms
      n16    (n,)    float64 values of the fp16 norms
      y      (n, d)  float64 rotated, normalised, sqrt(d)-scaled coordinates
      codes  (n, d)  uint8 centroid indices
    """
    x = np.asarray(x, dtype=np.float64)
    n_blocks, d = x.shape
    centroids, beta, _ = lloyd_max.codebook(bits)
    norm = np.sqrt(np.sum(x * x, axis=1))
    n16 = round_fp16(norm)
    safe = np.where(norm > 0, norm, 1.0)
    H = block_sylvester(d)             # sylvester(d) when d is a power of two
    # the rotation is linear, so H (D * x) / n equals H (D * u); rotating the exact
    # input first keeps coordinates that are exactly zero (ties at the middle
    # boundary of a structured block) exactly zero instead of +-1e-17
    z = (x * np.asarray(D, dtype=np.float64)[None, :]) @ H.T
    w = block_weights(d)               # all ones when d is a power of two
    if np.any(w != 1.0):
        z = z * w[None, :]
    y = np.where(norm[:, None] > 0, z / safe[:, None], 0.0)
    codes = np.zeros(y.shape, dtype=np.int64)
    for bj in beta:                        # count the boundaries below each coordinate
        codes += (y > bj)
    return {"norm": norm, "n16": n16, "y": y, "codes": codes.astype(np.uint8)}


def boundary_distance(y, bits):
    """float64 distance from each coordinate to its nearest decision boundary,
    and the code on the far side of that boundary."""
    _, beta, _ = lloyd_max.codebook(bits)
    y = np.asarray(y, dtype=np.float64)
    # nearest boundary: one of the two neighbours of y's position in the sorted list
    pos = np.searchsorted(beta, y)
    lo = np.clip(pos - 1, 0, len(beta) - 1)
    hi = np.clip(pos, 0, len(beta) - 1)
    d_lo, d_hi = np.abs(y - beta[lo]), np.abs(y - beta[hi])
    j = np.where(d_lo <= d_hi, lo, hi)
    dist = np.minimum(d_lo, d_hi)
    below = y <= beta[j]                  # code j on the lower side, j+1 above
    other = np.where(below, j + 1, j)
    return dist, other.astype(np.uint8)


def dequantize(codes, n16, bits, D):
    """xhat = (n16 / d) . D * (H c[code]) for every block, float64 (n, d)."""
    codes = np.asarray(codes)
    d = codes.shape[1]
    centroids, _, _ = lloyd_max.codebook(bits)
    c = centroids[codes.astype(np.int64)]
    H = block_sylvester(d)             # sylvester(d) when d is a power of two
    w = block_weights(d)               # all ones when d is a power of two
    if np.any(w != 1.0):
        c = c * w[None, :]
    return (np.asarray(n16, dtype=np.float64)[:, None] / d) * (c @ H.T) * np.asarray(D, dtype=np.float64)[None, :]


def residual_projection(d, D, G):
    """S, the m x d Gaussian projection the QJL stage applies to r: the seeded
    matrix G as given (d and D are accepted for symmetry with the codec calls
    and do not enter S)."""
    G = np.asarray(G, dtype=np.float64)
    assert G.shape[1] == d
    return G


def qjl_residual(x, codes, n16, bits, D, G):
    """Step 5: the QJL sketch of the quantization residual.

    Returns a dict with r (n, d), rnorm (n,), rnorm16 (n,), p = S r (n, m) and
    the packed sign bits (n, m/8) uint8.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[1]
    xhat = dequantize(codes, n16, bits, D)
    r = x - xhat
    rnorm = np.sqrt(np.sum(r * r, axis=1))
    S = residual_projection(d, D, G)
    p = r @ S.T
    return {"r": r, "rnorm": rnorm, "rnorm16": round_fp16(rnorm), "p": p,
            "bits": pack_bits_lsb(p > 0)}


def pack_codes(codes, bits):
    """Codes [n, d] (each below 2^bits) -> packed bytes [n, d * bits / 8].

    eliza quantization README, TurboQuant, "Algorithm in one paragraph", step 4: the indices
    are bit-packed into bytes, two per byte at 4 bits and four per byte at 2 bits.  Reading
    (the pages fix the density, not the order): each block is a little-endian bit stream,
    bit j of code i is stream bit bits * i + j, and stream bit p is bit p mod 8 of byte
    p div 8 -- at 4 bits code 2k is the low nibble of byte k, as for the QJL sign bits the
    first element takes the least significant bit."""
    codes = np.asarray(codes, dtype=np.int64)
    n, d = codes.shape
    if (d * bits) % 8:
        raise ValueError("d * bits must be a multiple of 8")
    if codes.size and (codes.min() < 0 or codes.max() >= (1 << bits)):
        raise ValueError("code out of range")
    out = np.zeros((n, d * bits // 8), dtype=np.uint8)
    for i in range(d):
        for j in range(bits):
            p = bits * i + j
            out[:, p // 8] |= (((codes[:, i] >> j) & 1) << (p % 8)).astype(np.uint8)
    return out


def unpack_codes(packed, bits, d):
    """Inverse of ``pack_codes``: packed bytes [n, d * bits / 8] -> codes [n, d] (uint8)."""
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    codes = np.zeros((n, d), dtype=np.int64)
    for i in range(d):
        for j in range(bits):
            p = bits * i + j
            codes[:, i] |= ((packed[:, p // 8].astype(np.int64) >> (p % 8)) & 1) << j
    return codes.astype(np.uint8)


def storage_bytes_per_block(d, bits_per_code_byte=8, m=0):
    """Bytes the codec stores per block: d code bytes + fp16 norm, plus m/8 sign
    bytes + fp16 residual norm when the QJL stage is on."""
    b = d * bits_per_code_byte // 8 + 2
    if m:
        b += m // 8 + 2
    return b


def mse_per_coordinate(x, codes, n16, bits, D):
    """Relative reconstruction error ||x - xhat||^2 / ||x||^2 per block."""
    xhat = dequantize(codes, n16, bits, D)
    num = np.sum((np.asarray(x, dtype=np.float64) - xhat) ** 2, axis=1)
    den = np.sum(np.asarray(x, dtype=np.float64) ** 2, axis=1)
    return num / den


SQRT_HALF_PI = math.sqrt(math.pi / 2.0)
