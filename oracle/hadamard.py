"""Sylvester Walsh-Hadamard matrix and the randomized Hadamard rotation, float64.

Test infrastructure (see the package docstring).

glq 0.7.2 README, "How it works" item 2: the randomized Hadamard transform is random
sign flips followed by the fast Walsh-Hadamard transform.  turbopress 0.4.2 README,
"Package layout" (hadamard.py): the seeded orthogonal transform R is the
Walsh-Hadamard transform times Rademacher signs, and (W R^T)(R x) = W x.

Reading used here: H is the Sylvester (natural-order) matrix
H[i, j] = (-1)^popcount(i AND j), which satisfies H H^T = d I, and
R = H . diag(D) / sqrt(d) with D the +-1 sign vector (signs applied first).
The oracle applies H as a dense matrix: the fast transform is only a faster
way of computing the same product.
"""

import math

import numpy as np


def sylvester(d):
    """Dense d x d Sylvester Hadamard matrix, entries +-1 (float64)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d, dtype=np.int64)
    anded = i[:, None] & i[None, :]
    parity = np.zeros_like(anded)
    v = anded.copy()
    while np.any(v):
        parity ^= v & 1
        v >>= 1
    return np.where(parity == 1, -1.0, 1.0)


def signs_from_mask(mask, d):
    """d/8-byte LSB-first mask -> +-1 float64 vector; bit j set means D_j = -1."""
    mask = np.asarray(mask, dtype=np.uint8)
    if mask.size * 8 != d:
        raise ValueError("mask must hold exactly d bits")
    bits = (mask[:, None] >> np.arange(8, dtype=np.uint8)) & 1
    return np.where(bits.reshape(d) == 1, -1.0, 1.0)


def rotation(d, D):
    """R = H . diag(D) / sqrt(d) as a dense float64 matrix."""
    H = sylvester(d)
    return H * np.asarray(D, dtype=np.float64)[None, :] / math.sqrt(d)
