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

Block sizes that are not powers of two (glq 0.7.2 README, "Advanced / Bit widths": a
non-power-of-two size is split into power-of-two blocks, 2688 = 2048 + 512 + 128;
turbopress 0.4.2 README, "Package layout": block-diagonal Walsh-Hadamard times Rademacher
signs): d is split into the powers of two of its binary expansion, largest first, and
R = blockdiag(H_{d_1} / sqrt(d_1), H_{d_2} / sqrt(d_2), ...) . diag(D), still orthogonal.
For a power of two this is the single-block R above.
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


def block_sizes(d):
    """Powers of two of d's binary expansion, largest first (2688 -> [2048, 512, 128])."""
    if d < 1:
        raise ValueError("d must be positive")
    return [1 << b for b in range(d.bit_length() - 1, -1, -1) if (d >> b) & 1]


def block_sylvester(d):
    """blockdiag(H_{d_1}, H_{d_2}, ...) over block_sizes(d), entries +-1 or 0 (float64)."""
    H = np.zeros((d, d))
    o = 0
    for s in block_sizes(d):
        H[o:o + s, o:o + s] = sylvester(s)
        o += s
    return H


def block_weights(d):
    """sqrt(d / d_k) for every coordinate of block k: sqrt(d) R = diag(w) . H_b . diag(D)."""
    return np.concatenate([np.full(s, math.sqrt(d / s)) for s in block_sizes(d)])


def block_rotation(d, D):
    """R = blockdiag(H_{d_k} / sqrt(d_k)) . diag(D) as a dense float64 matrix."""
    return (block_weights(d)[:, None] / math.sqrt(d)) * block_sylvester(d) * np.asarray(D, dtype=np.float64)[None, :]
