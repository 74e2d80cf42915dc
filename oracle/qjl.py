"""QJL key sketch and inner-product estimators, plain float64.

Test infrastructure (see the package docstring).

eliza quantization README, QJL, "Algorithm in one paragraph": for each key k the norm ||k|| is kept,
k is multiplied by a Gaussian Johnson-Lindenstrauss matrix and only the signs
of the m sketch coordinates are kept, eight per byte.  At attention time the
query is projected through the same matrix and the score is rebuilt from the
stored signs:
        <q, k>  ~  ||k|| . sqrt(pi/2) / m . < S q, sign(S k) >,
which is unbiased with variance ((pi/2) ||q||^2 ||k||^2 - <q,k>^2) / m
(turbopress 0.4.2 README, "Findings" item 1, gives the matching noise scale
sqrt(pi/2) ||r|| ||x|| / sqrt(k)).

Readings where the pages leave a step open: S is the m x d matrix applied as S k (the
pages store it as head_dim x proj_dim and multiply k on the left of it, the
same numbers transposed); the key norm is stored as fp16; sign(0) = -1 (bit 0);
a query head h reads KV head h // (Hq / Hkv).

The two-stage estimator combines the codec and the residual sketch:
        <q, x>  ~  <q, xhat> + rnorm16 . sqrt(pi/2) / m . < S q, sign(S r) >
with xhat the dequantized block and S = G, the seeded Gaussian matrix itself, applied
to the residual r = x - xhat in the block's own coordinates (no rotation enters S).
"""

import math

import numpy as np

from .numerics import round_fp16, pack_bits_lsb, unpack_bits_lsb
from . import codec

SQRT_HALF_PI = math.sqrt(math.pi / 2.0)


def sketch(k, G):
    """keys (n, d) float64, G (m, d) -> dict(norm, norm16, p = G k, bits (n, m/8))."""
    k = np.asarray(k, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    norm = np.sqrt(np.sum(k * k, axis=1))
    p = k @ G.T
    return {"norm": norm, "norm16": round_fp16(norm), "p": p, "bits": pack_bits_lsb(p > 0)}


def estimate(bits, norm16, Sq, m):
    """Estimator from packed bits (n, m/8), fp16 norms (n,), projected queries Sq (nq, m).

    Returns (nq, n): norm16[t] * sqrt(pi/2)/m * sum_i (2 bit_ti - 1) Sq_i.
    """
    s = np.where(unpack_bits_lsb(bits, m), 1.0, -1.0)          # (n, m)
    return (np.asarray(Sq, dtype=np.float64) @ s.T) * (np.asarray(norm16, dtype=np.float64)[None, :] * SQRT_HALF_PI / m)


def estimate_scale(norm16, Sq, m):
    """L1 scale of the summed terms, norm16 * sqrt(pi/2)/m * sum_i |Sq_i|  (nq, n)."""
    a = np.sum(np.abs(np.asarray(Sq, dtype=np.float64)), axis=1)
    return a[:, None] * (np.asarray(norm16, dtype=np.float64)[None, :] * SQRT_HALF_PI / m)


def score_gqa(bits, norm16, q, G):
    """GQA scores.  bits (B, Hkv, T, m/8), norm16 (B, Hkv, T), q (B, Hq, d), G (m, d).

    Returns scores (B, Hq, T) and their L1 scales (B, Hq, T).
    """
    B, Hkv, T, mb = bits.shape
    m = mb * 8
    Hq = q.shape[1]
    group = Hq // Hkv
    G = np.asarray(G, dtype=np.float64)
    out = np.zeros((B, Hq, T))
    scale = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            Sq = np.asarray(q[b, h], dtype=np.float64)[None, :] @ G.T
            out[b, h] = estimate(bits[b, g], norm16[b, g], Sq, m)[0]
            scale[b, h] = estimate_scale(norm16[b, g], Sq, m)[0]
    return out, scale


def two_stage(codes, n16, qbits, rnorm16, q, bits, D, G):
    """Two-stage estimate of <q, x> for every (query, block).

    codes (n, d), n16 (n,), qbits (n, m/8), rnorm16 (n,), q (nq, d).
    Returns (est (nq, n), scale (nq, n)) where scale is the L1 size of the summed
    terms, sum_j |q_j xhat_j| + rnorm16 sqrt(pi/2)/m sum_i |(S q)_i|.
    """
    codes = np.asarray(codes)
    d = codes.shape[1]
    m = np.asarray(qbits).shape[1] * 8
    q = np.asarray(q, dtype=np.float64)
    xhat = codec.dequantize(codes, n16, bits, D)
    S = codec.residual_projection(d, D, G)
    Sq = q @ S.T
    first = q @ xhat.T
    second = estimate(qbits, rnorm16, Sq, m)
    scale = np.abs(q) @ np.abs(xhat).T + estimate_scale(rnorm16, Sq, m)
    return first + second, scale


def storage_ratio(head_dim, m, norm_bytes=2, elem_bytes=2):
    """Bytes of a bf16 key over bytes of its sketch: head_dim*2 / (m/8 + 2)."""
    return head_dim * elem_bytes / (m / 8 + norm_bytes)


# --- outlier channels --------------------------------------------------------------------
# eliza quantization README, QJL, "Algorithm in one paragraph": a few head_dim indices carry
# disproportionately large norms; per group of group_size consecutive tokens the top-k
# outlier channels get a sketch of their own, with its own JL projection (dim_outlier).
# qjl_apply.py, calibrate_key_outliers: the channel norms are taken over the group's tokens
# and the indices come from a top-k over them, stored as uint8.
# Readings: a trailing group shorter than group_size is a group of its own; top-k order is
# decreasing norm with ties to the lower channel; the inlier part of a key is the key with
# its group's outlier channels zeroed, the outlier part the key on those channels only
# (zero elsewhere), each sketched as a QJL key with its own matrix (S for the inliers,
# S_o for the outliers) and its own fp16 norm, and the score is the sum of the two QJL
# estimators -- q.k = q.k_in + q.k_out, each term estimated without bias.

def outlier_channels(keys, group_size, n_out):
    """keys (T, d) of one head -> (n_groups, n_out) channel indices per group."""
    keys = np.asarray(keys, dtype=np.float64)
    T, d = keys.shape
    groups = []
    for g0 in range(0, T, group_size):
        nrm = np.sqrt(np.sum(keys[g0:g0 + group_size] ** 2, axis=0))
        order = sorted(range(d), key=lambda c: (-nrm[c], c))      # decreasing norm, lower channel first
        groups.append(order[:n_out])
    return np.asarray(groups, dtype=np.int64).reshape(-1, n_out)


def outlier_mask(idx, T, d, group_size):
    """(n_groups, n_out) indices -> boolean (T, d), True on each token's outlier channels."""
    idx = np.asarray(idx, dtype=np.int64)
    mask = np.zeros((T, d), dtype=bool)
    for g in range(idx.shape[0]):
        mask[g * group_size:(g + 1) * group_size, idx[g]] = True
    return mask


def split_sketch(keys, idx, group_size, S, S_o):
    """Inlier and outlier sketches of one head's keys (T, d): dict(in=sketch(k_in, S),
    out=sketch(k_out, S_o)) with k_in + k_out = k."""
    keys = np.asarray(keys, dtype=np.float64)
    mask = outlier_mask(idx, keys.shape[0], keys.shape[1], group_size)
    k_out = np.where(mask, keys, 0.0)
    k_in = keys - k_out
    return {"in": sketch(k_in, S), "out": sketch(k_out, S_o), "k_in": k_in, "k_out": k_out}


def estimate_split(sk, q, S, S_o):
    """Scores (nq, T) of queries q (nq, d) from a split sketch: the two QJL estimators summed."""
    q = np.asarray(q, dtype=np.float64)
    m, m_o = np.asarray(S).shape[0], np.asarray(S_o).shape[0]
    a = estimate(sk["in"]["bits"], sk["in"]["norm16"], q @ np.asarray(S, dtype=np.float64).T, m)
    b = estimate(sk["out"]["bits"], sk["out"]["norm16"], q @ np.asarray(S_o, dtype=np.float64).T, m_o)
    return a + b
