"""The seeded random quantities of the codec -- the rotation signs D and the Gaussian JL
matrix G -- rebuilt from a 64-bit seed, plain Python / numpy.

Test infrastructure (see the package docstring).

The pages make the seed the persisted state: eliza quantization README, TurboQuant, "CLI"
(``--base-seed``: layer i uses seed base_seed + i, and dequantizing with other signs gives
garbage) and QJL, "CLI" (``--projection-seed``); qjl_apply.py draws the JL matrix from a
seeded generator per layer.  The pages' generator is torch's Mersenne-Twister stream; the
reading taken here freezes a counter-based generator instead, so that a C library and this
oracle can each rebuild the same bytes from the seed alone:

  * SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
    OOPSLA 2014; the 64-bit finaliser constants of Vigna's public-domain splitmix64.c):
        mix(z) = z3 ^ (z3 >> 31), z3 = (z2 ^ (z2 >> 27)) * 0x94D049BB133111EB,
                 z2 = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9            (all mod 2^64)
    and the generator started in state s returns mix(s + (i + 1) * 0x9E3779B97F4A7C15) as its
    output i = 0, 1, 2, ...;
  * stream (seed, tag) starts in state s = mix(seed XOR tag), with tag 0x5349474E for the
    signs and 0x50524F4A for the projection;
  * signs: D_j = -1 exactly when the top bit of output j is set; the mask holds D_j as bit
    j % 8 of byte j // 8 (set means -1), the layout of the library's sign masks;
  * projection: element k = i d + j of the m x d row-major matrix; the pair (2p, 2p + 1) takes
    outputs 2p and 2p + 1 as uniforms u = ((out >> 11) + 0.5) 2^-53 in (0, 1) and the
    Box-Muller transform (Box and Muller, Ann. Math. Statist. 1958) in float64:
        G[2p] = sqrt(-2 ln u1) cos(2 pi u2),  G[2p + 1] = sqrt(-2 ln u1) sin(2 pi u2),
    each then rounded to the nearest bf16 (ties to even), stored as bf16 bit patterns.
"""

import math

import numpy as np

from .numerics import round_bf16, bf16_bits

GAMMA = 0x9E3779B97F4A7C15
TAG_SIGNS = 0x5349474E
TAG_PROJ = 0x50524F4A
_M64 = (1 << 64) - 1


def mix64(z):
    """The SplitMix64 output function of one 64-bit integer (Python int arithmetic mod 2^64)."""
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def splitmix64(state, n):
    """The first n outputs of SplitMix64 started in `state` (list of Python ints)."""
    out = []
    for _ in range(n):
        state = (state + GAMMA) & _M64
        out.append(mix64(state))
    return out


def stream(seed, tag, n):
    """Outputs 0 .. n-1 of stream (seed, tag)."""
    return splitmix64(mix64((int(seed) & _M64) ^ tag), n)


def sign_mask(seed, d):
    """d/8-byte mask (uint8), bit j % 8 of byte j // 8 set exactly when D_j = -1."""
    if d % 8:
        raise ValueError("d must be a multiple of 8")
    mask = np.zeros(d // 8, dtype=np.uint8)
    for j, v in enumerate(stream(seed, TAG_SIGNS, d)):
        if v >> 63:
            mask[j >> 3] |= np.uint8(1 << (j & 7))
    return mask


def signs(seed, d):
    """The +-1 vector D (float64) of `sign_mask`."""
    m = sign_mask(seed, d)
    return np.array([-1.0 if (m[j >> 3] >> (j & 7)) & 1 else 1.0 for j in range(d)])


def gaussian(seed, n):
    """n float64 N(0,1) values of the projection stream (Box-Muller over output pairs)."""
    if n % 2:
        raise ValueError("n must be even")
    raw = stream(seed, TAG_PROJ, n)
    out = np.empty(n)
    for p in range(n // 2):
        u1 = ((raw[2 * p] >> 11) + 0.5) * 2.0 ** -53
        u2 = ((raw[2 * p + 1] >> 11) + 0.5) * 2.0 ** -53
        rad = math.sqrt(-2.0 * math.log(u1))
        out[2 * p] = rad * math.cos(2.0 * math.pi * u2)
        out[2 * p + 1] = rad * math.sin(2.0 * math.pi * u2)
    return out


def projection(seed, m, d):
    """G, m x d row-major, as bf16 bit patterns (uint16)."""
    return bf16_bits(round_bf16(gaussian(seed, m * d))).reshape(m, d)


def projection_values(seed, m, d):
    """G as float64 values (exactly the bf16 values of `projection`)."""
    return round_bf16(gaussian(seed, m * d)).reshape(m, d)
