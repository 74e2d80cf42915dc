"""IEEE-754 rounding and bit packing, written out in float64 / integer numpy.

Test infrastructure (see the package docstring).

* Norms are stored as fp16 (eliza quantization README, PolarQuant, "Algorithm in one paragraph":
  the block L2 norm is stored as fp16).
* bf16 is the dtype of the weights / keys and of the dequantized output.
* QJL sign bits are packed eight per byte, least significant bit first, and
  bit value 1 means sign +1 (qjl_apply.py, ``_qjl_decode_keys``: the byte is
  shifted right by 0..7 and masked with 1, then mapped to 2*bit - 1).
"""

import numpy as np


def _round_to_format(x, mant_bits, emin, emax):
    """Round float64 values to the nearest value of a binary format, ties to even.

    The format has ``mant_bits`` fraction bits, normal exponents in
    [emin, emax] and gradual underflow.  Values beyond the largest finite
    number after rounding become +-inf.  NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    a = np.abs(xf)
    # exponent e with 2**e <= a < 2**(e+1)
    _, e2 = np.frexp(a)          # a = f * 2**e2, 0.5 <= f < 1
    e = e2.astype(np.int64) - 1
    e = np.maximum(e, emin)      # below the normal range the quantum is fixed
    quantum_exp = e - mant_bits
    scaled = np.ldexp(a, -quantum_exp)          # exact (power-of-two scaling)
    r = np.rint(scaled)                          # numpy rint: ties to even
    rounded = np.ldexp(r, quantum_exp)
    max_finite = np.ldexp(2.0 - 2.0 ** (-mant_bits), emax)
    rounded = np.where(rounded > max_finite, np.inf, rounded)
    out[finite] = np.copysign(rounded, xf)
    return out


def round_fp16(x):
    """float64 -> nearest fp16 value (as float64), IEEE RNE, overflow to inf."""
    return _round_to_format(x, mant_bits=10, emin=-14, emax=15)


def round_bf16(x):
    """float64 -> nearest bf16 value (as float64), IEEE RNE, overflow to inf."""
    return _round_to_format(x, mant_bits=7, emin=-126, emax=127)


def round_fp32(x):
    """float64 -> nearest fp32 value (as float64), IEEE RNE, overflow to inf."""
    return _round_to_format(x, mant_bits=23, emin=-126, emax=127)


def fp16_bits(x):
    """fp16-representable float64 values -> their uint16 bit patterns."""
    return np.asarray(round_fp16(x)).astype(np.float16).view(np.uint16)


def fp16_from_bits(u):
    """uint16 fp16 bit patterns -> float64."""
    return np.asarray(u, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits(x):
    """bf16-representable float64 values -> their uint16 bit patterns."""
    v = np.asarray(round_bf16(x)).astype(np.float32)   # exact: bf16 is a subset of fp32
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(u):
    """uint16 bf16 bit patterns -> float64 (exact)."""
    u32 = np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def pack_bits_lsb(bits):
    """Boolean array [..., m] -> uint8 [..., m/8]; bit j of byte k is element 8k+j."""
    bits = np.asarray(bits, dtype=bool)
    m = bits.shape[-1]
    if m % 8:
        raise ValueError("bit count must be a multiple of 8")
    b = bits.reshape(bits.shape[:-1] + (m // 8, 8)).astype(np.uint8)
    weights = (1 << np.arange(8)).astype(np.uint8)
    return (b * weights).sum(axis=-1).astype(np.uint8)


def unpack_bits_lsb(packed, m=None):
    """uint8 [..., m/8] -> bool [..., m], the inverse of ``pack_bits_lsb``."""
    packed = np.asarray(packed, dtype=np.uint8)
    shifts = np.arange(8, dtype=np.uint8)
    bits = (packed[..., :, None] >> shifts) & 1
    bits = bits.reshape(packed.shape[:-1] + (packed.shape[-1] * 8,)).astype(bool)
    if m is not None:
        bits = bits[..., :m]
    return bits
