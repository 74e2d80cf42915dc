"""Pins for the oracle's rounding and bit packing (CPU only)."""

import os

import numpy as np
import pytest

from oracle import numerics as nm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_rne_of_f32(a):
    # independent integer formulation of RNE fp32 -> bf16 for finite fp32 inputs
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def test_fp16_matches_numpy_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, 6e-8, 3e-8, 2.9e-8, 5.96e-8]),
    ])
    ours = nm.round_fp16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(ours, ref)


def test_fp16_ties_to_even_from_float64():
    one = 1.0
    ulp = 2.0 ** -10
    assert nm.round_fp16(one + ulp / 2) == one                 # tie -> even (1.0)
    assert nm.round_fp16(one + 3 * ulp / 2) == one + 2 * ulp   # tie -> even
    # a hair above the tie: float64 input, must not be rounded via fp32 first
    assert nm.round_fp16(one + ulp / 2 + 2.0 ** -40) == one + ulp
    assert nm.round_fp16(65520.0) == np.inf
    assert nm.round_fp16(65519.99) == 65504.0


def test_fp32_matches_numpy_cast():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(50000) * 10.0 ** rng.integers(-40, 38, 50000)
    assert np.array_equal(nm.round_fp32(x), x.astype(np.float32).astype(np.float64))


def test_bf16_matches_integer_rne_on_fp32_inputs():
    rng = np.random.default_rng(3)
    a = (rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000)).astype(np.float32)
    assert np.array_equal(nm.round_bf16(a.astype(np.float64)), _bf16_rne_of_f32(a))


def test_bf16_ties_and_bits_roundtrip():
    ulp = 2.0 ** -7
    assert nm.round_bf16(1.0 + ulp / 2) == 1.0
    assert nm.round_bf16(1.0 + ulp / 2 + 2.0 ** -30) == 1.0 + ulp
    v = np.array([1.0, -2.5, 0.0078125, 3.0e38, -1.0e-40])
    r = nm.round_bf16(v)
    assert np.array_equal(nm.bf16_from_bits(nm.bf16_bits(r)), r)


def test_bit_order_golden():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "qjl_bit_order.txt")) if not l.startswith("#")]
    for row in rows:
        byte = int(row[0], 16)
        signs = np.array([int(s) for s in row[1:]])
        bits = nm.unpack_bits_lsb(np.array([byte], dtype=np.uint8))
        assert np.array_equal(np.where(bits, 1, -1), signs)
        assert nm.pack_bits_lsb(signs > 0)[0] == byte


def test_pack_unpack_inverse():
    rng = np.random.default_rng(4)
    b = rng.integers(0, 2, size=(7, 64)).astype(bool)
    assert np.array_equal(nm.unpack_bits_lsb(nm.pack_bits_lsb(b)), b)
    with pytest.raises(ValueError):
        nm.pack_bits_lsb(np.zeros(12, dtype=bool))
