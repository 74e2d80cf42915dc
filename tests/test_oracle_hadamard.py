"""Pins for the oracle's Hadamard matrix and randomized rotation (CPU only)."""

import math

import numpy as np
import pytest

from oracle import hadamard


def _kron_sylvester(d):
    H = np.array([[1.0]])
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


def _fwht_butterfly(v):
    # the in-place radix-2 butterfly the pages name ("butterfly operations")
    v = np.array(v, dtype=np.float64, copy=True)
    d = v.shape[-1]
    h = 1
    while h < d:
        v = v.reshape(v.shape[:-1] + (d // (2 * h), 2, h))
        a, b = v[..., 0, :].copy(), v[..., 1, :].copy()
        v[..., 0, :], v[..., 1, :] = a + b, a - b
        v = v.reshape(v.shape[:-3] + (d,))
        h *= 2
    return v


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 64, 128, 256, 512])
def test_orthogonality_exact(d):
    H = hadamard.sylvester(d)
    assert np.array_equal(H @ H.T, d * np.eye(d))
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H, d * np.eye(d))


@pytest.mark.parametrize("d", [2, 4, 8, 32, 128, 512])
def test_popcount_definition_equals_kronecker_recursion(d):
    assert np.array_equal(hadamard.sylvester(d), _kron_sylvester(d))


@pytest.mark.parametrize("d", [4, 8, 64, 128, 256, 512])
def test_dense_equals_fast_butterfly(d):
    x = np.random.default_rng(d).standard_normal((5, d))
    assert np.allclose(x @ hadamard.sylvester(d).T, _fwht_butterfly(x), atol=1e-12, rtol=0)


def test_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        hadamard.sylvester(96)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotation_is_orthogonal_and_preserves_norm(d):
    rng = np.random.default_rng(7)
    D = rng.choice([-1.0, 1.0], size=d)
    R = hadamard.rotation(d, D)
    assert np.allclose(R @ R.T, np.eye(d), atol=1e-13)
    x = rng.standard_normal((10, d))
    assert np.allclose(np.linalg.norm(x @ R.T, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    # turbopress 0.4.2 README, "Package layout": (W R^T)(R x) = W x
    W = rng.standard_normal((3, d))
    assert np.allclose((W @ R.T) @ (R @ x.T), W @ x.T, atol=1e-11)


def test_signs_from_mask_lsb_first():
    mask = np.array([0b00000101, 0x80], dtype=np.uint8)
    D = hadamard.signs_from_mask(mask, 16)
    expect = np.ones(16)
    expect[[0, 2, 15]] = -1
    assert np.array_equal(D, expect)
    with pytest.raises(ValueError):
        hadamard.signs_from_mask(mask, 8)


def test_rotated_gaussian_coordinates_are_standard_normal():
    # eliza quantization README, PolarQuant: after the rotation the coordinates of a
    # unit block are ~N(0, 1/d); scaled by sqrt(d) they are ~N(0, 1).
    d = 128
    rng = np.random.default_rng(11)
    D = rng.choice([-1.0, 1.0], size=d)
    x = rng.standard_normal((4000, d)) * np.exp(rng.standard_normal(d))   # uneven channel scales
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    y = math.sqrt(d) * (u @ hadamard.rotation(d, D).T)
    assert abs(np.mean(y)) < 0.01
    assert abs(np.var(y) - 1.0) < 0.01


# ---- block-diagonal rotation for sizes that are not powers of two ----------------------------

def test_block_sizes_page_example():
    """glq 0.7.2 README, "Advanced / Bit widths": 2688 is split as 2048 + 512 + 128."""
    assert hadamard.block_sizes(2688) == [2048, 512, 128]


@pytest.mark.parametrize("d", [1, 3, 96, 192, 320, 448, 576, 1000, 1024])
def test_block_sizes_binary_expansion(d):
    s = hadamard.block_sizes(d)
    assert sum(s) == d and s == sorted(s, reverse=True) and len(set(s)) == len(s)
    assert all(b & (b - 1) == 0 for b in s)
    if d & (d - 1) == 0:
        assert s == [d]


@pytest.mark.parametrize("d", [64, 256])
def test_block_sylvester_is_sylvester_for_powers_of_two(d):
    assert np.array_equal(hadamard.block_sylvester(d), hadamard.sylvester(d))
    assert np.all(hadamard.block_weights(d) == 1.0)


@pytest.mark.parametrize("d", [3, 96, 192, 320, 576])
def test_block_rotation_orthogonal_and_per_block(d):
    rng = np.random.default_rng(d)
    D = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    R = hadamard.block_rotation(d, D)
    np.testing.assert_allclose(R @ R.T, np.eye(d), atol=1e-12)
    # built slice by slice from the power-of-two rotation of each block
    x = rng.standard_normal(d)
    o = 0
    for s in hadamard.block_sizes(d):
        ref = hadamard.rotation(s, D[o:o + s]) @ x[o:o + s]
        np.testing.assert_allclose((R @ x)[o:o + s], ref, atol=1e-12)
        o += s
