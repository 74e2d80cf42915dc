"""Pins for the oracle's dense rotation and Beta-distribution codebook (CPU only).

Closed forms (d = 3: the coordinate is uniform on [-1, 1], whose Lloyd-Max quantizer is the
uniform one), the large-d limit (sqrt(d) times the codebook tends to the N(0,1) codebook),
conditional means by direct numerical integration, orthogonality of the rotation and the
codec's identities."""

import math

import numpy as np
import pytest

from oracle import dense, lloyd_max


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_d3_is_the_uniform_quantizer(bits):
    L = 1 << bits
    c, beta, mse = dense.beta_codebook(bits, 3)
    np.testing.assert_allclose(c, -1.0 + (2.0 * np.arange(L) + 1.0) / L, atol=1e-10)
    np.testing.assert_allclose(beta, -1.0 + 2.0 * np.arange(1, L) / L, atol=1e-10)
    np.testing.assert_allclose(mse, (2.0 / L) ** 2 / 12.0, rtol=1e-8)


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_large_d_tends_to_the_gaussian_codebook(bits):
    d = 8192
    c, beta, mse = dense.beta_codebook(bits, d)
    g, gb, gmse = lloyd_max.codebook(bits)
    np.testing.assert_allclose(math.sqrt(d) * c, g, rtol=2e-3, atol=2e-3)
    np.testing.assert_allclose(d * mse, gmse, rtol=5e-3)


@pytest.mark.parametrize("d,bits", [(64, 3), (128, 2), (16, 4)])
def test_centroids_are_conditional_means_by_integration(d, bits):
    c, beta, mse = dense.beta_codebook(bits, d)
    assert np.all(np.diff(c) > 0) and np.allclose(c, -c[::-1], atol=1e-12)
    np.testing.assert_allclose(beta, 0.5 * (c[1:] + c[:-1]), atol=1e-12)
    t = np.linspace(-1.0, 1.0, 2_000_001)
    f = dense.beta_density(t, d)
    assert abs(np.trapezoid(f, t) - 1.0) < 1e-9
    edges = np.concatenate([[-1.0], beta, [1.0]])
    for k in range(len(c)):
        sel = (t >= edges[k]) & (t <= edges[k + 1])
        m = np.trapezoid(f[sel], t[sel])
        assert abs(np.trapezoid(t[sel] * f[sel], t[sel]) / m - c[k]) < 1e-6
    # distortion by integration
    idx = np.searchsorted(beta, t)
    assert abs(np.trapezoid((t - c[idx]) ** 2 * f, t) - mse) < 1e-8


def test_haar_rotation_orthogonal_with_sign_fix():
    rng = np.random.default_rng(0)
    G = rng.standard_normal((32, 32))
    Pi = dense.haar_rotation(G)
    np.testing.assert_allclose(Pi @ Pi.T, np.eye(32), atol=1e-12)
    Q, R = np.linalg.qr(G)
    np.testing.assert_allclose(np.abs(Pi), np.abs(Q), atol=1e-12)
    # Pi^T G is upper triangular with a positive diagonal
    U = Pi.T @ G
    assert np.all(np.diag(U) > 0) and np.allclose(np.tril(U, -1), 0.0, atol=1e-10)


def test_codec_identities():
    d, bits = 64, 3
    rng = np.random.default_rng(1)
    Pi = dense.haar_rotation(rng.standard_normal((d, d)))
    x = rng.standard_normal((2000, d)) * np.exp(rng.standard_normal((2000, 1)))
    x[0] = 0.0
    q = dense.quantize(x, bits, Pi)
    assert np.all(q["codes"][0] == (1 << (bits - 1)) - 1) and q["n16"][0] == 0.0
    np.testing.assert_allclose(np.sum(q["y"][1:] ** 2, axis=1), 1.0, atol=1e-12)
    xhat = dense.dequantize(q["codes"], q["n16"], bits, Pi)
    # per-coordinate distortion of unit vectors close to the table value
    u = x[1:] / q["norm"][1:, None]
    err = np.mean(np.sum((u - xhat[1:] / q["n16"][1:, None]) ** 2, axis=1)) / d
    assert abs(err - dense.beta_codebook(bits, d)[2]) < 0.05 * dense.beta_codebook(bits, d)[2]


def test_orientation_with_a_non_symmetric_rotation():
    """y = Pi x / ||x|| element by element, and xhat = n16 Pi^T c, with Pi a signed cyclic shift
    (orthogonal, not symmetric): (Pi x)_i = s_i x_{(i+1) mod d}.  A transposed Pi would read
    x_{i-1} instead and fail every coordinate."""
    d, bits = 16, 3
    rng = np.random.default_rng(3)
    s = rng.choice([-1.0, 1.0], size=d)
    Pi = np.zeros((d, d))
    for i in range(d):
        Pi[i, (i + 1) % d] = s[i]
    assert not np.allclose(Pi, Pi.T)
    x = rng.standard_normal((50, d))
    q = dense.quantize(x, bits, Pi)
    nrm = np.sqrt(np.sum(x * x, axis=1))
    for i in range(d):
        np.testing.assert_array_equal(q["y"][:, i], s[i] * x[:, (i + 1) % d] / nrm)
    c, beta, _ = dense.beta_codebook(bits, d)
    xhat = dense.dequantize(q["codes"], q["n16"], bits, Pi)
    for i in range(d):
        # (Pi^T c)_{(i+1) mod d} = s_i c_i
        np.testing.assert_array_equal(xhat[:, (i + 1) % d], q["n16"] * (s[i] * c[q["codes"][:, i].astype(np.int64)]))
