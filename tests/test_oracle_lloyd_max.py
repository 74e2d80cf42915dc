"""Pins for the oracle's Lloyd-Max N(0,1) codebook (CPU only).

Independent checks: the textbook table (golden file), the 1-bit closed form,
numerical integration of the conditional means and of the distortion with
scipy.integrate.quad (not the closed-form expressions the oracle iterates),
Monte Carlo distortion, symmetry and local optimality.
"""

import math
import os

import numpy as np
import pytest
from scipy import integrate

from oracle import lloyd_max

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    out = {}
    for line in open(os.path.join(GOLDEN, "lloyd_max_gaussian.txt")):
        if line.startswith("#") or not line.strip():
            continue
        b, c_top, c_2nd, mse = line.split()
        out[int(b)] = (float(c_top), float(c_2nd), float(mse))
    return out


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_textbook_table(bits):
    c, beta, mse = lloyd_max.codebook(bits)
    c_top, c_2nd, mse_ref = _golden()[bits]
    assert abs(mse - mse_ref) <= 1e-3 * mse_ref
    if not math.isnan(c_top):
        assert abs(c[-1] - c_top) <= 1e-3 * c_top
    if not math.isnan(c_2nd):
        assert abs(c[-2] - c_2nd) <= 1e-3 * c_2nd


def test_one_bit_closed_form():
    c, beta, mse = lloyd_max.codebook(1)
    assert abs(c[1] - math.sqrt(2 / math.pi)) < 1e-12
    assert abs(c[0] + math.sqrt(2 / math.pi)) < 1e-12
    assert beta[0] == 0.0
    assert abs(mse - (1 - 2 / math.pi)) < 1e-12


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6])
def test_symmetry_and_midpoints(bits):
    c, beta, _ = lloyd_max.codebook(bits)
    L = 1 << bits
    assert c.shape == (L,) and beta.shape == (L - 1,)
    assert np.all(np.diff(c) > 0)
    assert np.allclose(c, -c[::-1], atol=0, rtol=0)
    assert np.allclose(beta, 0.5 * (c[:-1] + c[1:]), atol=1e-15)
    assert beta[L // 2 - 1] == 0.0


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_centroids_are_conditional_means_by_quadrature(bits):
    c, beta, mse = lloyd_max.codebook(bits)
    pdf = lambda x: math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)
    edges = [-np.inf] + list(beta) + [np.inf]
    total = 0.0
    for k in range(len(c)):
        a, b = edges[k], edges[k + 1]
        mass = integrate.quad(pdf, a, b, epsabs=1e-14, epsrel=1e-13)[0]
        first = integrate.quad(lambda x: x * pdf(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(first / mass - c[k]) < 1e-9
        total += integrate.quad(lambda x: (x - c[k]) ** 2 * pdf(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
    assert abs(total - mse) < 1e-10


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_monte_carlo_distortion(bits):
    c, beta, mse = lloyd_max.codebook(bits)
    x = np.random.default_rng(bits).standard_normal(2_000_000)
    idx = np.searchsorted(beta, x, side="left")
    emp = np.mean((x - c[idx]) ** 2)
    assert abs(emp - mse) < 0.01 * mse


@pytest.mark.parametrize("bits", [2, 3])
def test_local_optimality(bits):
    c, beta, mse = lloyd_max.codebook(bits)
    pdf = lambda x: math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)

    def distortion(cc, bb):
        edges = [-np.inf] + list(bb) + [np.inf]
        return sum(integrate.quad(lambda x: (x - cc[k]) ** 2 * pdf(x), edges[k], edges[k + 1])[0]
                   for k in range(len(cc)))

    base = distortion(c, beta)
    for k in range(len(c)):
        for eps in (1e-3, -1e-3):
            cc = c.copy()
            cc[k] += eps
            assert distortion(cc, beta) > base
    for k in range(len(beta)):
        for eps in (1e-3, -1e-3):
            bb = beta.copy()
            bb[k] += eps
            assert distortion(c, bb) > base


@pytest.mark.slow
@pytest.mark.parametrize("bits", [7, 8])
def test_high_bit_codebooks_converge(bits):
    c, beta, mse = lloyd_max.codebook(bits)
    # high-resolution (Panter-Dite) approximation of the Gaussian distortion
    panter_dite = (math.sqrt(3) * math.pi / 2) / (1 << bits) ** 2
    assert 0.8 < mse / panter_dite < 1.05
    assert np.allclose(c, -c[::-1])
