"""Pins for the oracle's QJL sketch and estimators (CPU only).

Monte Carlo over seeds against the closed-form mean and variance of the sign
estimator, the pages' compression table, the page's pseudo-inverse decode
(which fixes the sign convention) and the two-stage estimator's unbiasedness.
"""

import math
import os

import numpy as np
import pytest

from oracle import qjl, codec, numerics

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
N_MC = 20000


def _mc(q, k, m, n=N_MC, seed=0):
    """Sample the estimator over n independent Gaussian matrices."""
    d = k.shape[0]
    rng = np.random.default_rng(seed)
    est = np.empty(n)
    for t in range(n):
        G = rng.standard_normal((m, d))
        sk = qjl.sketch(k[None, :], G)
        Sq = (G @ q)[None, :]
        est[t] = qjl.estimate(sk["bits"], sk["norm16"], Sq, m)[0, 0]
    return est


def _closed_form_var(q, k, m):
    return ((math.pi / 2) * np.dot(q, q) * np.dot(k, k) - np.dot(q, k) ** 2) / m


@pytest.mark.parametrize("case", ["random", "parallel", "orthogonal", "outlier"])
def test_estimator_unbiased_with_closed_form_variance(case):
    d, m = 32, 64
    rng = np.random.default_rng(42)
    k = rng.standard_normal(d)
    if case == "outlier":
        k[3] *= 20.0
    k /= np.linalg.norm(k)                 # norm 1: the fp16 norm is exact
    q = rng.standard_normal(d) * 2.0
    if case == "parallel":
        q = 1.5 * k
    elif case == "orthogonal":
        q = q - np.dot(q, k) * k
    est = _mc(q, k, m)
    var = _closed_form_var(q, k, m)
    sigma = math.sqrt(var)
    assert abs(est.mean() - np.dot(q, k)) <= 4.5 * sigma / math.sqrt(N_MC)
    assert abs(est.var() / var - 1.0) < 0.05
    # turbopress 0.4.2 README, "Findings" item 1: noise scale sqrt(pi/2) ||r|| ||x|| / sqrt(k)
    assert sigma <= math.sqrt(math.pi / 2) * np.linalg.norm(q) * np.linalg.norm(k) / math.sqrt(m) + 1e-12


def test_storage_ratio_golden():
    for line in open(os.path.join(GOLDEN, "qjl_storage_ratio.txt")):
        if line.startswith("#") or not line.strip():
            continue
        hd, m, ratio = line.split()
        assert round(qjl.storage_ratio(int(hd), int(m)), 2) == float(ratio)


def test_pseudo_inverse_decode_fixes_sign_convention():
    # qjl_apply.py, _qjl_decode_keys: unpack LSB-first, map to 2*bit-1, multiply by the
    # right pseudo-inverse of the (head_dim, proj_dim) matrix, rescale to the stored norm.
    d, m = 128, 256
    rng = np.random.default_rng(3)
    G = rng.standard_normal((m, d))
    k = rng.standard_normal((50, d))
    sk = qjl.sketch(k, G)
    P = G.T                                    # the pages' (head_dim, proj_dim) layout
    signs = np.where(numerics.unpack_bits_lsb(sk["bits"], m), 1.0, -1.0)
    pinv = P.T @ np.linalg.inv(P @ P.T)
    khat = signs @ pinv
    khat *= (sk["norm16"] / np.linalg.norm(khat, axis=1))[:, None]
    cos = np.sum(khat * k, axis=1) / (np.linalg.norm(khat, axis=1) * np.linalg.norm(k, axis=1))
    assert np.all(cos > 0.7)


def test_gqa_head_mapping():
    rng = np.random.default_rng(8)
    B, Hkv, Hq, T, d, m = 2, 2, 8, 16, 32, 64
    G = rng.standard_normal((m, d))
    keys = rng.standard_normal((B, Hkv, T, d))
    q = rng.standard_normal((B, Hq, d))
    bits = np.zeros((B, Hkv, T, m // 8), dtype=np.uint8)
    n16 = np.zeros((B, Hkv, T))
    for b in range(B):
        for g in range(Hkv):
            s = qjl.sketch(keys[b, g], G)
            bits[b, g], n16[b, g] = s["bits"], s["norm16"]
    scores, scale = qjl.score_gqa(bits, n16, q, G)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            signs = np.where(numerics.unpack_bits_lsb(bits[b, g], m), 1.0, -1.0)
            ref = n16[b, g] * math.sqrt(math.pi / 2) / m * (signs @ (G @ q[b, h]))
            assert np.allclose(scores[b, h], ref, rtol=1e-12, atol=1e-12)
    assert np.all(scale >= np.abs(scores) - 1e-12)


def test_two_stage_estimator_unbiased_given_codes():
    d, m, bits = 32, 32, 2
    rng = np.random.default_rng(21)
    D = rng.choice([-1.0, 1.0], size=d)
    x = rng.standard_normal((1, d))
    q = rng.standard_normal((1, d))
    qz = codec.quantize(x, bits, D)
    xhat = codec.dequantize(qz["codes"], qz["n16"], bits, D)
    r = x - xhat
    est = np.empty(N_MC)
    for t in range(N_MC):
        G = rng.standard_normal((m, d))
        res = codec.qjl_residual(x, qz["codes"], qz["n16"], bits, D, G)
        est[t] = qjl.two_stage(qz["codes"], qz["n16"], res["bits"], res["rnorm16"], q, bits, D, G)[0][0, 0]
    rn = np.linalg.norm(r)
    ratio = numerics.round_fp16(rn) / rn
    qx_hat, qr = float((q @ xhat.T)[0, 0]), float((q @ r.T)[0, 0])
    mean_expect = qx_hat + qr * ratio
    var = _closed_form_var(q[0], r[0], m) * ratio ** 2
    assert abs(est.mean() - mean_expect) <= 4.5 * math.sqrt(var / N_MC)
    assert abs(est.var() / var - 1.0) < 0.05
    # and the estimate is unbiased for <q, x> up to the fp16 rounding of ||r||
    assert abs(est.mean() - float((q @ x.T)[0, 0])) <= 4.5 * math.sqrt(var / N_MC) + abs(qr) * abs(ratio - 1)
