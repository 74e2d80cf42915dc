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


# --- outlier channels (eliza README, QJL, "Algorithm in one paragraph"; qjl_apply.py,
# calibrate_key_outliers) ---------------------------------------------------------------

def test_outlier_channels_fixture_and_ties():
    d, gs = 8, 4
    keys = np.tile(np.arange(1.0, d + 1.0), (10, 1))        # channel norm grows with the channel
    keys[4:8, 2] = 100.0                                     # group 1: channel 2 dominates
    idx = qjl.outlier_channels(keys, gs, 3)
    assert idx.tolist() == [[7, 6, 5], [2, 7, 6], [7, 6, 5]]  # 10 tokens: groups of 4, 4 and 2
    flat = np.ones((4, d))
    assert qjl.outlier_channels(flat, gs, 3).tolist() == [[0, 1, 2]]   # equal norms: lower channels


@pytest.mark.parametrize("d,gs,n_out", [(16, 8, 3), (64, 32, 8), (128, 32, 8)])
def test_outlier_channels_against_pairwise_ranks(d, gs, n_out):
    """A channel is chosen iff fewer than n_out channels outrank it (larger norm, or equal
    norm and a lower index) -- ranks counted pairwise, no sorting."""
    rng = np.random.default_rng(d + gs)
    keys = rng.standard_normal((3 * gs + 5, d))
    keys[:, 5] *= 6.0
    idx = qjl.outlier_channels(keys, gs, n_out)
    for g in range(idx.shape[0]):
        blk = keys[g * gs:(g + 1) * gs]
        nrm = np.sqrt((blk ** 2).sum(axis=0))
        outrank = (nrm[None, :] > nrm[:, None]) | ((nrm[None, :] == nrm[:, None]) &
                                                    (np.arange(d)[None, :] < np.arange(d)[:, None]))
        rank = outrank.sum(axis=1)                          # channels outranking each channel
        assert set(idx[g].tolist()) == set(np.nonzero(rank < n_out)[0].tolist())
        assert np.all(np.diff(nrm[idx[g]]) <= 0)            # decreasing norm


def test_split_sketch_partitions_each_key():
    rng = np.random.default_rng(3)
    T, d, gs = 40, 32, 16
    keys = rng.standard_normal((T, d))
    idx = qjl.outlier_channels(keys, gs, 4)
    S, S_o = rng.standard_normal((64, d)), rng.standard_normal((32, d))
    sk = qjl.split_sketch(keys, idx, gs, S, S_o)
    assert np.array_equal(sk["k_in"] + sk["k_out"], keys)
    for t in range(T):
        nz = set(np.nonzero(sk["k_out"][t])[0].tolist())
        assert nz <= set(idx[t // gs].tolist())
        assert np.all(sk["k_in"][t, idx[t // gs]] == 0.0)
    assert np.allclose(sk["in"]["norm"] ** 2 + sk["out"]["norm"] ** 2, (keys ** 2).sum(axis=1))
    # no outlier channels: the inlier part is the whole key and the score is the plain estimator
    none = qjl.split_sketch(keys, np.zeros((3, 0), dtype=np.int64), gs, S, S_o)
    q = rng.standard_normal((5, d))
    plain = qjl.estimate(qjl.sketch(keys, S)["bits"], qjl.sketch(keys, S)["norm16"], q @ S.T, 64)
    assert np.array_equal(qjl.estimate_split(none, q, S, S_o), plain)


def test_split_estimator_unbiased():
    """Monte Carlo over both matrices: mean -> q.k, variance -> the sum of the two terms'
    closed forms."""
    d, m, m_o, gs = 32, 64, 32, 1
    rng = np.random.default_rng(11)
    k = rng.standard_normal(d)
    k[[2, 9]] *= 15.0
    k /= np.linalg.norm(k)
    q = rng.standard_normal(d)
    idx = qjl.outlier_channels(k[None, :], gs, 2)
    assert sorted(idx[0].tolist()) == [2, 9]
    n = 12000
    est = np.empty(n)
    for t in range(n):
        S, S_o = rng.standard_normal((m, d)), rng.standard_normal((m_o, d))
        sk = qjl.split_sketch(k[None, :], idx, gs, S, S_o)
        est[t] = qjl.estimate_split(sk, q[None, :], S, S_o)[0, 0]
    k_out = np.zeros(d)
    k_out[[2, 9]] = k[[2, 9]]
    k_in = k - k_out
    n_in, n_o = numerics.round_fp16(np.linalg.norm(k_in)), numerics.round_fp16(np.linalg.norm(k_out))
    # the stored norms are fp16: the estimator is unbiased for q.k_in * n_in/|k_in| + ...
    mean = np.dot(q, k_in) * n_in / np.linalg.norm(k_in) + np.dot(q, k_out) * n_o / np.linalg.norm(k_out)
    var = (_closed_form_var(q, k_in * n_in / np.linalg.norm(k_in), m)
           + _closed_form_var(q, k_out * n_o / np.linalg.norm(k_out), m_o))
    assert abs(est.mean() - mean) <= 4.5 * math.sqrt(var / n)
    assert abs(est.var() / var - 1.0) < 0.06
    assert abs(mean - np.dot(q, k)) < 1e-3 * np.linalg.norm(q)
