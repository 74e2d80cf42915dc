"""Pins for the oracle's decode attention over a quantized cache (CPU only).

Checked against torch's scaled_dot_product_attention in float64 (a library softmax
attention, independent of the oracle's own), closed forms (an all-zero query averages the
values, a dominant key selects its value) and the linear-in-q form of the two-stage
estimator (the QJL term equals <q, rnorm16 sqrt(pi/2)/m G^T (2 b - 1)>).
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention, codec, hadamard, numerics


def _cache(rng, T, d, bits, m, scale=1.0):
    """Quantized keys and values of T tokens, via the oracle codec; separate sign masks."""
    D_k = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    D_v = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    k = rng.standard_normal((T, d)) * scale
    v = rng.standard_normal((T, d)) * scale
    kq = codec.quantize(k, bits, D_k)
    vq = codec.quantize(v, bits, D_v)
    out = {"D_k": D_k, "D_v": D_v, "k_codes": kq["codes"], "k_n16": kq["n16"],
           "v_codes": vq["codes"], "v_n16": vq["n16"], "G": None, "k_qbits": None, "k_rn16": None}
    if m:
        G = numerics.round_bf16(rng.standard_normal((m, d)))
        res = codec.qjl_residual(k, kq["codes"], kq["n16"], bits, D_k, G)
        out.update(G=G, k_qbits=res["bits"], k_rn16=res["rnorm16"])
    return out


def _run(c, q, bits, k_win, v_win, scale=None):
    return attention.decode_attention(q, c["k_codes"], c["k_n16"], c["v_codes"], c["v_n16"], bits,
                                      c["D_k"], c["D_v"], k_win, v_win, scale=scale,
                                      k_qbits=c["k_qbits"], k_rn16=c["k_rn16"], G=c["G"])


def _sdpa(q, K, V, scale):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None], scale=scale)
    return out[0].numpy()


@pytest.mark.parametrize("d,bits,T,W", [(64, 2, 37, 5), (128, 4, 50, 0), (32, 3, 0, 9), (256, 1, 20, 16)])
def test_matches_library_attention_without_qjl(d, bits, T, W):
    rng = np.random.default_rng(d + T + W)
    c = _cache(rng, T, d, bits, 0)
    q = rng.standard_normal((3, d)) * 2.0
    k_win = rng.standard_normal((W, d)) if W else None
    v_win = rng.standard_normal((W, d)) if W else None
    scale = 1.0 / math.sqrt(d)
    got = _run(c, q, bits, k_win, v_win)["out"]
    K = [codec.dequantize(c["k_codes"], c["k_n16"], bits, c["D_k"])] if T else []
    V = [codec.dequantize(c["v_codes"], c["v_n16"], bits, c["D_v"])] if T else []
    if W:
        K.append(k_win)
        V.append(v_win)
    ref = _sdpa(q, np.concatenate(K), np.concatenate(V), scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d,bits,m,T,W", [(64, 3, 64, 40, 4), (128, 2, 256, 33, 0)])
def test_matches_library_attention_with_qjl(d, bits, m, T, W):
    """The two-stage score is <q, khat + rnorm16 sqrt(pi/2)/m G^T (2 b - 1)>: attention over those
    effective keys, by the library routine."""
    rng = np.random.default_rng(7 * d + m)
    c = _cache(rng, T, d, bits, m)
    q = rng.standard_normal((4, d))
    k_win = rng.standard_normal((W, d)) if W else None
    v_win = rng.standard_normal((W, d)) if W else None
    scale = 0.3
    got = _run(c, q, bits, k_win, v_win, scale=scale)["out"]
    signs = np.where(numerics.unpack_bits_lsb(c["k_qbits"], m), 1.0, -1.0)
    k_eff = codec.dequantize(c["k_codes"], c["k_n16"], bits, c["D_k"]) + \
        (c["k_rn16"][:, None] * math.sqrt(math.pi / 2) / m) * (signs @ c["G"])
    vhat = codec.dequantize(c["v_codes"], c["v_n16"], bits, c["D_v"])
    K = np.concatenate([k_eff] + ([k_win] if W else []))
    V = np.concatenate([vhat] + ([v_win] if W else []))
    np.testing.assert_allclose(got, _sdpa(q, K, V, scale), rtol=1e-11, atol=1e-12)


def test_zero_query_averages_values():
    rng = np.random.default_rng(3)
    d, bits, T, W = 64, 4, 25, 7
    c = _cache(rng, T, d, bits, 64)
    k_win, v_win = rng.standard_normal((W, d)), rng.standard_normal((W, d))
    res = _run(c, np.zeros((1, d)), bits, k_win, v_win)
    vhat = codec.dequantize(c["v_codes"], c["v_n16"], bits, c["D_v"])
    ref = (vhat.sum(axis=0) + v_win.sum(axis=0)) / (T + W)
    np.testing.assert_allclose(res["out"][0], ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(res["p"], 1.0 / (T + W), rtol=1e-12)


def test_dominant_key_selects_its_value():
    """One window key far along q: its probability is 1 to double precision."""
    rng = np.random.default_rng(4)
    d, bits, T = 128, 3, 30
    c = _cache(rng, T, d, bits, 0)
    q = rng.standard_normal((1, d))
    k_win = np.stack([rng.standard_normal(d), 100.0 * q[0]])
    v_win = rng.standard_normal((2, d))
    res = _run(c, q, bits, k_win, v_win)
    np.testing.assert_allclose(res["out"][0], v_win[1], rtol=0, atol=1e-12)


def test_token_order_and_head_signs():
    """Reordering the quantized tokens (keys with their values) leaves the output unchanged;
    dequantizing the values with the key signs instead changes it (the two masks are distinct
    inputs)."""
    rng = np.random.default_rng(5)
    d, bits, T = 64, 4, 21
    c = _cache(rng, T, d, bits, 64)
    q = rng.standard_normal((2, d))
    base = _run(c, q, bits, None, None)["out"]
    perm = rng.permutation(T)
    c2 = dict(c)
    for key in ("k_codes", "k_n16", "v_codes", "v_n16", "k_qbits", "k_rn16"):
        c2[key] = c[key][perm]
    np.testing.assert_allclose(_run(c2, q, bits, None, None)["out"], base, rtol=1e-12, atol=1e-14)
    c3 = dict(c, D_v=c["D_k"])
    assert np.max(np.abs(_run(c3, q, bits, None, None)["out"] - base)) > 1e-3


def test_rotation_commutes_with_the_weighted_sum():
    """sum_t p_t vhat_t = D . H (sum_t p_t n16_t / d . c[code_t]): the weighted sum can be taken
    over centroid vectors in the rotated basis and rotated back once (checked on the oracle's
    dequantize, which rotates every vector)."""
    from oracle import lloyd_max
    rng = np.random.default_rng(6)
    d, bits, T = 128, 4, 19
    c = _cache(rng, T, d, bits, 0)
    p = rng.random(T)
    p /= p.sum()
    vhat = codec.dequantize(c["v_codes"], c["v_n16"], bits, c["D_v"])
    cent = lloyd_max.codebook(bits)[0][c["v_codes"].astype(np.int64)]
    acc = (p * c["v_n16"] / d) @ cent
    np.testing.assert_allclose(p @ vhat, c["D_v"] * (hadamard.sylvester(d) @ acc), rtol=1e-12, atol=1e-14)


def test_empty_cache_rejected():
    with pytest.raises(ValueError):
        attention.decode_attention(np.zeros((1, 8)), np.zeros((0, 8), np.uint8), np.zeros(0),
                                   np.zeros((0, 8), np.uint8), np.zeros(0), 2, np.ones(8), np.ones(8))
