"""GPU parity of the fused decode attention (pq_query_prep + pq_attention) against the oracle
(needs an MI355X).

Tolerance, derived from the arithmetic.  Per query the output error is at most
    A * (2.5 * dz + 4e-6 * sqrt(d)),   A = sum_t p_t max_e |v_te|,
where dz bounds the logit error of every token:
  * quantized tokens: the query terms are integers of 21 bits relative to their largest
    entry, so the score is off by at most 2^-21 max|H(D q)| sum_e |c_e| n16/d
    + 2^-21 max|G q| rnorm16 sqrt(pi/2), plus 1e-6 of the score's L1 size (fp32 query
    preparation); times the softmax scale, plus the fp32 rounding of the logit;
  * window tokens: fp32 dot products of bf16 values (exact products), 1e-6 of their L1 size;
and a logit error dz moves the probabilities by at most 2 dz in L1.  The second term covers
the fp16 hi + lo pairs of probabilities and centroids (2^-22 each), fp32 accumulation and
the inverse rotation, which spreads an error in the rotated basis over sqrt(d).
"""

import math

import numpy as np
import pytest
import torch

import kv_cache_quantization_amd as pq
import synth
from oracle import attention, codec, hadamard, lloyd_max, numerics
from tests import parity, seeded

pytestmark = pytest.mark.gpu


def _case(label):
    print("\n[case] %s" % label, flush=True)


def _f16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float16)).cuda()


def _check(got, q, kc, kn, vc, vn, bits, D_k, D_v, k_win, v_win, scale, qbits=None, rn=None, G=None, label=""):
    """Compare one head's GPU output (n_q, d) with the oracle; returns the worst err / tol."""
    d = q.shape[1]
    res = attention.decode_attention(q, kc, kn, vc, vn, bits, D_k, D_v, k_win, v_win, scale=scale,
                                     k_qbits=qbits, k_rn16=rn, G=G)
    ref, p, z, values = res["out"], res["p"], res["z"], res["v"]
    T = kc.shape[0]
    dz = 2.0 ** -23 * np.abs(z)
    if T:
        qrot = (q * D_k[None, :]) @ hadamard.sylvester(d).T
        cent = lloyd_max.codebook(bits)[0]
        c_l1 = np.sum(np.abs(cent[kc.astype(np.int64)]), axis=1) * kn / d           # (T,)
        ds = 2.0 ** -21 * np.max(np.abs(qrot), axis=1)[:, None] * c_l1[None, :] + 1e-6 * res["score_l1"]
        if G is not None:
            sq = q @ G.T
            ds += 2.0 ** -21 * np.max(np.abs(sq), axis=1)[:, None] * (rn * math.sqrt(math.pi / 2))[None, :]
        dz[:, :T] += abs(scale) * ds
    if k_win is not None and k_win.shape[0]:
        dz[:, T:] += abs(scale) * 1e-6 * (np.abs(q) @ np.abs(k_win).T)
    A = p @ np.max(np.abs(values), axis=1)
    tol = A * (2.5 * np.max(dz, axis=1) + 4e-6 * math.sqrt(d)) + 1e-30
    err = np.max(np.abs(got - ref), axis=1)
    worst = float(np.max(err / tol))
    assert worst <= 1.0, "%s: attention off by %.3g of the bound (err %s, tol %s)" % (label, worst, err, tol)
    return worst


CASES = [
    # d, bits, m, n_heads, n_q, n_tok, n_win, packed, scale
    (128, 3, 128, 2, 16, 16 * 9 + 5, 7, False, None),
    (64, 2, 64, 3, 5, 40, 0, False, None),
    (256, 4, 0, 2, 7, 100, 3, False, None),
    (512, 3, 512, 1, 16, 16 * 3 + 1, 5, False, None),
    (128, 4, 256, 1, 3, 1, 0, False, None),             # one token, m != d
    (64, 1, 0, 2, 1, 0, 9, False, None),                # window only
    (256, 3, 256, 2, 16, 1000, 128, True, None),
    (128, 3, 64, 2, 4, 333, 2, True, 0.7),              # packed odd width, peaky softmax
    (512, 4, 0, 1, 2, 70, 0, True, None),
    (64, 3, 64, 1, 16, 16 * 300 + 11, 16, True, None),
    (128, 4, 0, 1, 16, 16 * 2048 + 37, 4, False, None),  # ranges of two tiles
    (256, 2, 512, 1, 9, 16 * 1100 + 3, 1, False, 0.2),   # ranges of several tiles, m > d
]


@pytest.mark.parametrize("d,bits,m,n_heads,n_q,n_tok,n_win,packed,scale", CASES)
def test_attention_random_codes(d, bits, m, n_heads, n_q, n_tok, n_win, packed, scale):
    """Attention over arbitrary codes, norms, residual bits and windows (drawn on the oracle side)."""
    _case("attention d=%d bits=%d m=%d heads=%d n_q=%d n_tok=%d n_win=%d packed=%d" %
          (d, bits, m, n_heads, n_q, n_tok, n_win, packed))
    rng = np.random.default_rng(d * 11 + bits * 5 + m + n_tok + n_win)
    kc = rng.integers(0, 1 << bits, size=(n_heads, n_tok, d), dtype=np.uint8)
    vc = rng.integers(0, 1 << bits, size=(n_heads, n_tok, d), dtype=np.uint8)
    kn = numerics.round_fp16(np.exp(rng.uniform(-1, 2.5, size=(n_heads, n_tok))))
    vn = numerics.round_fp16(np.exp(rng.uniform(-3, 3, size=(n_heads, n_tok))))
    if n_tok:
        kn[0, 0] = 0.0                                   # a zero key block
        vn[0, -1] = 0.0                                  # a zero value block
    qbits = rng.integers(0, 256, size=(n_heads, n_tok, m // 8), dtype=np.uint8)
    rn = numerics.round_fp16(kn * rng.uniform(0.0, 0.3, size=(n_heads, n_tok)))
    qf = rng.standard_normal((n_heads, n_q, d)).astype(np.float32)
    if n_q > 1:
        qf[0, 1] = 0.0                                   # an all-zero query: uniform weights
    qu = synth.bf16_from_f32(qf)
    kw = synth.bf16_from_f32(2.0 * rng.standard_normal((n_heads, n_win, d)).astype(np.float32))
    vw = synth.bf16_from_f32(rng.standard_normal((n_heads, n_win, d)).astype(np.float32))
    k_seed, v_seed, g_seed = d + 3, d + 4, d + 5
    sm = scale if scale is not None else 1.0 / math.sqrt(d)

    Gt = seeded.gpu_proj(g_seed, m, d) if m else None
    qt = parity.bf16_tensor(qu)
    prep = pq.query_prep(qt, seeded.gpu_signs(k_seed, d), Gt) if n_tok else None
    if packed:
        kc_in = codec.pack_codes(kc.reshape(-1, d), bits) if n_tok else np.zeros((0, d * bits // 8), np.uint8)
        vc_in = codec.pack_codes(vc.reshape(-1, d), bits) if n_tok else np.zeros((0, d * bits // 8), np.uint8)
    else:
        kc_in, vc_in = kc, vc
    keys = (parity.u8_tensor(kc_in), _f16(kn), parity.u8_tensor(qbits) if m else None, _f16(rn) if m else None)
    values = (parity.u8_tensor(vc_in), _f16(vn))
    out = pq.attention(prep, keys, values, seeded.gpu_signs(v_seed, d), d, bits, n_heads, n_q, n_tok, m=m,
                       k_win=parity.bf16_tensor(kw) if n_win else None, v_win=parity.bf16_tensor(vw) if n_win else None,
                       q=qt if n_win else None, sm_scale=scale, packed=packed)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    q = numerics.bf16_from_bits(qu)
    D_k = seeded.oracle_D(k_seed, d)
    D_v = seeded.oracle_D(v_seed, d)
    G = seeded.oracle_G(g_seed, m, d) if m else None
    worst = 0.0
    for h in range(n_heads):
        worst = max(worst, _check(got[h], q[h], kc[h], kn[h], vc[h], vn[h], bits, D_k, D_v,
                                  numerics.bf16_from_bits(kw[h]) if n_win else None,
                                  numerics.bf16_from_bits(vw[h]) if n_win else None, sm,
                                  qbits[h] if m else None, rn[h] if m else None, G, label="head %d" % h))
    print("[worst err/tol] %.3g" % worst, flush=True)


@pytest.mark.parametrize("d", [256, 512])
def test_attention_end_to_end_config5_shape(d):
    """Config-5 recipe on a slice of tokens: keys (QJL m = d) and values quantized on the GPU,
    attention from the stored codes with a 128-token window; byte and packed codes agree."""
    n_heads, n_tok, n_q, n_win = 2, 16 * 40 + 7, 16, 128
    _case("attention end to end d=%d tokens=%d window=%d" % (d, n_tok, n_win))
    c = synth.config5_attention(d, kv_heads=n_heads, tokens=n_tok, n_q=n_q, window=n_win)
    bits, m = c["bits"], c["m"]
    kst, vst = seeded.gpu_signs(c["k_sign_seed"], d), seeded.gpu_signs(c["v_sign_seed"], d)
    Gt = seeded.gpu_proj(c["proj_seed"], m, d)
    kx, vx = parity.bf16_tensor(c["k"]), parity.bf16_tensor(c["v"])
    kcod, knrm, kqb, krn = pq.quantize(kx, d, bits, kst, Gt)
    vcod, vnrm, _, _ = pq.quantize(vx, d, bits, vst)
    qt = parity.bf16_tensor(c["q"])
    kw, vw = parity.bf16_tensor(c["k_win"]), parity.bf16_tensor(c["v_win"])
    prep = pq.query_prep(qt, kst, Gt)
    out = pq.attention(prep, (kcod, knrm, kqb, krn), (vcod, vnrm), vst, d, bits, n_heads, n_q, n_tok, m=m,
                       k_win=kw, v_win=vw, q=qt)
    pk = pq.quantize(kx, d, bits, kst, Gt, packed=True)[0]
    pv = pq.quantize(vx, d, bits, vst, packed=True)[0]
    outp = pq.attention(prep, (pk, knrm, kqb, krn), (pv, vnrm), vst, d, bits, n_heads, n_q, n_tok, m=m,
                        k_win=kw, v_win=vw, q=qt, packed=True)
    torch.cuda.synchronize()
    assert torch.equal(outp, out)
    got = out.cpu().numpy().astype(np.float64)
    kc = kcod.cpu().numpy().reshape(n_heads, n_tok, d)
    vc = vcod.cpu().numpy().reshape(n_heads, n_tok, d)
    kn = parity.f16_values(knrm).reshape(n_heads, n_tok)
    vn = parity.f16_values(vnrm).reshape(n_heads, n_tok)
    qb = kqb.cpu().numpy().reshape(n_heads, n_tok, m // 8)
    rn = parity.f16_values(krn).reshape(n_heads, n_tok)
    q = numerics.bf16_from_bits(c["q"])
    D_k = seeded.oracle_D(c["k_sign_seed"], d)
    D_v = seeded.oracle_D(c["v_sign_seed"], d)
    G = seeded.oracle_G(c["proj_seed"], m, d)
    for h in range(n_heads):
        _check(got[h], q[h], kc[h], kn[h], vc[h], vn[h], bits, D_k, D_v, numerics.bf16_from_bits(c["k_win"][h]),
               numerics.bf16_from_bits(c["v_win"][h]), 1.0 / math.sqrt(d), qb[h], rn[h], G, label="e2e head %d" % h)


def test_attention_reuses_work_and_output():
    """Two calls in a row on one work buffer, the second with fewer tokens and heads: the
    second result does not depend on what the first left behind."""
    d, bits, n_q = 128, 4, 16
    _case("attention work reuse")
    rng = np.random.default_rng(99)
    res = []
    work = torch.empty((pq.attention_work_bytes(d, 3, 5000),), dtype=torch.uint8, device="cuda")
    for n_heads, n_tok in ((3, 5000), (2, 700)):
        kc = rng.integers(0, 16, size=(n_heads, n_tok, d), dtype=np.uint8)
        vc = rng.integers(0, 16, size=(n_heads, n_tok, d), dtype=np.uint8)
        kn = numerics.round_fp16(np.exp(rng.uniform(-1, 2, size=(n_heads, n_tok))))
        vn = numerics.round_fp16(np.exp(rng.uniform(-1, 2, size=(n_heads, n_tok))))
        qu = synth.bf16_from_f32(rng.standard_normal((n_heads, n_q, d)).astype(np.float32))
        prep = pq.query_prep(parity.bf16_tensor(qu), seeded.gpu_signs(7, d))
        out = pq.attention(prep, (parity.u8_tensor(kc), _f16(kn), None, None), (parity.u8_tensor(vc), _f16(vn)),
                           seeded.gpu_signs(8, d), d, bits, n_heads, n_q, n_tok, work=work)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        q = numerics.bf16_from_bits(qu)
        for h in range(n_heads):
            _check(got[h], q[h], kc[h], kn[h], vc[h], vn[h], bits, seeded.oracle_D(7, d),
                   seeded.oracle_D(8, d), None, None, 1.0 / math.sqrt(d), label="reuse h%d" % h)
        res.append(got)


@pytest.mark.parametrize("d", [256, 512])
def test_attention_config5_full_sampled(d):
    """Config-5 attention shapes at full size (8 KV heads x 65,536 quantized tokens + a 128-token
    window, 16 queries), one call as the benchmark makes it; the oracle checks every head at
    d = 256 and the first and last heads at d = 512 (all their queries) from the GPU's stored
    codes; every output is finite."""
    _case("attention config-5 full size d=%d" % d)
    c = synth.config5_attention(d)
    H, T, _ = c["k"].shape
    n_q, bits, m = c["q"].shape[1], c["bits"], c["m"]
    kst, vst = seeded.gpu_signs(c["k_sign_seed"], d), seeded.gpu_signs(c["v_sign_seed"], d)
    Gt = seeded.gpu_proj(c["proj_seed"], m, d)
    kcod, knrm, kqb, krn = pq.quantize(parity.bf16_tensor(c["k"]), d, bits, kst, Gt)
    vcod, vnrm, _, _ = pq.quantize(parity.bf16_tensor(c["v"]), d, bits, vst)
    qt = parity.bf16_tensor(c["q"])
    prep = pq.query_prep(qt, kst, Gt)
    out = pq.attention(prep, (kcod, knrm, kqb, krn), (vcod, vnrm), vst, d, bits, H, n_q, T, m=m,
                       k_win=parity.bf16_tensor(c["k_win"]), v_win=parity.bf16_tensor(c["v_win"]), q=qt)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    q = numerics.bf16_from_bits(c["q"])
    D_k = seeded.oracle_D(c["k_sign_seed"], d)
    D_v = seeded.oracle_D(c["v_sign_seed"], d)
    G = seeded.oracle_G(c["proj_seed"], m, d)
    for h in (range(H) if d == 256 else (0, H - 1)):     # every head at d = 256
        kc = kcod[h * T:(h + 1) * T].cpu().numpy()
        vc = vcod[h * T:(h + 1) * T].cpu().numpy()
        kn = parity.f16_values(knrm[h * T:(h + 1) * T])
        vn = parity.f16_values(vnrm[h * T:(h + 1) * T])
        qb = kqb[h * T:(h + 1) * T].cpu().numpy()
        rn = parity.f16_values(krn[h * T:(h + 1) * T])
        worst = _check(got[h], q[h], kc, kn, vc, vn, bits, D_k, D_v, numerics.bf16_from_bits(c["k_win"][h]),
                       numerics.bf16_from_bits(c["v_win"][h]), 1.0 / math.sqrt(d), qb, rn, G,
                       label="full d=%d head %d" % (d, h))
        print("[head %d worst err/tol] %.3g" % (h, worst), flush=True)
