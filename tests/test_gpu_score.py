"""GPU parity of the two-stage score (pq_query_prep + pq_score) against the oracle
(needs an MI355X)."""

import numpy as np
import pytest
import torch

import kv_cache_quantization_amd as pq
import synth
from oracle import codec, hadamard, numerics, qjl
from tests import parity, seeded

pytestmark = pytest.mark.gpu


def _case(label):
    print("\n[case] %s" % label, flush=True)


def _queries(rng, n_heads, n_q, d):
    q = rng.standard_normal((n_heads, n_q, d)).astype(np.float32)
    q[0, 0, :3] *= 40.0                      # a query dominated by a few entries
    if n_q > 1:
        q[0, 1] = 0.0                        # an all-zero query
    return synth.bf16_from_f32(q)


def _reference(codes, n16, qbits, rn16, q, bits, D, G, m):
    """Oracle scores and their L1 scale for one head: (n_q, n_tok) each."""
    if m:
        return qjl.two_stage(codes, n16, qbits, rn16, q, bits, D, G)
    xhat = codec.dequantize(codes, n16, bits, D)
    return q @ xhat.T, np.abs(q) @ np.abs(xhat).T


def _check_prep(prep, qu, D, G, d, m, n_heads, n_q):
    """prep's H (D q) and G q against the oracle (D, G from the oracle's generator)."""
    qrot, sq = pq.prep_views(prep, d, m, n_heads)
    qrot, sq = qrot.cpu().numpy().astype(np.float64), sq.cpu().numpy().astype(np.float64)
    q = numerics.bf16_from_bits(qu)
    H = hadamard.sylvester(d)
    ref = (q * D) @ H.T                                   # H (D q)
    assert np.all(np.abs(qrot[:, :n_q] - ref) <= 1e-6 * (np.abs(q) @ np.abs(H).T) + 1e-30)
    assert np.all(qrot[:, n_q:] == 0.0)
    if m:
        ref = q @ G.T
        assert np.all(np.abs(sq[:, :n_q] - ref) <= 1e-5 * (np.abs(q) @ np.abs(G).T) + 1e-30)
        assert np.all(sq[:, n_q:] == 0.0)


CASES = [
    # d, bits, m, n_heads, n_q, n_tok
    (128, 3, 128, 2, 16, 16 * 9 + 5),
    (64, 1, 64, 3, 5, 40),
    (256, 2, 0, 2, 7, 100),
    (512, 4, 512, 1, 16, 16 * 3 + 1),
    (256, 3, 256, 2, 1, 17),
    (512, 3, 832, 1, 16, 33),                 # d + m at its limit
    (128, 4, 1024, 1, 3, 64),
    (64, 2, 0, 1, 16, 1),
]


@pytest.mark.parametrize("d,bits,m,n_heads,n_q,n_tok", CASES)
def test_two_stage_random_codes(d, bits, m, n_heads, n_q, n_tok):
    """Scores from arbitrary codes, norms and residual bits (drawn on the oracle side)."""
    _case("two-stage d=%d bits=%d m=%d heads=%d n_q=%d n_tok=%d" % (d, bits, m, n_heads, n_q, n_tok))
    rng = np.random.default_rng(d * 7 + bits * 3 + m + n_tok)
    codes = rng.integers(0, 1 << bits, size=(n_heads, n_tok, d), dtype=np.uint8)
    n16 = numerics.round_fp16(np.exp(rng.uniform(-4, 4, size=(n_heads, n_tok))))
    n16[0, 0] = 0.0                                       # a zero block
    qbits = rng.integers(0, 256, size=(n_heads, n_tok, m // 8), dtype=np.uint8)
    rn16 = numerics.round_fp16(n16 * rng.uniform(0.0, 0.3, size=(n_heads, n_tok)))
    qu = _queries(rng, n_heads, n_q, d)
    st = seeded.gpu_signs(d + 1, d)
    prep = pq.query_prep(parity.bf16_tensor(qu), st, seeded.gpu_proj(d + 2, m, d) if m else None)
    out = pq.score(prep, parity.u8_tensor(codes), torch.from_numpy(n16.astype(np.float16)).cuda(), d, bits,
                   n_heads, n_q, n_tok, parity.u8_tensor(qbits) if m else None,
                   torch.from_numpy(rn16.astype(np.float16)).cuda() if m else None, m=m)
    torch.cuda.synchronize()
    D = seeded.oracle_D(d + 1, d)
    G = seeded.oracle_G(d + 2, m, d) if m else None
    _check_prep(prep, qu, D, G, d, m, n_heads, n_q)
    got = out.cpu().numpy().astype(np.float64)
    q = numerics.bf16_from_bits(qu)
    for h in range(n_heads):
        ref, scale = _reference(codes[h], n16[h], qbits[h], rn16[h], q[h], bits, D, G, m)
        parity.check_scores(got[h], ref, np.maximum(scale, 1e-30), label="two-stage h%d" % h)
    # the same codes bit-packed on the oracle side: identical integer sums, identical scores
    pk = codec.pack_codes(codes.reshape(n_heads * n_tok, d), bits)
    outp = pq.score(prep, parity.u8_tensor(pk), torch.from_numpy(n16.astype(np.float16)).cuda(), d, bits,
                    n_heads, n_q, n_tok, parity.u8_tensor(qbits) if m else None,
                    torch.from_numpy(rn16.astype(np.float16)).cuda() if m else None, m=m, packed=True)
    torch.cuda.synchronize()
    assert torch.equal(outp, out)


@pytest.mark.parametrize("d", [256, 512])
def test_two_stage_end_to_end_config5_shape(d):
    """Config-5 recipe (log-normal channel scales, 3-bit, m = d) on a slice of tokens:
    quantize on the GPU, then score from the GPU's stored codes, norms and bits."""
    n_heads, n_tok, n_q = 2, 16 * 20 + 9, 16
    _case("two-stage end to end d=%d tokens=%d" % (d, n_tok))
    c = synth.config5_tensor(d, kv_heads=n_heads, tokens=n_tok, n_q=n_q)
    bits, m = c["bits"], c["m"]
    st = seeded.gpu_signs(c["sign_seed"], d)
    Gt = seeded.gpu_proj(c["proj_seed"], m, d)
    codes, norms, qb, rn = pq.quantize(parity.bf16_tensor(c["x"]), d, bits, st, Gt)
    prep = pq.query_prep(parity.bf16_tensor(c["q"]), st, Gt)
    out = pq.score(prep, codes, norms, d, bits, n_heads, n_q, n_tok, qb, rn, m=m)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    codes_np = codes.cpu().numpy().reshape(n_heads, n_tok, d)
    n16 = parity.f16_values(norms).reshape(n_heads, n_tok)
    qbits = qb.cpu().numpy().reshape(n_heads, n_tok, m // 8)
    rn16 = parity.f16_values(rn).reshape(n_heads, n_tok)
    q = numerics.bf16_from_bits(c["q"])
    D = seeded.oracle_D(c["sign_seed"], d)
    G = seeded.oracle_G(c["proj_seed"], m, d)
    for h in range(n_heads):
        ref, scale = qjl.two_stage(codes_np[h], n16[h], qbits[h], rn16[h], q[h], bits, D, G)
        parity.check_scores(got[h], ref, np.maximum(scale, 1e-30), label="e2e two-stage h%d" % h)
    # quantize and score with packed codes: the same scores
    pcodes, _, _, _ = pq.quantize(parity.bf16_tensor(c["x"]), d, bits, st, Gt, packed=True)
    outp = pq.score(prep, pcodes, norms, d, bits, n_heads, n_q, n_tok, qb, rn, m=m, packed=True)
    torch.cuda.synchronize()
    assert torch.equal(outp, out)
