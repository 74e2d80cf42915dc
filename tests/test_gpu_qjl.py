"""GPU parity of qjl_sketch / qjl_project / qjl_score against the oracle (needs an MI355X)."""

import numpy as np
import pytest
import torch

import kv_cache_quantization_amd as pq
import synth
from oracle import numerics, qjl
from tests import parity, seeded

pytestmark = pytest.mark.gpu


def _case(label):
    print("\n[case] %s" % label, flush=True)


@pytest.mark.parametrize("d,m,n", [(128, 256, 16 * 40 + 7), (64, 64, 16 * 8 + 1), (256, 128, 16 * 9 + 4),
                                   (512, 512, 16 * 3 + 15), (128, 24, 16 * 5 + 2),
                                   # m a multiple of 128 (row-grouped kernel), ragged pass tails
                                   (64, 128, 16 * 4 * 3 + 17), (64, 512, 16 * 11 + 3), (128, 128, 16 * 4 * 5),
                                   (128, 256, 5), (256, 128, 16 * 2 * 7 + 31)])
def test_sketch_parity(d, m, n):
    _case("sketch d=%d m=%d n=%d" % (d, m, n))
    rng = np.random.default_rng(d + m)
    k = rng.standard_normal((n, d)).astype(np.float32)
    k[:, 3] *= 20.0
    k[0] = 0.0
    ku = synth.bf16_from_f32(k)
    bits, norms = pq.qjl_sketch(parity.bf16_tensor(ku), seeded.gpu_proj(7, m, d))
    torch.cuda.synchronize()
    st = parity.check_sketch(numerics.bf16_from_bits(ku), seeded.oracle_G(7, m, d), bits.cpu().numpy(),
                             parity.f16_values(norms), label="sketch")
    print("  stats", st, flush=True)


@pytest.mark.parametrize("d,m", [(128, 256), (64, 64), (512, 128)])
def test_project_parity(d, m):
    _case("project d=%d m=%d" % (d, m))
    rng = np.random.default_rng(5)
    q = synth.bf16_from_f32(rng.standard_normal((37, d)).astype(np.float32))
    sq = pq.qjl_project(parity.bf16_tensor(q), seeded.gpu_proj(11, m, d))
    torch.cuda.synchronize()
    G = seeded.oracle_G(11, m, d)
    ref = numerics.bf16_from_bits(q) @ G.T
    scale = np.abs(numerics.bf16_from_bits(q)) @ np.abs(G).T
    assert np.all(np.abs(sq.cpu().numpy() - ref) <= 1e-5 * scale + 1e-30)


@pytest.mark.parametrize("B,Hkv,Hq,T,m", [(2, 2, 8, 16 * 21 + 5, 256), (1, 3, 6, 16 * 7 + 1, 64),
                                          (3, 1, 3, 40, 512), (1, 2, 2, 33, 1024), (2, 4, 4, 100, 192)])
def test_score_parity_random_bits(B, Hkv, Hq, T, m):
    """Scores from arbitrary bits and norms (inputs drawn on the oracle side)."""
    _case("score B=%d Hkv=%d Hq=%d T=%d m=%d" % (B, Hkv, Hq, T, m))
    rng = np.random.default_rng(T + m)
    bits = rng.integers(0, 256, size=(B, Hkv, T, m // 8), dtype=np.uint8)
    n16 = numerics.round_fp16(np.exp(rng.uniform(-3, 3, size=(B, Hkv, T))))
    sq = (rng.standard_normal((B, Hq, m)) * 3.0).astype(np.float32)
    sq[0, 0, :5] *= 50.0                               # a few dominant projections
    if Hq > 1:
        sq[0, 1] = 0.0                                 # an all-zero query
    out = pq.qjl_score(torch.from_numpy(sq).cuda(), parity.u8_tensor(bits),
                       torch.from_numpy(n16.astype(np.float16)).cuda(), B, Hkv, Hq, T)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    group = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // group
            Sq = sq[b, h].astype(np.float64)[None, :]
            ref = qjl.estimate(bits[b, g], n16[b, g], Sq, m)[0]
            scale = qjl.estimate_scale(n16[b, g], Sq, m)[0]
            parity.check_scores(got[b, h], ref, np.maximum(scale, 1e-30), label="score b%d h%d" % (b, h))


def test_sketch_then_score_end_to_end():
    _case("sketch -> project -> score")
    B, Hkv, Hq, T, d, m = 2, 2, 8, 16 * 13 + 3, 128, 256
    c = synth.config4(batch=B, kv_heads=Hkv, tokens=T, q_heads=Hq, m=m)
    kt = parity.bf16_tensor(c["keys"])
    qt = parity.bf16_tensor(c["q"])
    Gt = seeded.gpu_proj(c["proj_seed"], m, d)
    bits, norms = pq.qjl_sketch(kt, Gt)
    sq = pq.qjl_project(qt, Gt)
    sc = pq.qjl_score(sq, bits, norms, B, Hkv, Hq, T)
    torch.cuda.synchronize()
    G = seeded.oracle_G(c["proj_seed"], m, d)
    keys = numerics.bf16_from_bits(c["keys"])
    q = numerics.bf16_from_bits(c["q"])
    # the sketch itself
    parity.check_sketch(keys.reshape(-1, d), G, bits.cpu().numpy(), parity.f16_values(norms), label="e2e sketch")
    # scores from the oracle's own sketch; undecided bits (|p| within the band) may go either way
    got = sc.cpu().numpy().astype(np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            s = qjl.sketch(keys[b, g], G)
            Sq = (G @ q[b, h])[None, :]
            ref = qjl.estimate(s["bits"], s["norm16"], Sq, m)[0]
            scale = qjl.estimate_scale(s["norm16"], Sq, m)[0]
            near = np.abs(s["p"]) < parity.BAND * s["norm"][:, None]
            slack = 2 * s["norm16"] * qjl.SQRT_HALF_PI / m * (near * np.abs(Sq)).sum(axis=1)
            # fp16 norm may sit one rounding away
            slack += np.abs(ref) * 1e-3
            assert np.all(np.abs(got[b, h] - ref) <= 1e-3 * scale + slack)
