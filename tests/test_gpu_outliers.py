"""GPU parity of the QJL outlier-channel path (qjl_outlier_channels, qjl_sketch_split,
qjl_score_add) against the oracle (needs an MI355X).  eliza quantization README, QJL,
"Algorithm in one paragraph": a top-k outlier sketch per group of group_size consecutive
tokens with its own JL projection."""

import numpy as np
import pytest
import torch

import kv_cache_quantization_amd as pq
import synth
from oracle import numerics, qjl
from tests import parity, seeded

pytestmark = pytest.mark.gpu

TIE = 1e-5          # channel norms this close (relative) may rank either way (fp32 sums)


def _case(label):
    print("\n[case] %s" % label, flush=True)


def _check_outliers(keys, gpu_idx, gs, n_out, label):
    """keys (T, d) float64 of one head; gpu_idx (n_groups, n_out).  The GPU's choice must be
    a valid top-n_out in decreasing norm; it must equal the oracle's wherever the ranking has
    no near-tie."""
    T, d = keys.shape
    ref = qjl.outlier_channels(keys, gs, n_out)
    assert gpu_idx.shape == ref.shape, label
    for g in range(ref.shape[0]):
        blk = keys[g * gs:(g + 1) * gs]
        ss = (blk ** 2).sum(axis=0)
        sel = gpu_idx[g].astype(np.int64)
        assert len(set(sel.tolist())) == n_out, "%s g%d: repeated channel" % (label, g)
        rest = np.setdiff1d(np.arange(d), sel)
        tol = TIE * max(ss.max(), 1e-300)
        if rest.size:
            assert ss[sel].min() >= ss[rest].max() - tol, "%s g%d: not a top-%d" % (label, g, n_out)
        assert np.all(np.diff(ss[sel]) <= tol), "%s g%d: not in decreasing norm" % (label, g)
        order = np.sort(ss)[::-1]
        gaps = np.abs(np.diff(order[:n_out + 1]))
        if gaps.size == 0 or gaps.min() > tol:
            assert np.array_equal(sel, ref[g]), "%s g%d: differs from the oracle" % (label, g)


@pytest.mark.parametrize("d,gs,n_out,heads,T", [(128, 32, 8, 3, 32 * 5 + 7), (64, 16, 4, 2, 50),
                                                 (256, 32, 16, 2, 96), (128, 7, 1, 1, 40),
                                                 (64, 64, 64, 1, 64)])
def test_outlier_channels_parity(d, gs, n_out, heads, T):
    _case("outlier channels d=%d gs=%d n_out=%d heads=%d T=%d" % (d, gs, n_out, heads, T))
    rng = np.random.default_rng(d + gs + n_out)
    x = rng.standard_normal((heads, T, d)).astype(np.float32)
    x[:, :, rng.choice(d, 3, replace=False)] *= np.float32(12.0)   # persistent outlier channels
    u = synth.bf16_from_f32(x)
    idx = pq.qjl_outlier_channels(parity.bf16_tensor(u), gs, n_out)
    torch.cuda.synchronize()
    keys = numerics.bf16_from_bits(u)
    gi = idx.cpu().numpy()
    for h in range(heads):
        _check_outliers(keys[h], gi[h], gs, n_out, "head %d" % h)


@pytest.mark.parametrize("B,Hkv,Hq,T,d,m,m_o,gs,n_out", [
    (2, 2, 8, 32 * 6 + 5, 128, 256, 256, 32, 8),      # config-4 geometry, ragged last group
    (1, 3, 3, 100, 64, 64, 128, 16, 4),
    (1, 1, 4, 64, 256, 128, 64, 32, 8),
])
def test_split_sketch_and_score(B, Hkv, Hq, T, d, m, m_o, gs, n_out):
    _case("split sketch + score B=%d Hkv=%d Hq=%d T=%d d=%d m=%d m_o=%d" % (B, Hkv, Hq, T, d, m, m_o))
    c = synth.config4(seed=3, batch=B, kv_heads=Hkv, tokens=T, head_dim=d, q_heads=Hq, m=m)
    kt, qt = parity.bf16_tensor(c["keys"]), parity.bf16_tensor(c["q"])
    Gt, Got = seeded.gpu_proj(c["proj_seed"], m, d), seeded.gpu_proj(synth.OUTLIER_PROJ_SEED, m_o, d)
    idx = pq.qjl_outlier_channels(kt, gs, n_out)
    kf = kt.view(B * Hkv, T, d)
    ix = idx.view(B * Hkv, -1, n_out)
    b_in, n_in = pq.qjl_sketch(kf, Gt, split=(ix, T, gs, 0))
    b_out, n_out16 = pq.qjl_sketch(kf, Got, split=(ix, T, gs, 1))
    sq, sqo = pq.qjl_project(qt, Gt), pq.qjl_project(qt, Got)
    sc = pq.qjl_score(sq, b_in, n_in, B, Hkv, Hq, T)
    sc = pq.qjl_score(sqo, b_out, n_out16, B, Hkv, Hq, T, out=sc, accumulate=True)
    torch.cuda.synchronize()
    keys = numerics.bf16_from_bits(c["keys"]).reshape(B * Hkv, T, d)
    G, Go = seeded.oracle_G(c["proj_seed"], m, d), seeded.oracle_G(synth.OUTLIER_PROJ_SEED, m_o, d)
    q = numerics.bf16_from_bits(c["q"])
    gi = ix.cpu().numpy()
    bi, bo = b_in.view(B * Hkv, T, m // 8).cpu().numpy(), b_out.view(B * Hkv, T, m_o // 8).cpu().numpy()
    ni = parity.f16_values(n_in).reshape(B * Hkv, T)
    no = parity.f16_values(n_out16).reshape(B * Hkv, T)
    got = sc.cpu().numpy().astype(np.float64)
    group = Hq // Hkv
    for hh in range(B * Hkv):
        _check_outliers(keys[hh], gi[hh], gs, n_out, "head %d" % hh)
        sk = qjl.split_sketch(keys[hh], gi[hh], gs, G, Go)     # the GPU's channels, the oracle's split
        parity.check_sketch(sk["k_in"], G, bi[hh], ni[hh], label="inliers h%d" % hh)
        parity.check_sketch(sk["k_out"], Go, bo[hh], no[hh], label="outliers h%d" % hh)
        b, g = divmod(hh, Hkv)
        for h in range(g * group, (g + 1) * group):
            Sq, Soq = (G @ q[b, h])[None, :], (Go @ q[b, h])[None, :]
            ref = qjl.estimate(bi[hh], ni[hh], Sq, m)[0] + qjl.estimate(bo[hh], no[hh], Soq, m_o)[0]
            scale = qjl.estimate_scale(ni[hh], Sq, m)[0] + qjl.estimate_scale(no[hh], Soq, m_o)[0]
            parity.check_scores(got[b, h], ref, np.maximum(scale, 1e-30), label="split score b%d h%d" % (b, h))
