"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark
uses (one call over the whole tensor).  The oracle checks whole outputs -- every block of
configs 1 and 2, one whole tensor of each of config 3's seven shapes, every key of config 4,
every block of both config-5 tensors -- in chunks, and the band flips are counted over the
whole output and held to 1e-6 of it; scores are checked for whole (batch, head) groups.
Needs an MI355X."""

import numpy as np
import pytest
import torch

import kv_cache_quantization_amd as pq
import synth
from oracle import codec, lloyd_max, numerics, qjl
from tests import parity, seeded

pytestmark = pytest.mark.gpu


def _case(label):
    print("\n[case] %s" % label, flush=True)


def _sample(n, k, seed, extra=()):
    """Sorted distinct indices: the first and last 64, k seeded random ones and extra."""
    rng = np.random.default_rng(seed)
    idx = np.concatenate([np.arange(min(64, n)), np.arange(max(0, n - 64), n),
                          rng.integers(0, n, size=k), np.asarray(extra, dtype=np.int64)])
    return np.unique(idx)


def _codes_in_range(codes, bits):
    assert int(codes.max().item()) < (1 << bits)


def _relative_mse(x, xhat):
    """sum ||x - xhat||^2 / sum ||x||^2 over all blocks, accumulated on the GPU in fp64."""
    x = x.double()
    e = (x - xhat.double()).pow(2).sum()
    return float(e / x.pow(2).sum())


def _whole_codec(label, x_u16, d, bits, D, codes, norms, out, G=None, qb=None, rn=None, chunk=32768,
                 x_f32=None):
    """Every block of a quantize (+ QJL) and dequantize call against the oracle, in chunks of
    blocks; flips are tallied over the whole output.  GPU outputs are host arrays."""
    n = codes.shape[0]
    tally = parity.Tally()
    worst = 0.0
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        xs = x_f32[s:e].astype(np.float64) if x_f32 is not None else numerics.bf16_from_bits(x_u16[s:e])
        n16 = norms[s:e]
        tally.add(parity.check_quantize(xs, bits, D, codes[s:e], n16, G, None if qb is None else qb[s:e],
                                        None if rn is None else rn[s:e], label="%s blocks %d.." % (label, s),
                                        cap=False))
        if out is not None:
            worst = max(worst, parity.check_dequantize(codes[s:e], n16, bits, D, out[s:e].astype(np.float64),
                                                       x_f32 is None, label="%s dequantize %d.." % (label, s)))
        if (s // chunk) % 8 == 7:
            print("  %s: %d / %d blocks" % (label, e, n), flush=True)
    stats = tally.finish(label)
    print("  %s: worst dequantize error %.3g (relative)" % (label, worst), flush=True)
    return stats


def test_config1_full():
    _case("config1 full: 256x512 fp32, d=128, 4-bit")
    c = synth.config1()
    d, bits = c["d"], c["bits"]
    x = torch.from_numpy(c["x"]).cuda()
    st = seeded.gpu_signs(c["sign_seed"], d)
    codes, norms, _, _ = pq.quantize(x, d, bits, st)
    out = pq.dequantize(codes, norms, d, bits, st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    D = seeded.oracle_D(c["sign_seed"], d)
    _whole_codec("config1", None, d, bits, D, codes.cpu().numpy(), parity.f16_values(norms),
                 out.cpu().numpy(), x_f32=c["x"].reshape(-1, d))


def test_config2_full():
    _case("config2 full: 4096x4096 bf16, d=128, 5-bit, QJL m=64 -- every block")
    c = synth.config2()
    d, bits, m = c["d"], c["bits"], c["m"]
    x = parity.bf16_tensor(c["x"])
    st = seeded.gpu_signs(c["sign_seed"], d)
    Gt = seeded.gpu_proj(c["proj_seed"], m, d)
    codes, norms, qb, rn = pq.quantize(x, d, bits, st, Gt)
    out = pq.dequantize(codes, norms, d, bits, st)
    torch.cuda.synchronize()
    n = codes.shape[0]
    _codes_in_range(codes, bits)
    mse = _relative_mse(x.view(n, d), out.view(n, d))
    assert 0.3 * lloyd_max.codebook(bits)[2] < mse < 3.0 * lloyd_max.codebook(bits)[2], mse
    D = seeded.oracle_D(c["sign_seed"], d)
    G = seeded.oracle_G(c["proj_seed"], m, d)
    _whole_codec("config2", c["x"].reshape(-1, d), d, bits, D, codes.cpu().numpy(), parity.f16_values(norms),
                 out.float().cpu().numpy(), G, qb.cpu().numpy(), parity.f16_values(rn))


@pytest.mark.parametrize("t", [0, 1, 2, 3, 4, 5, 6])
def test_config3_tensor_whole(t):
    """Layer 0's seven tensors (q, k, v, o, gate, up, down): every block."""
    layout = synth.config3_layout()
    _, layer, name, rows, cols = layout[t]
    _case("config3 tensor %d (layer %d %s %dx%d), d=128, 4-bit -- every block" % (t, layer, name, rows, cols))
    xu, sseed = synth.config3_tensor(t, rows, cols)
    d, bits = 128, 4
    x = parity.bf16_tensor(xu)
    st = seeded.gpu_signs(sseed, d)
    codes, norms, _, _ = pq.quantize(x, d, bits, st)
    out = pq.dequantize(codes, norms, d, bits, st)
    torch.cuda.synchronize()
    n = codes.shape[0]
    _codes_in_range(codes, bits)
    mse = _relative_mse(x.view(n, d), out.view(n, d))
    assert 0.3 * lloyd_max.codebook(bits)[2] < mse < 3.0 * lloyd_max.codebook(bits)[2], mse
    del x
    D = seeded.oracle_D(sseed, d)
    _whole_codec("config3 t%d %s" % (t, name), xu.reshape(-1, d), d, bits, D, codes.cpu().numpy(),
                 parity.f16_values(norms), out.float().cpu().numpy(), chunk=65536)


def test_config3_last_tensor_sampled():
    """The last tensor of the weight set (layer 31's down projection, rotation seed 42 + 223)."""
    t = 223
    _, layer, name, rows, cols = synth.config3_layout()[t]
    _case("config3 tensor %d (layer %d %s %dx%d) sampled" % (t, layer, name, rows, cols))
    xu, sseed = synth.config3_tensor(t, rows, cols)
    d, bits = 128, 4
    st = seeded.gpu_signs(sseed, d)
    codes, norms, _, _ = pq.quantize(parity.bf16_tensor(xu), d, bits, st)
    out = pq.dequantize(codes, norms, d, bits, st)
    torch.cuda.synchronize()
    idx = _sample(codes.shape[0], 4000, 30 + t)
    sel = torch.from_numpy(idx).cuda()
    D = seeded.oracle_D(sseed, d)
    st_ = parity.check_quantize(numerics.bf16_from_bits(xu.reshape(-1, d)[idx]), bits, D, codes[sel].cpu().numpy(),
                                parity.f16_values(norms[sel]), label="config3 t%d" % t)
    parity.check_dequantize(codes[sel].cpu().numpy(), parity.f16_values(norms[sel]), bits, D,
                            out[sel].float().cpu().numpy().astype(np.float64), True, label="config3 t%d dq" % t)
    parity.report("config3 t%d sampled" % t, st_)


def test_config4_full():
    _case("config4 full: keys 4x8x32768x128 bf16, m=256, 32 query heads -- every key")
    c = synth.config4()
    B, Hkv, T, d = c["keys"].shape
    Hq, m = c["q"].shape[1], c["m"]
    kt = parity.bf16_tensor(c["keys"])
    Gt = seeded.gpu_proj(c["proj_seed"], m, d)
    bits, norms = pq.qjl_sketch(kt, Gt)
    sq = pq.qjl_project(parity.bf16_tensor(c["q"]), Gt)
    sc = pq.qjl_score(sq, bits, norms, B, Hkv, Hq, T)
    torch.cuda.synchronize()
    G = seeded.oracle_G(c["proj_seed"], m, d)
    keys_flat = c["keys"].reshape(-1, d)
    bits_np = bits.cpu().numpy()
    n16_np = parity.f16_values(norms)
    n = keys_flat.shape[0]
    tally = parity.Tally()
    chunk = 65536
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        tally.add(parity.check_sketch(numerics.bf16_from_bits(keys_flat[s:e]), G, bits_np[s:e], n16_np[s:e],
                                      label="config4 sketch %d.." % s, cap=False))
        if (s // chunk) % 4 == 3:
            print("  config4 sketch: %d / %d keys" % (e, n), flush=True)
    tally.finish("config4 sketch")
    # every token's score for two whole (batch, KV head) groups (four query heads each), from the
    # GPU's stored bits and norms
    q = numerics.bf16_from_bits(c["q"])
    bv = bits_np.reshape(B, Hkv, T, m // 8)
    nv = n16_np.reshape(B, Hkv, T)
    got = sc.cpu().numpy().astype(np.float64)
    group = Hq // Hkv
    worst = 0.0
    for b, g in ((0, 0), (B - 1, Hkv - 1)):
        Sq = q[b, g * group:(g + 1) * group] @ G.T
        ref = qjl.estimate(bv[b, g], nv[b, g], Sq, m)
        scale = qjl.estimate_scale(nv[b, g], Sq, m)
        worst = max(worst, parity.check_scores(got[b, g * group:(g + 1) * group], ref, np.maximum(scale, 1e-30),
                                               label="config4 score b%d g%d" % (b, g)))
    print("  config4 scores: %d tokens x %d heads, worst error / L1 size %.3g" % (T, 2 * group, worst), flush=True)


@pytest.mark.parametrize("d", [256, 512])
def test_config5_tensor_full(d):
    _case("config5 tensor d=%d full: 8x65536 vectors, 3-bit, QJL m=d, 16 queries per head -- every block" % d)
    c = synth.config5_tensor(d)
    H, T, _ = c["x"].shape
    n_q, bits, m = c["q"].shape[1], c["bits"], c["m"]
    st = seeded.gpu_signs(c["sign_seed"], d)
    Gt = seeded.gpu_proj(c["proj_seed"], m, d)
    x = parity.bf16_tensor(c["x"])
    codes, norms, qb, rn = pq.quantize(x, d, bits, st, Gt)
    out = pq.dequantize(codes, norms, d, bits, st)
    prep = pq.query_prep(parity.bf16_tensor(c["q"]), st, Gt)
    sc = pq.score(prep, codes, norms, d, bits, H, n_q, T, qb, rn, m=m)
    torch.cuda.synchronize()
    _codes_in_range(codes, bits)
    del x
    D = seeded.oracle_D(c["sign_seed"], d)
    G = seeded.oracle_G(c["proj_seed"], m, d)
    cn, nn, qn, rnn = codes.cpu().numpy(), parity.f16_values(norms), qb.cpu().numpy(), parity.f16_values(rn)
    _whole_codec("config5 d%d" % d, c["x"].reshape(-1, d), d, bits, D, cn, nn,
                 out.float().cpu().numpy(), G, qn, rnn, chunk=16384 if d == 512 else 32768)
    # every token's scores for two whole heads (16 queries each), from the GPU's stored outputs
    q = numerics.bf16_from_bits(c["q"])
    got = sc.cpu().numpy().astype(np.float64)
    worst = 0.0
    for h in (0, H - 1):
        sl = slice(h * T, (h + 1) * T)
        ref, scale = qjl.two_stage(cn[sl], nn[sl], qn[sl], rnn[sl], q[h], bits, D, G)
        worst = max(worst, parity.check_scores(got[h], ref, np.maximum(scale, 1e-30),
                                               label="config5 d%d score h%d" % (d, h)))
    print("  config5 d%d scores: %d tokens x 2 heads x %d queries, worst error / L1 size %.3g" % (d, T, n_q, worst),
          flush=True)


def test_single_launch_beyond_4gib():
    """One quantize + dequantize call whose input spans more than 2^32 bytes and whose code
    array spans more than 2^31: a seeded 64 MiB weight tiled on the device, blocks past
    both offsets checked against the oracle."""
    d, bits = 128, 4
    n_blocks = (1 << 24) + 4096 + 7                       # ragged tail
    _case("single launch n_blocks=%d (%.2f GB of bf16)" % (n_blocks, n_blocks * d * 2 / 1e9))
    xu, sseed = synth.config3_tensor(0, 4096, 8192)       # 262144 blocks
    base = parity.bf16_tensor(xu).view(-1, d)
    reps = -(-n_blocks // base.shape[0])
    x = base.repeat(reps, 1)[:n_blocks].contiguous()
    st = seeded.gpu_signs(sseed, d)
    codes, norms, _, _ = pq.quantize(x, d, bits, st)
    out = pq.dequantize(codes, norms, d, bits, st)
    torch.cuda.synchronize()
    del x
    nb = base.shape[0]
    pick = np.unique(np.concatenate([np.arange(n_blocks - 300, n_blocks), (1 << 24) + np.arange(-40, 40),
                                     (1 << 23) + np.arange(-40, 40),
                                     np.random.default_rng(7).integers(0, n_blocks, 500)]))
    src = pick % nb
    xs = numerics.bf16_from_bits(xu.reshape(-1, d)[src])
    D = seeded.oracle_D(sseed, d)
    sel = torch.from_numpy(pick).cuda()
    parity.check_quantize(xs, bits, D, codes[sel].cpu().numpy(), parity.f16_values(norms[sel]), label="4GiB")
    parity.check_dequantize(codes[sel].cpu().numpy(), parity.f16_values(norms[sel]), bits, D,
                            out[sel].float().cpu().numpy().astype(np.float64), True, label="4GiB dq")


@pytest.mark.parametrize("d", [256, 512])
def test_config5_packed_full(d):
    """Config 5 with the 3-bit codes bit-packed: the packed quantize equals the byte-code one
    packed by the oracle (every block), and dequantize and two-stage scores from the packed
    codes equal the byte-code results over the whole tensor."""
    _case("config5 packed d=%d full" % d)
    c = synth.config5_tensor(d)
    H, T, _ = c["x"].shape
    n_q, bits, m = c["q"].shape[1], c["bits"], c["m"]
    st = seeded.gpu_signs(c["sign_seed"], d)
    Gt = seeded.gpu_proj(c["proj_seed"], m, d)
    x = parity.bf16_tensor(c["x"])
    codes, norms, qb, rn = pq.quantize(x, d, bits, st, Gt)
    pk, norms_p, qb_p, rn_p = pq.quantize(x, d, bits, st, Gt, packed=True)
    assert torch.equal(norms, norms_p) and torch.equal(qb, qb_p) and torch.equal(rn, rn_p)
    assert torch.equal(pq.dequantize(pk, norms, d, bits, st, packed=True), pq.dequantize(codes, norms, d, bits, st))
    prep = pq.query_prep(parity.bf16_tensor(c["q"]), st, Gt)
    s_b = pq.score(prep, codes, norms, d, bits, H, n_q, T, qb, rn, m=m)
    s_p = pq.score(prep, pk, norms, d, bits, H, n_q, T, qb, rn, m=m, packed=True)
    torch.cuda.synchronize()
    assert torch.equal(s_b, s_p)
    cn, pn = codes.cpu().numpy(), pk.cpu().numpy()
    for s in range(0, cn.shape[0], 65536):
        assert np.array_equal(pn[s:s + 65536], codec.pack_codes(cn[s:s + 65536], bits)), s


def test_config4_outliers_full_sampled():
    """Config-4 keys (4 x 8 x 32768 x 128) with outlier channels (groups of 32 tokens, top 8,
    a 256-row outlier projection): sampled groups, keys and scores against the oracle."""
    from tests.test_gpu_outliers import _check_outliers
    _case("config4 outliers full: groups of 32, top 8, m_o=256")
    c = synth.config4()
    B, Hkv, T, d = c["keys"].shape
    Hq, m = c["q"].shape[1], c["m"]
    gs, n_out, m_o = 32, 8, 256
    kt = parity.bf16_tensor(c["keys"]).view(B * Hkv, T, d)
    Gt, Got = seeded.gpu_proj(c["proj_seed"], m, d), seeded.gpu_proj(synth.OUTLIER_PROJ_SEED, m_o, d)
    idx = pq.qjl_outlier_channels(kt, gs, n_out)
    b_in, n_in = pq.qjl_sketch(kt, Gt, split=(idx, T, gs, 0))
    b_out, n_o = pq.qjl_sketch(kt, Got, split=(idx, T, gs, 1))
    qt = parity.bf16_tensor(c["q"])
    sc = pq.qjl_score(pq.qjl_project(qt, Gt), b_in, n_in, B, Hkv, Hq, T)
    sc = pq.qjl_score(pq.qjl_project(qt, Got), b_out, n_o, B, Hkv, Hq, T, out=sc, accumulate=True)
    torch.cuda.synchronize()
    G, Go = seeded.oracle_G(c["proj_seed"], m, d), seeded.oracle_G(synth.OUTLIER_PROJ_SEED, m_o, d)
    q = numerics.bf16_from_bits(c["q"])
    n_groups = T // gs
    gi = idx.cpu().numpy()
    rng = np.random.default_rng(44)
    for hh in (0, 5, B * Hkv - 1):
        b, g = divmod(hh, Hkv)
        groups = np.unique(np.concatenate([[0, n_groups - 1], rng.integers(0, n_groups, 40)]))
        toks = np.concatenate([np.arange(gg * gs, (gg + 1) * gs) for gg in groups])
        keys = numerics.bf16_from_bits(c["keys"][b, g][toks])
        sub_idx = gi[hh][groups]
        _check_outliers(keys, sub_idx, gs, n_out, "config4 head %d" % hh)
        sk = qjl.split_sketch(keys, sub_idx, gs, G, Go)
        tsel = torch.from_numpy(hh * T + toks).cuda()
        bi, ni = b_in[tsel].cpu().numpy(), parity.f16_values(n_in[tsel])
        bo, no = b_out[tsel].cpu().numpy(), parity.f16_values(n_o[tsel])
        parity.check_sketch(sk["k_in"], G, bi, ni, label="config4 inliers h%d" % hh)
        parity.check_sketch(sk["k_out"], Go, bo, no, label="config4 outliers h%d" % hh)
        got = sc[b][:, torch.from_numpy(toks).cuda()].cpu().numpy().astype(np.float64)
        for h in range(g * (Hq // Hkv), (g + 1) * (Hq // Hkv)):
            Sq, Soq = (G @ q[b, h])[None, :], (Go @ q[b, h])[None, :]
            ref = qjl.estimate(bi, ni, Sq, m)[0] + qjl.estimate(bo, no, Soq, m_o)[0]
            scale = qjl.estimate_scale(ni, Sq, m)[0] + qjl.estimate_scale(no, Soq, m_o)[0]
            parity.check_scores(got[h], ref, np.maximum(scale, 1e-30), label="config4 split score b%d h%d" % (b, h))
