"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark
uses (one call over the whole tensor).  The oracle checks sampled blocks, keys and
tokens one by one; properties that hold at any size are checked on every output.
Needs an MI355X."""

import numpy as np
import pytest
import torch

import kv_cache_quantization_amd as pq
import synth
from oracle import hadamard, lloyd_max, numerics, qjl
from tests import parity

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


def test_config1_full():
    _case("config1 full: 256x512 fp32, d=128, 4-bit")
    c = synth.config1()
    d, bits = c["d"], c["bits"]
    x = torch.from_numpy(c["x"]).cuda()
    st = parity.u8_tensor(c["signs"])
    codes, norms, _, _ = pq.quantize(x, d, bits, st)
    out = pq.dequantize(codes, norms, d, bits, st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    D = hadamard.signs_from_mask(c["signs"], d)
    xs = c["x"].astype(np.float64).reshape(-1, d)
    parity.check_quantize(xs, bits, D, codes.cpu().numpy(), parity.f16_values(norms), label="config1")
    parity.check_dequantize(codes.cpu().numpy(), parity.f16_values(norms), bits, D,
                            out.cpu().numpy().astype(np.float64), False, label="config1 dequantize")


def test_config2_full_sampled():
    _case("config2 full: 4096x4096 bf16, d=128, 5-bit, QJL m=64")
    c = synth.config2()
    d, bits, m = c["d"], c["bits"], c["m"]
    x = parity.bf16_tensor(c["x"])
    st = parity.u8_tensor(c["signs"])
    Gt = parity.bf16_tensor(c["G"])
    codes, norms, qb, rn = pq.quantize(x, d, bits, st, Gt)
    out = pq.dequantize(codes, norms, d, bits, st)
    torch.cuda.synchronize()
    n = codes.shape[0]
    _codes_in_range(codes, bits)
    # every block: reconstruction error near the Lloyd-Max distortion of N(0,1) coordinates
    mse = _relative_mse(x.view(n, d), out.view(n, d))
    assert 0.3 * lloyd_max.codebook(bits)[2] < mse < 3.0 * lloyd_max.codebook(bits)[2], mse
    outlier_blocks = np.unique(c["outlier_positions"] // d)[::8]
    idx = _sample(n, 3000, 21, outlier_blocks)
    xs = numerics.bf16_from_bits(c["x"].reshape(-1, d)[idx])
    D = hadamard.signs_from_mask(c["signs"], d)
    G = numerics.bf16_from_bits(c["G"])
    sel = torch.from_numpy(idx).cuda()
    stats = parity.check_quantize(xs, bits, D, codes[sel].cpu().numpy(), parity.f16_values(norms[sel]), G,
                                  qb[sel].cpu().numpy(), parity.f16_values(rn[sel]), label="config2 sampled")
    parity.check_dequantize(codes[sel].cpu().numpy(), parity.f16_values(norms[sel]), bits, D,
                            out[sel].float().cpu().numpy().astype(np.float64), True, label="config2 dequantize")
    print("  sampled %d blocks" % idx.size, stats, flush=True)


@pytest.mark.parametrize("t", [0, 1, 4, 6, 223])
def test_config3_tensor_sampled(t):
    layout = synth.config3_layout()
    _, layer, name, rows, cols = layout[t]
    _case("config3 tensor %d (layer %d %s %dx%d), d=128, 4-bit" % (t, layer, name, rows, cols))
    xu, signs = synth.config3_tensor(t, rows, cols)
    d, bits = 128, 4
    x = parity.bf16_tensor(xu)
    st = parity.u8_tensor(signs)
    codes, norms, _, _ = pq.quantize(x, d, bits, st)
    out = pq.dequantize(codes, norms, d, bits, st)
    torch.cuda.synchronize()
    n = codes.shape[0]
    _codes_in_range(codes, bits)
    mse = _relative_mse(x.view(n, d), out.view(n, d))
    assert 0.3 * lloyd_max.codebook(bits)[2] < mse < 3.0 * lloyd_max.codebook(bits)[2], mse
    idx = _sample(n, 2000, 30 + t)
    xs = numerics.bf16_from_bits(xu.reshape(-1, d)[idx])
    D = hadamard.signs_from_mask(signs, d)
    sel = torch.from_numpy(idx).cuda()
    parity.check_quantize(xs, bits, D, codes[sel].cpu().numpy(), parity.f16_values(norms[sel]),
                          label="config3 t%d" % t)
    parity.check_dequantize(codes[sel].cpu().numpy(), parity.f16_values(norms[sel]), bits, D,
                            out[sel].float().cpu().numpy().astype(np.float64), True, label="config3 t%d dq" % t)


def test_config4_full_sampled():
    _case("config4 full: keys 4x8x32768x128 bf16, m=256, 32 query heads")
    c = synth.config4()
    B, Hkv, T, d = c["keys"].shape
    Hq, m = c["q"].shape[1], c["m"]
    kt = parity.bf16_tensor(c["keys"])
    Gt = parity.bf16_tensor(c["G"])
    bits, norms = pq.qjl_sketch(kt, Gt)
    sq = pq.qjl_project(parity.bf16_tensor(c["q"]), Gt)
    sc = pq.qjl_score(sq, bits, norms, B, Hkv, Hq, T)
    torch.cuda.synchronize()
    G = numerics.bf16_from_bits(c["G"])
    keys_flat = c["keys"].reshape(-1, d)
    idx = _sample(keys_flat.shape[0], 4000, 41)
    sel = torch.from_numpy(idx).cuda()
    parity.check_sketch(numerics.bf16_from_bits(keys_flat[idx]), G, bits[sel].cpu().numpy(),
                        parity.f16_values(norms[sel]), label="config4 sketch")
    # scores on sampled tokens of every (batch, query head), from the GPU's stored bits and norms
    q = numerics.bf16_from_bits(c["q"])
    bits_np = bits.view(B, Hkv, T, m // 8)
    n16 = norms.view(B, Hkv, T)
    tok = _sample(T, 500, 42)
    tsel = torch.from_numpy(tok).cuda()
    got = sc[:, :, tsel].cpu().numpy().astype(np.float64)
    group = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            kb = bits_np[b, g][tsel].cpu().numpy()
            kn = parity.f16_values(n16[b, g][tsel])
            Sq = q[b, g * group:(g + 1) * group] @ G.T
            ref = qjl.estimate(kb, kn, Sq, m)
            scale = qjl.estimate_scale(kn, Sq, m)
            parity.check_scores(got[b, g * group:(g + 1) * group], ref, np.maximum(scale, 1e-30),
                                label="config4 score b%d g%d" % (b, g))


@pytest.mark.parametrize("d", [256, 512])
def test_config5_tensor_full_sampled(d):
    _case("config5 tensor d=%d full: 8x65536 vectors, 3-bit, QJL m=d, 16 queries per head" % d)
    c = synth.config5_tensor(d)
    H, T, _ = c["x"].shape
    n_q, bits, m = c["q"].shape[1], c["bits"], c["m"]
    st = parity.u8_tensor(c["signs"])
    Gt = parity.bf16_tensor(c["G"])
    x = parity.bf16_tensor(c["x"])
    codes, norms, qb, rn = pq.quantize(x, d, bits, st, Gt)
    out = pq.dequantize(codes, norms, d, bits, st)
    prep = pq.query_prep(parity.bf16_tensor(c["q"]), st, Gt)
    sc = pq.score(prep, codes, norms, d, bits, H, n_q, T, qb, rn, m=m)
    torch.cuda.synchronize()
    n = codes.shape[0]
    _codes_in_range(codes, bits)
    D = hadamard.signs_from_mask(c["signs"], d)
    G = numerics.bf16_from_bits(c["G"])
    idx = _sample(n, 1500, 50 + d)
    sel = torch.from_numpy(idx).cuda()
    xs = numerics.bf16_from_bits(c["x"].reshape(-1, d)[idx])
    stats = parity.check_quantize(xs, bits, D, codes[sel].cpu().numpy(), parity.f16_values(norms[sel]), G,
                                  qb[sel].cpu().numpy(), parity.f16_values(rn[sel]), label="config5 d%d" % d)
    parity.check_dequantize(codes[sel].cpu().numpy(), parity.f16_values(norms[sel]), bits, D,
                            out[sel].float().cpu().numpy().astype(np.float64), True, label="config5 d%d dq" % d)
    print("  sampled %d blocks" % idx.size, stats, flush=True)
    q = numerics.bf16_from_bits(c["q"])
    tok = _sample(T, 300, 60 + d)
    tsel = torch.from_numpy(tok).cuda()
    got = sc[:, :, tsel].cpu().numpy().astype(np.float64)
    cv = codes.view(H, T, d)
    nv, qv, rv = norms.view(H, T), qb.view(H, T, m // 8), rn.view(H, T)
    for h in range(H):
        ref, scale = qjl.two_stage(cv[h][tsel].cpu().numpy(), parity.f16_values(nv[h][tsel]),
                                   qv[h][tsel].cpu().numpy(), parity.f16_values(rv[h][tsel]), q[h], bits, D, G)
        parity.check_scores(got[h], ref, np.maximum(scale, 1e-30), label="config5 d%d score h%d" % (d, h))


def test_single_launch_beyond_4gib():
    """One quantize + dequantize call whose input spans more than 2^32 bytes and whose code
    array spans more than 2^31: a seeded 64 MiB weight tiled on the device, blocks past
    both offsets checked against the oracle."""
    d, bits = 128, 4
    n_blocks = (1 << 24) + 4096 + 7                       # ragged tail
    _case("single launch n_blocks=%d (%.2f GB of bf16)" % (n_blocks, n_blocks * d * 2 / 1e9))
    xu, signs = synth.config3_tensor(0, 4096, 8192)       # 262144 blocks
    base = parity.bf16_tensor(xu).view(-1, d)
    reps = -(-n_blocks // base.shape[0])
    x = base.repeat(reps, 1)[:n_blocks].contiguous()
    st = parity.u8_tensor(signs)
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
    D = hadamard.signs_from_mask(signs, d)
    sel = torch.from_numpy(pick).cuda()
    parity.check_quantize(xs, bits, D, codes[sel].cpu().numpy(), parity.f16_values(norms[sel]), label="4GiB")
    parity.check_dequantize(codes[sel].cpu().numpy(), parity.f16_values(norms[sel]), bits, D,
                            out[sel].float().cpu().numpy().astype(np.float64), True, label="4GiB dq")


@pytest.mark.parametrize("d", [256, 512])
def test_config5_packed_full(d):
    """Config 5 with the 3-bit codes bit-packed: the packed quantize equals the byte-code one
    packed by the oracle (sampled blocks), and dequantize and two-stage scores from the
    packed codes equal the byte-code results over the whole tensor."""
    from oracle import codec
    _case("config5 packed d=%d full" % d)
    c = synth.config5_tensor(d)
    H, T, _ = c["x"].shape
    n_q, bits, m = c["q"].shape[1], c["bits"], c["m"]
    st = parity.u8_tensor(c["signs"])
    Gt = parity.bf16_tensor(c["G"])
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
    n = codes.shape[0]
    idx = _sample(n, 2000, 90 + d)
    sel = torch.from_numpy(idx).cuda()
    assert np.array_equal(pk[sel].cpu().numpy(), codec.pack_codes(codes[sel].cpu().numpy(), bits))


def test_config4_outliers_full_sampled():
    """Config-4 keys (4 x 8 x 32768 x 128) with outlier channels (groups of 32 tokens, top 8,
    a 256-row outlier projection): sampled groups, keys and scores against the oracle."""
    from tests.test_gpu_outliers import _check_outliers
    _case("config4 outliers full: groups of 32, top 8, m_o=256")
    c = synth.config4()
    B, Hkv, T, d = c["keys"].shape
    Hq, m = c["q"].shape[1], c["m"]
    gs, n_out, m_o = 32, 8, 256
    Gou = synth.projection(synth.BASE_SEED + 1000, m_o, d)
    kt = parity.bf16_tensor(c["keys"]).view(B * Hkv, T, d)
    Gt, Got = parity.bf16_tensor(c["G"]), parity.bf16_tensor(Gou)
    idx = pq.qjl_outlier_channels(kt, gs, n_out)
    b_in, n_in = pq.qjl_sketch(kt, Gt, split=(idx, T, gs, 0))
    b_out, n_o = pq.qjl_sketch(kt, Got, split=(idx, T, gs, 1))
    qt = parity.bf16_tensor(c["q"])
    sc = pq.qjl_score(pq.qjl_project(qt, Gt), b_in, n_in, B, Hkv, Hq, T)
    sc = pq.qjl_score(pq.qjl_project(qt, Got), b_out, n_o, B, Hkv, Hq, T, out=sc, accumulate=True)
    torch.cuda.synchronize()
    G, Go = numerics.bf16_from_bits(c["G"]), numerics.bf16_from_bits(Gou)
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
