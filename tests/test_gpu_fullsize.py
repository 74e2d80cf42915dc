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
