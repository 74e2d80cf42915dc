"""GPU parity of pq_quantize / pq_dequantize against the oracle (needs an MI355X)."""

import math

import numpy as np
import pytest
import torch

import kv_cache_quantization_amd as pq
import synth
from oracle import hadamard, numerics
from tests import parity, seeded

pytestmark = pytest.mark.gpu


def _case(label):
    print("\n[case] %s" % label, flush=True)


def _inputs(n, d, dtype, seed, std=0.02, special=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)).astype(np.float32) * np.float32(std)
    if special and n >= 8:
        x[0] = 0.0                                   # zero block
        x[1] = 0.0
        x[1, 5] = -3.0                               # one-hot block
        x[2] = np.float32(7.0)                       # constant block
        x[3] *= np.float32(1e4)                      # large norm
        x[4] *= np.float32(1e-12)                    # tiny norm
        x[5, ::7] *= np.float32(20.0)                # outlier channels
    if dtype == "bf16":
        u = synth.bf16_from_f32(x)
        return parity.bf16_tensor(u), numerics.bf16_from_bits(u)
    return torch.from_numpy(x).cuda(), x.astype(np.float64)


def _signs(d, seed):
    """(GPU sign mask from the library's generator, oracle D from the oracle's)."""
    return seeded.gpu_signs(seed, d), seeded.oracle_D(seed, d)


def _proj(m, d, seed):
    """(GPU G from the library's generator, oracle G from the oracle's)."""
    return seeded.gpu_proj(seed, m, d), seeded.oracle_G(seed, m, d)


CODEC_CASES = [
    # d, bits, dtype, n_blocks, m
    (128, 4, "f32", 1024, 0),
    (128, 5, "bf16", 16 * 37 + 5, 64),
    (128, 4, "bf16", 16 * 20 + 11, 0),
    (64, 3, "bf16", 16 * 30 + 3, 32),
    (64, 2, "f32", 16 * 9 + 15, 0),
    (256, 3, "bf16", 16 * 12 + 7, 256),
    (256, 6, "bf16", 16 * 10 + 1, 0),
    (512, 3, "bf16", 16 * 8 + 9, 512),
    (512, 4, "f32", 16 * 4 + 2, 0),
    (128, 1, "bf16", 16 * 8 + 3, 8),
    (128, 8, "bf16", 16 * 6 + 13, 24),
    (128, 2, "bf16", 16 * 5, 1024),
    # projections beyond LDS (walked in 128-row chunks): fp32 input, a partial last chunk and
    # N-tile group (m = 600: 38 N tiles, 75-byte bit rows), and d = 256
    (128, 3, "f32", 16 * 3 + 7, 600),
    (256, 4, "f32", 16 * 5 + 3, 512),
    (256, 3, "bf16", 16 * 6 + 5, 512),
]


@pytest.mark.parametrize("d,bits,dtype,n,m", CODEC_CASES)
def test_quantize_dequantize_parity(d, bits, dtype, n, m):
    _case("quantize d=%d bits=%d %s n=%d m=%d" % (d, bits, dtype, n, m))
    xt, x = _inputs(n, d, dtype, seed=d * 100 + bits)
    st, D = _signs(d, seed=d + bits)
    Gt, G = _proj(m, d, seed=m + d) if m else (None, None)
    codes, norms, qb, rn = pq.quantize(xt, d, bits, st, Gt)
    torch.cuda.synchronize()
    gc = codes.cpu().numpy()
    stats = parity.check_quantize(x, bits, D, gc, parity.f16_values(norms), G,
                                  qb.cpu().numpy() if m else None, parity.f16_values(rn) if m else None,
                                  label="quantize d=%d b=%d" % (d, bits))
    print("  stats", stats, flush=True)
    # dequantize the GPU's own codes and norms, both output dtypes
    for out_dt, bf in ((torch.float32, False), (torch.bfloat16, True)):
        _case("dequantize d=%d bits=%d out=%s" % (d, bits, out_dt))
        out = pq.dequantize(codes, norms, d, bits, st, out_dtype=out_dt)
        torch.cuda.synchronize()
        gv = out.float().cpu().numpy().astype(np.float64)
        err = parity.check_dequantize(gc, parity.f16_values(norms), bits, D, gv, bf, label="dequant")
        print("  max rel err", err, flush=True)


@pytest.mark.parametrize("d,bits", [(64, 3), (128, 5), (256, 4), (512, 2), (512, 8), (512, 1)])
def test_dequantize_random_codes(d, bits):
    """Dequantize arbitrary codes and norms (inputs the oracle side draws)."""
    _case("dequantize random codes d=%d bits=%d" % (d, bits))
    rng = np.random.default_rng(d + bits)
    n = 16 * 11 + 9
    codes = rng.integers(0, 1 << bits, size=(n, d), dtype=np.uint8)
    n16 = numerics.round_fp16(np.exp(rng.uniform(-8, 8, size=n)))
    n16[0] = 0.0
    st, D = _signs(d, seed=3)
    ct = parity.u8_tensor(codes)
    nt = torch.from_numpy(n16.astype(np.float16)).cuda()
    for out_dt, bf in ((torch.float32, False), (torch.bfloat16, True)):
        out = pq.dequantize(ct, nt, d, bits, st, out_dtype=out_dt)
        torch.cuda.synchronize()
        parity.check_dequantize(codes, n16, bits, D, out.float().cpu().numpy().astype(np.float64), bf,
                                label="dequant random")


def test_fp16_norm_overflow_is_inf():
    _case("norm overflow")
    d, bits = 128, 4
    x = np.zeros((16, d), dtype=np.float32)
    x[:, :] = 7000.0                      # norm 79195.9 > 65504: fp16 +inf
    x[3, :] = 5000.0                      # norm 56568.5: finite
    st, D = _signs(d, 1)
    codes, norms, _, _ = pq.quantize(torch.from_numpy(x).cuda(), d, bits, st)
    torch.cuda.synchronize()
    nv = parity.f16_values(norms)
    assert np.isinf(nv[0]) and np.isfinite(nv[3])
    parity.check_quantize(x.astype(np.float64), bits, D, codes.cpu().numpy(), nv, label="overflow")


def test_determinism_repeated_calls():
    _case("determinism")
    d, bits, m = 128, 5, 64
    xt, _ = _inputs(16 * 64 + 3, d, "bf16", seed=9)
    st, _ = _signs(d, 2)
    Gt, _ = _proj(m, d, 5)
    a = pq.quantize(xt, d, bits, st, Gt)
    b = pq.quantize(xt, d, bits, st, Gt)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    o1 = pq.dequantize(a[0], a[1], d, bits, st)
    o2 = pq.dequantize(a[0], a[1], d, bits, st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_empty_and_single_block():
    _case("empty / single block")
    d, bits = 128, 4
    st, D = _signs(d, 4)
    empty = torch.empty((0,), dtype=torch.bfloat16, device="cuda")
    c, nn, _, _ = pq.quantize(empty, d, bits, st)
    assert c.shape == (0, d)
    xt, x = _inputs(1, d, "bf16", seed=1, special=False)
    c, nn, _, _ = pq.quantize(xt, d, bits, st)
    torch.cuda.synchronize()
    parity.check_quantize(x, bits, D, c.cpu().numpy(), parity.f16_values(nn), label="single")


@pytest.mark.parametrize("d,dtype,m", [(128, "bf16", 0), (128, "bf16", 64), (256, "bf16", 0), (256, "bf16", 256),
                                        (256, "bf16", 512), (128, "f32", 0), (128, "f32", 64), (512, "bf16", 0),
                                        (512, "bf16", 512), (64, "bf16", 32), (256, "f32", 512)])
def test_extreme_norms(d, dtype, m):
    """Blocks whose norms lie outside [2^-60, 2^61), where a sum of squares in fp32 underflows or
    overflows (the norm is then taken from entries scaled by a power of two; on the matrix cores
    the entries themselves go in scaled), mixed in the same tiles with ordinary ones, with and
    without the QJL stage: the matrix-core rotation (bf16, d = 128 and 256), the butterflies
    (fp32 input, d = 64 and 512), the projection from LDS and the chunked form."""
    _case("extreme norms d=%d %s m=%d" % (d, dtype, m))
    bits, n = 5, 16 * 4 + 5
    rng = np.random.default_rng(31 + d)
    x = rng.standard_normal((n, d)) * 0.02
    x[1] *= 2.0 ** -75                    # norm near 2^-78
    if m == 0:
        # norms past the fp16 range: the QJL residual of such a block is not finite
        x[6] = rng.standard_normal(d) * 2.0 ** 55   # norm near 2^58.5
        x[9] = rng.standard_normal(d) * 2.0 ** 58   # norm near 2^61.5
        if dtype == "f32":
            x[10] = rng.standard_normal(d) * 2.0 ** 66   # a sum of squares beyond fp32
    else:
        x[6] = rng.standard_normal(d) * 2.0 ** 12   # norm near 2^15.5 (finite in fp16)
    x[17] = rng.standard_normal(d) * 1e-39      # subnormal entries (norm near 1e-38)
    x[18, ::3] = 0.0
    x[18] *= 2.0 ** -66
    x[33] *= 2.0 ** 40                    # in range
    x[64] *= 2.0 ** -90                   # ragged last tile
    if dtype == "f32":
        x[20] = rng.standard_normal(d) * 1e-42    # fp32 subnormal entries
        xs = x.astype(np.float32)
        xt = torch.from_numpy(xs).cuda()
        xs = xs.astype(np.float64)
    else:
        u = synth.bf16_from_f32(x.astype(np.float32))
        xt, xs = parity.bf16_tensor(u), numerics.bf16_from_bits(u)
    xs = xs.reshape(n, d)
    st, D = _signs(d, 6)
    if m:
        Gt, G = _proj(m, d, 8)
        codes, norms, qb, rn = pq.quantize(xt, d, bits, st, Gt)
        torch.cuda.synchronize()
        parity.check_quantize(xs, bits, D, codes.cpu().numpy(), parity.f16_values(norms), G, qb.cpu().numpy(),
                              parity.f16_values(rn), label="extreme norms qjl")
    else:
        codes, norms, _, _ = pq.quantize(xt, d, bits, st)
        torch.cuda.synchronize()
        parity.check_quantize(xs, bits, D, codes.cpu().numpy(), parity.f16_values(norms), label="extreme norms")
