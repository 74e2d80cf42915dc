"""GPU parity of the codec with a dense random rotation and the sphere-coordinate codebook
(pq_quantize_dense / pq_dequantize_dense) against the oracle (needs an MI355X).

Codes: equal, except a code whose oracle coordinate lies within 1e-4/sqrt(d) (the codec band on
the N(0,1) scale, carried to the sphere-coordinate scale) of the boundary between the two codes,
at most max(1, 1e-6 n) of them.  Norms: fp16 equal or the neighbouring value near a rounding
midpoint.  Dequantize: the oracle's reconstruction from the GPU's codes and norms, within
2e-5 n16 max|c| (fp32 sums over d terms) for fp32 output and one bf16 ulp for bf16 output."""

import math

import numpy as np
import pytest
import torch

import kv_cache_quantization_amd as pq
import synth
from oracle import dense, numerics
from tests import parity, seeded

pytestmark = pytest.mark.gpu


def _case(label):
    print("\n[case] %s" % label, flush=True)


def _rotation(seed, d):
    """A Haar-distributed rotation drawn as the pages draw it (QR of a seeded Gaussian matrix
    with the sign fix), rounded to fp32: an input of the codec."""
    G = np.random.default_rng(seed).standard_normal((d, d))
    Q, R = np.linalg.qr(G)
    return (Q * np.sign(np.diag(R))[None, :]).astype(np.float32)


CASES = [(64, 3, 1000, True), (128, 4, 777, True), (128, 5, 64, False), (48, 2, 37, True), (16, 1, 1, False),
         (128, 3, 16 * 4096 + 5, True),
         # one block per wave: Pi in LDS (d <= 192), Pi read from global memory (d = 208 .. 512)
         (192, 4, 50, True), (208, 2, 33, False), (256, 3, 301, True), (512, 3, 77, False), (512, 1, 5, True)]


@pytest.mark.parametrize("d,bits,n,bf16", CASES)
def test_dense_codec(d, bits, n, bf16):
    _case("dense rotation d=%d bits=%d n=%d bf16=%d" % (d, bits, n, bf16))
    rng = np.random.default_rng(d * 5 + bits + n)
    xf = (rng.standard_normal((n, d)) * np.exp(0.5 * rng.standard_normal((n, 1)))).astype(np.float32)
    if n > 2:
        xf[1] = 0.0
    Pi = _rotation(d + bits, d)
    if bf16:
        xu = synth.bf16_from_f32(xf)
        xt = parity.bf16_tensor(xu)
        x = synth.bf16_to_f32(xu).astype(np.float64)
    else:
        xt = torch.from_numpy(xf).cuda()
        x = xf.astype(np.float64)
    rot = torch.from_numpy(Pi).cuda()
    codes, norms = pq.quantize_dense(xt, d, bits, rot)
    o32 = pq.dequantize_dense(codes, norms, d, bits, rot, out_dtype=torch.float32)
    o16 = pq.dequantize_dense(codes, norms, d, bits, rot, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    gc = codes.cpu().numpy()
    gn = parity.f16_values(norms)
    P = Pi.astype(np.float64)
    ref = dense.quantize(x, bits, P)
    diff = np.argwhere(gc != ref["codes"])
    beta = ref["beta"]
    for b, i in diff:
        lo = min(int(gc[b, i]), int(ref["codes"][b, i]))
        assert abs(int(gc[b, i]) - int(ref["codes"][b, i])) == 1, "code off by more than one at %s" % ((b, i),)
        assert abs(ref["y"][b, i] - beta[lo]) < 1e-4 / math.sqrt(d), "code differs away from a boundary at %s" % ((b, i),)
    assert len(diff) <= max(1, int(1e-6 * gc.size))
    parity.pick_candidate(gn, parity.fp16_candidates(ref["norm"]), "dense norms")
    refd = dense.dequantize(gc, gn, bits, P)
    cmax = float(np.max(np.abs(dense.beta_codebook(bits, d)[0])))
    err = np.abs(o32.cpu().numpy().astype(np.float64) - refd)
    assert np.all(err <= 2e-5 * gn[:, None] * cmax + 1e-30)
    r16 = numerics.round_bf16(refd)
    ulp = np.ldexp(1.0, np.frexp(np.abs(r16))[1] - 8)
    e16 = np.abs(o16.float().cpu().numpy().astype(np.float64) - r16)
    assert np.all((e16 <= ulp) | (np.abs(o16.float().cpu().numpy() - refd) <= 2e-5 * gn[:, None] * cmax))


@pytest.mark.parametrize("d", [128, 64, 48, 256])
def test_dense_tiny_blocks(d):
    """fp32 blocks whose values sit far below 1 (1e-20, 1e-30, and 1e-41, in fp32's subnormal
    range): the codes follow the rotation of the block's direction, as for unit-scale blocks
    (the kernels scale each block by a power of two before the fp32 products)."""
    _case("dense rotation tiny blocks d=%d" % d)
    bits, n = 3, 96
    rng = np.random.default_rng(d + 77)
    xf = rng.standard_normal((n, d)).astype(np.float32)
    xf[0:32] *= np.float32(1e-20)
    xf[32:64] *= np.float32(1e-30)
    xf[64:96] = (xf[64:96].astype(np.float64) * 1e-41).astype(np.float32)   # subnormal fp32 values
    assert np.all(np.abs(xf[64:96]) < 1.2e-38)
    Pi = _rotation(d + 5, d)
    codes, norms = pq.quantize_dense(torch.from_numpy(xf).cuda(), d, bits, torch.from_numpy(Pi).cuda())
    torch.cuda.synchronize()
    gc = codes.cpu().numpy()
    ref = dense.quantize(xf.astype(np.float64), bits, Pi.astype(np.float64))
    diff = np.argwhere(gc != ref["codes"])
    for b, i in diff:
        lo = min(int(gc[b, i]), int(ref["codes"][b, i]))
        assert abs(int(gc[b, i]) - int(ref["codes"][b, i])) == 1, "code off by more than one at %s" % ((b, i),)
        # subnormal inputs carry fewer significant bits: their blocks get a wider band
        band = 1e-4 if b < 64 else 1e-2
        assert abs(ref["y"][b, i] - ref["beta"][lo]) < band / math.sqrt(d), "code differs away from a boundary at %s" % ((b, i),)
    assert len(diff) <= max(1, int(1e-6 * gc.size)) + int(np.sum(diff[:, 0] >= 64))
    assert np.all(parity.f16_values(norms) == 0.0)          # below fp16's range


def _bf16_grid(e_lo, e_hi):
    """Every positive bf16 value in [2^e_lo, 2^e_hi)."""
    return np.array([(1.0 + m / 128.0) * 2.0 ** e for e in range(e_lo, e_hi) for m in range(128)])


@pytest.mark.parametrize("d", [128, 64])
def test_dense_bf16_codes_near_boundaries(d):
    """bf16 blocks built so that many rotated coordinates sit between 1e-7 and 1e-4 of a boundary
    (Pi a signed permutation, a block holds c values +-p and d - c values +-q with p / ||x|| next
    to a boundary): hundreds of codes per 16-block tile are decided again in fp64, the queue of
    each wave fills and drains several times per tile, and every code equals the oracle's (its y
    and the kernel's fp64 y are the same correctly rounded quotient here)."""
    _case("dense rotation bf16 codes near boundaries d=%d" % d)
    bits = 3
    rng = np.random.default_rng(d + 901)
    _, beta, _ = dense.beta_codebook(bits, d)
    P = _bf16_grid(0, 1)
    Q = _bf16_grid(-4, 2)
    picks = []
    for bk in beta[beta > 0]:
        for c in (d // 2, d // 4, d // 8):                  # fewer p values reach larger ratios
            ratio = P[:, None] / np.sqrt(c * P[:, None] ** 2 + (d - c) * Q[None, :] ** 2)
            dist = np.abs(ratio - bk)
            ii, jj = np.nonzero((dist > 1e-7) & (dist < 1e-4))
            if ii.size >= 16:
                break
        assert ii.size >= 16, "no bf16 pair lands next to boundary %r" % bk
        sel = rng.choice(ii.size, 16, replace=False)
        picks += [(P[ii[s]], Q[jj[s]], c) for s in sel]
    n = len(picks) * 2 + 5                                  # ragged last tile
    x = np.zeros((n, d))
    for b in range(n):
        p, q, c = picks[b % len(picks)]
        row = np.concatenate([np.full(c, p), np.full(d - c, q)]) * rng.choice([-1.0, 1.0], d)
        x[b] = row[rng.permutation(d)]
    xu = synth.bf16_from_f32(x.astype(np.float32))
    assert np.array_equal(synth.bf16_to_f32(xu).astype(np.float64), x)
    Pi = np.zeros((d, d), np.float32)
    Pi[np.arange(d), rng.permutation(d)] = rng.choice([-1.0, 1.0], d)
    codes, norms = pq.quantize_dense(parity.bf16_tensor(xu), d, bits, torch.from_numpy(Pi).cuda())
    torch.cuda.synchronize()
    ref = dense.quantize(x, bits, Pi.astype(np.float64))
    near = np.min(np.abs(ref["y"][:, :, None] - beta[None, None, :]), axis=2) < 1e-4
    assert near.sum() >= n * d // 8
    gc = codes.cpu().numpy()
    bad = np.argwhere(gc != ref["codes"])
    assert bad.size == 0, "%d codes differ, first at %s" % (len(bad), bad[0])
    parity.pick_candidate(parity.f16_values(norms), parity.fp16_candidates(ref["norm"]), "dense norms")


@pytest.mark.parametrize("d", [128, 64])
def test_dense_bf16_extreme_blocks(d):
    """bf16 blocks scaled by 2^-100 (squares below fp32's range), 2^125 (sum of squares above
    it, norm beyond fp16's), all-zero blocks and unit-scale ones: every code equals the oracle's
    (the kernel takes such blocks' norms in fp64 and scales them by a power of two before the
    bf16 products), norms are 0, inf or the oracle's fp16 rounding."""
    _case("dense rotation bf16 extreme blocks d=%d" % d)
    bits, n = 3, 16 * 10 + 3
    rng = np.random.default_rng(d + 555)
    xf = rng.standard_normal((n, d)).astype(np.float32)
    xu = synth.bf16_from_f32(xf)
    x = synth.bf16_to_f32(xu).astype(np.float64)
    x[0:40] *= 2.0 ** -100
    x[40:80] *= 2.0 ** 125
    x[80:100] = 0.0
    xu = synth.bf16_from_f32(x.astype(np.float32))
    assert np.array_equal(synth.bf16_to_f32(xu).astype(np.float64), x)
    Pi = _rotation(d + 17, d)
    codes, norms = pq.quantize_dense(parity.bf16_tensor(xu), d, bits, torch.from_numpy(Pi).cuda())
    torch.cuda.synchronize()
    ref = dense.quantize(x, bits, Pi.astype(np.float64))
    gc = codes.cpu().numpy()
    bad = np.argwhere(gc != ref["codes"])
    assert bad.size == 0, "%d codes differ, first at %s" % (len(bad), bad[0])
    gn = parity.f16_values(norms)
    assert np.all(gn[0:40] == 0.0) and np.all(np.isinf(gn[40:80])) and np.all(gn[80:100] == 0.0)
    parity.pick_candidate(gn[100:], parity.fp16_candidates(ref["norm"][100:]), "dense norms")


@pytest.mark.parametrize("d", [128, 64])
def test_dense_unaligned_buffers(d):
    """bf16 input and fp32 output 4 bytes off 16-byte alignment take the fp32 matrix-core kernels:
    their codes are the oracle's fp64 decisions as the aligned run's are, norms are the oracle's
    fp16 rounding, and both reconstructions meet the fp32 bound against the oracle."""
    _case("dense rotation unaligned buffers d=%d" % d)
    bits, n = 3, 16 * 9 + 7
    rng = np.random.default_rng(d + 313)
    xu = synth.bf16_from_f32(rng.standard_normal((n, d)).astype(np.float32))
    x = synth.bf16_to_f32(xu).astype(np.float64)
    whole = parity.bf16_tensor(np.concatenate([np.zeros(2, np.uint16), xu.reshape(-1)]))
    x_off = whole[2:].view(n, d)                           # data 4 bytes past a 16-byte boundary
    assert x_off.data_ptr() % 16 != 0
    Pi = _rotation(d + 29, d)
    rot = torch.from_numpy(Pi).cuda()
    codes_a, norms_a = pq.quantize_dense(parity.bf16_tensor(xu), d, bits, rot)
    codes_u, norms_u = pq.quantize_dense(x_off, d, bits, rot)
    out_big = torch.empty(n * d + 1, dtype=torch.float32, device="cuda")
    out_off = out_big[1:].view(n, d)
    assert out_off.data_ptr() % 16 != 0
    o_u = pq.dequantize_dense(codes_a, norms_a, d, bits, rot, out_dtype=torch.float32, out=out_off)
    o_a = pq.dequantize_dense(codes_a, norms_a, d, bits, rot, out_dtype=torch.float32)
    torch.cuda.synchronize()
    P = Pi.astype(np.float64)
    ref = dense.quantize(x, bits, P)
    for codes, norms, what in ((codes_a, norms_a, "aligned"), (codes_u, norms_u, "unaligned")):
        gc = codes.cpu().numpy()
        bad = np.argwhere(gc != ref["codes"])
        assert bad.size == 0, "%s: %d codes differ, first at %s" % (what, len(bad), bad[0])
        parity.pick_candidate(parity.f16_values(norms), parity.fp16_candidates(ref["norm"]), "dense norms " + what)
    gn = parity.f16_values(norms_a)
    refd = dense.dequantize(codes_a.cpu().numpy(), gn, bits, P)
    cmax = float(np.max(np.abs(dense.beta_codebook(bits, d)[0])))
    for o, what in ((o_a, "aligned"), (o_u, "unaligned")):
        err = np.abs(o.cpu().numpy().astype(np.float64) - refd)
        assert np.all(err <= 2e-5 * gn[:, None] * cmax + 1e-30), what
