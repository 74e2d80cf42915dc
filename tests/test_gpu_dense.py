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
from tests import parity

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
         (128, 3, 16 * 4096 + 5, True)]


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
