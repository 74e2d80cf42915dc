"""GPU parity of the codec with the block-diagonal rotation (pq_quantize_bd / pq_dequantize_bd),
for block sizes that are not powers of two, against the oracle (needs an MI355X)."""

import numpy as np
import pytest
import torch

import kv_cache_quantization_amd as pq
import synth
from oracle import hadamard
from tests import parity, seeded

pytestmark = pytest.mark.gpu


def _case(label):
    print("\n[case] %s" % label, flush=True)


CASES = [
    # d, bits, n_blocks, bf16 input
    (96, 4, 37, True),
    (192, 3, 1000, True),
    (320, 5, 257, False),
    (576, 2, 64, True),
    (2688, 4, 19, True),        # the pages' example split, 2048 + 512 + 128
    (4064, 8, 5, False),        # seven parts, 2048 down to 32
    (256, 4, 100, True),        # a power of two: one part
    (160, 1, 1, True),
]


@pytest.mark.parametrize("d,bits,n,bf16", CASES)
def test_blockdiag_codec(d, bits, n, bf16):
    _case("block-diagonal d=%d bits=%d n=%d bf16=%d" % (d, bits, n, bf16))
    rng = np.random.default_rng(d + bits + n)
    xf = (rng.standard_normal((n, d)) * np.exp(0.5 * rng.standard_normal((n, 1)))).astype(np.float32)
    xf[0, : d // 3] *= 8.0                                  # an uneven block: energy in the first parts
    if n > 2:
        xf[1] = 0.0                                         # a zero block
    D = seeded.oracle_D(d + 7, d)
    if bf16:
        xu = synth.bf16_from_f32(xf)
        xt = parity.bf16_tensor(xu)
        x = synth.bf16_to_f32(xu).astype(np.float64)
    else:
        xt = torch.from_numpy(xf).cuda()
        x = xf.astype(np.float64)
    st = seeded.gpu_signs(d + 7, d)
    codes, norms = pq.quantize_bd(xt, d, bits, st)
    out32 = pq.dequantize_bd(codes, norms, d, bits, st, out_dtype=torch.float32)
    out16 = pq.dequantize_bd(codes, norms, d, bits, st, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    gc = codes.cpu().numpy()
    gn = parity.f16_values(norms)
    parity.check_quantize(x, bits, D, gc, gn, label="bd d=%d" % d)
    parity.check_dequantize(gc, gn, bits, D, out32.cpu().numpy().astype(np.float64), False, label="bd fp32 d=%d" % d)
    parity.check_dequantize(gc, gn, bits, D, out16.float().cpu().numpy().astype(np.float64), True,
                            label="bd bf16 d=%d" % d)


def test_blockdiag_weight_2688_sampled():
    """A 16384 x 2688 bf16 weight (the pages' 2688 example as the block size), one call as the
    benchmark makes it; the oracle checks sampled rows."""
    d, bits, rows = 2688, 4, 16384
    _case("block-diagonal weight %dx%d" % (rows, d))
    c, _ = synth.weight_with_outlier_entries(5, rows, d)
    st = seeded.gpu_signs(synth.BASE_SEED + d, d)
    codes, norms = pq.quantize_bd(parity.bf16_tensor(c), d, bits, st)
    out = pq.dequantize_bd(codes, norms, d, bits, st)
    torch.cuda.synchronize()
    idx = np.unique(np.concatenate([np.arange(32), np.arange(rows - 32, rows),
                                    np.random.default_rng(3).integers(0, rows, 96)]))
    x = synth.bf16_to_f32(c[idx]).astype(np.float64)
    D = seeded.oracle_D(synth.BASE_SEED + d, d)
    gc = codes.cpu().numpy()[idx]
    gn = parity.f16_values(norms)[idx]
    parity.check_quantize(x, bits, D, gc, gn, label="bd weight")
    parity.check_dequantize(gc, gn, bits, D, out.float().cpu().numpy().astype(np.float64)[idx], True,
                            label="bd weight bf16")
