"""Bit-exact determinism across launch geometries (glq 0.7.2 README, "Inference kernels": the
kernels give bit-identical results run to run).  The same blocks quantized and dequantized in
one call, in two calls split at a block that is not a tile boundary (every block of the second
part lands in another tile row and another wave), and through the grouped call (another work
split over the grid) give identical codes, norms, residual bits and outputs.  Needs an MI355X."""

import numpy as np
import pytest
import torch

import kv_cache_quantization_amd as pq
import synth
from tests import parity, seeded

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,bits,m", [(128, 5, 64), (256, 3, 256), (512, 3, 512), (64, 4, 0), (128, 4, 0),
                                      (256, 5, 0)])
def test_split_and_grouped_calls_agree(d, bits, m):
    print("\n[case] determinism d=%d bits=%d m=%d" % (d, bits, m), flush=True)
    n, k = 16 * 97 + 11, 16 * 41 + 7                      # k: split inside a tile
    rng = np.random.default_rng(d + m)
    x = parity.bf16_tensor(synth.bf16_from_f32((rng.standard_normal((n, d)) * 0.02).astype(np.float32)))
    st = seeded.gpu_signs(7, d)
    G = seeded.gpu_proj(9, m, d) if m else None
    full = pq.quantize(x, d, bits, st, G)
    a = pq.quantize(x[:k].contiguous(), d, bits, st, G)
    b = pq.quantize(x[k:].contiguous(), d, bits, st, G)
    again = pq.quantize(x, d, bits, st, G)
    out = pq.dequantize(full[0], full[1], d, bits, st)
    oa = pq.dequantize(full[0][:k].contiguous(), full[1][:k].contiguous(), d, bits, st)
    ob = pq.dequantize(full[0][k:].contiguous(), full[1][k:].contiguous(), d, bits, st)
    torch.cuda.synchronize()
    for i, name in enumerate(("codes", "norms", "qjl_bits", "rnorms")):
        if full[i] is None:
            continue
        assert torch.equal(torch.cat([a[i], b[i]]), full[i]), name
        assert torch.equal(again[i], full[i]), name
    assert torch.equal(torch.cat([oa, ob]), out)
    if m == 0:
        # the grouped call over the two parts and the whole tensor, in one launch
        g = pq.quantize_many([x[:k].contiguous(), x[k:].contiguous(), x], d, bits, [st, st, st])
        go = pq.dequantize_many([c for c, _ in g], [nm for _, nm in g], d, bits, [st, st, st])
        torch.cuda.synchronize()
        assert torch.equal(torch.cat([g[0][0], g[1][0]]), full[0]) and torch.equal(g[2][0], full[0])
        assert torch.equal(torch.cat([g[0][1], g[1][1]]), full[1]) and torch.equal(g[2][1], full[1])
        assert torch.equal(torch.cat([go[0], go[1]]), out) and torch.equal(go[2], out)


@pytest.mark.parametrize("d,dtype,m", [(128, "bf16", 64), (256, "bf16", 256), (512, "bf16", 512), (128, "f32", 64),
                                       (64, "bf16", 32)])
def test_residual_stage_leaves_codes_alone(d, dtype, m):
    """The codes and norms of a call with the QJL residual stage equal those of the same call
    without it (the stage only adds the residual's signs and norm; the kernels that carry it take
    the codes by the same arithmetic)."""
    print("\n[case] codes with and without QJL d=%d %s m=%d" % (d, dtype, m), flush=True)
    n, bits = 16 * 53 + 9, 4
    rng = np.random.default_rng(3 * d + m)
    x = (rng.standard_normal((n, d)) * np.exp(rng.standard_normal((n, 1)))).astype(np.float32)
    xt = torch.from_numpy(x).cuda() if dtype == "f32" else parity.bf16_tensor(synth.bf16_from_f32(x))
    st = seeded.gpu_signs(11, d)
    G = seeded.gpu_proj(13, m, d)
    with_q = pq.quantize(xt, d, bits, st, G)
    without = pq.quantize(xt, d, bits, st)
    torch.cuda.synchronize()
    assert torch.equal(with_q[0], without[0])
    assert torch.equal(with_q[1], without[1])
