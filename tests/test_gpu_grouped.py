"""GPU parity of the grouped codec (pq_quantize_many / pq_dequantize_many): many tensors in one
launch give exactly the outputs of one pq_quantize / pq_dequantize call per tensor, and the
oracle checks sampled blocks; config 3's layer-0 tensors (q, k, v, o, gate, up, down) as one
grouped pass.  Needs an MI355X."""

import numpy as np
import pytest
import torch

import kv_cache_quantization_amd as pq
import synth
from oracle import codec, numerics
from tests import parity, seeded

pytestmark = pytest.mark.gpu


def _case(label):
    print("\n[case] %s" % label, flush=True)


# block counts: empty, single block, ragged tails, several full tiles
SIZES = [37, 0, 1, 16, 16 * 9 + 5, 15, 16 * 40, 16 * 3 + 1]


@pytest.mark.parametrize("d,bits,dtype,packed", [(128, 4, "bf16", False), (128, 3, "bf16", True),
                                                 (64, 2, "f32", False), (256, 5, "bf16", True),
                                                 (512, 3, "bf16", False), (128, 8, "f32", True)])
def test_grouped_equals_single_calls(d, bits, dtype, packed):
    _case("grouped d=%d bits=%d %s packed=%d tensors=%d" % (d, bits, dtype, packed, len(SIZES)))
    rng = np.random.default_rng(d + bits)
    xs, xs64, sts, Ds = [], [], [], []
    for i, n in enumerate(SIZES):
        x = (rng.standard_normal((n, d)) * np.exp(rng.standard_normal((n, 1)))).astype(np.float32)
        if n > 3:
            x[2] = 0.0                                   # a zero block
        if dtype == "bf16":
            u = synth.bf16_from_f32(x)
            xs.append(parity.bf16_tensor(u))
            xs64.append(numerics.bf16_from_bits(u).reshape(n, d))
        else:
            xs.append(torch.from_numpy(x).cuda())
            xs64.append(x.astype(np.float64))
        sts.append(seeded.gpu_signs(100 + i, d))
        Ds.append(seeded.oracle_D(100 + i, d))
    grouped = pq.quantize_many(xs, d, bits, sts, packed=packed)
    singles = [pq.quantize(x, d, bits, st, packed=packed)[:2] for x, st in zip(xs, sts)]
    codes = [c for c, _ in grouped]
    norms = [nm for _, nm in grouped]
    outs = pq.dequantize_many(codes, norms, d, bits, sts, packed=packed,
                              out_dtype=torch.float32 if dtype == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    for i, ((gc, gn), (sc, sn)) in enumerate(zip(grouped, singles)):
        assert torch.equal(gc, sc) and torch.equal(gn, sn), "tensor %d" % i
        ref = pq.dequantize(sc, sn, d, bits, sts[i], packed=packed, out_dtype=outs[i].dtype)
        torch.cuda.synchronize()
        assert torch.equal(outs[i], ref), "tensor %d dequantize" % i
    # the oracle on the first and the largest tensors
    for i in (0, int(np.argmax(SIZES))):
        gc = codes[i].cpu().numpy()
        if packed:
            gc = codec.unpack_codes(gc, bits, d)
        n16 = parity.f16_values(norms[i])
        parity.check_quantize(xs64[i], bits, Ds[i], gc, n16, label="grouped t%d" % i)
        parity.check_dequantize(gc, n16, bits, Ds[i], outs[i].float().cpu().numpy().astype(np.float64),
                                dtype == "bf16", label="grouped t%d dq" % i)


def test_grouped_config3_layer0():
    """Config 3's first layer (seven tensors, 128 Mi bf16 values) as one grouped quantize pass and
    one grouped dequantize pass: identical to the per-tensor calls."""
    _case("grouped config3 layer 0 (7 tensors)")
    d, bits = 128, 4
    xs, sts = [], []
    for t, _, name, rows, cols in synth.config3_layout(1):
        xu, sseed = synth.config3_tensor(t, rows, cols)
        xs.append(parity.bf16_tensor(xu))
        sts.append(seeded.gpu_signs(sseed, d))
    grouped = pq.quantize_many(xs, d, bits, sts)
    outs = pq.dequantize_many([c for c, _ in grouped], [n for _, n in grouped], d, bits, sts)
    for i, (x, st) in enumerate(zip(xs, sts)):
        c, n, _, _ = pq.quantize(x, d, bits, st)
        torch.cuda.synchronize()
        assert torch.equal(c, grouped[i][0]) and torch.equal(n, grouped[i][1]), "tensor %d" % i
        assert torch.equal(pq.dequantize(c, n, d, bits, st), outs[i]), "tensor %d dequantize" % i


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (256, "bf16"), (128, "f32")])
def test_grouped_extreme_norms(d, dtype):
    """Tensors of blocks whose norms leave [2^-60, 2^61) (tiny, subnormal entries, huge) in one
    grouped launch beside an ordinary tensor: the oracle's codes, and the single calls' bytes."""
    _case("grouped extreme norms d=%d %s" % (d, dtype))
    bits = 4
    rng = np.random.default_rng(7 + d)
    xs, xs64, sts, Ds = [], [], [], []
    for i, n in enumerate((16 * 3 + 5, 16 * 2)):
        x = rng.standard_normal((n, d)) * 0.02
        if i == 0:
            x[0] *= 2.0 ** -80
            x[3] = rng.standard_normal(d) * 1e-39
            x[7] = rng.standard_normal(d) * 2.0 ** 58
            x[20] *= 2.0 ** -66
            x[n - 1] *= 2.0 ** -100
        x = x.astype(np.float32)
        if dtype == "bf16":
            u = synth.bf16_from_f32(x)
            xs.append(parity.bf16_tensor(u))
            xs64.append(numerics.bf16_from_bits(u).reshape(n, d))
        else:
            xs.append(torch.from_numpy(x).cuda())
            xs64.append(x.astype(np.float64))
        sts.append(seeded.gpu_signs(20 + i, d))
        Ds.append(seeded.oracle_D(20 + i, d))
    grouped = pq.quantize_many(xs, d, bits, sts)
    torch.cuda.synchronize()
    for i in range(len(xs)):
        c, nm, _, _ = pq.quantize(xs[i], d, bits, sts[i])
        torch.cuda.synchronize()
        assert torch.equal(c, grouped[i][0]) and torch.equal(nm, grouped[i][1]), "tensor %d" % i
        parity.check_quantize(xs64[i], bits, Ds[i], grouped[i][0].cpu().numpy(), parity.f16_values(grouped[i][1]),
                              label="grouped extreme t%d" % i)
