"""GPU parity of pq_quantize_packed / pq_dequantize_packed against the oracle (needs an
MI355X).  Codes bit-packed into bytes (eliza quantization README, TurboQuant, "Algorithm in
one paragraph", step 4) at every width 1..8: the packed bytes are unpacked with the oracle's
own unpacker and held to the same rule as byte codes."""

import numpy as np
import pytest
import torch

import kv_cache_quantization_amd as pq
import synth
from oracle import codec, numerics
from tests import parity, seeded
from tests.test_gpu_codec import _case, _inputs, _proj, _signs

pytestmark = pytest.mark.gpu

PACKED_CASES = [
    # d, bits, dtype, n_blocks, m
    (128, 4, "bf16", 16 * 20 + 11, 0),
    (128, 4, "f32", 16 * 9 + 1, 64),
    (128, 2, "bf16", 16 * 7 + 5, 128),
    (128, 1, "bf16", 16 * 4 + 3, 0),
    (128, 8, "bf16", 16 * 3 + 13, 0),
    (64, 4, "bf16", 16 * 6 + 7, 32),
    (64, 2, "f32", 16 * 5, 0),
    (64, 1, "bf16", 16 * 3 + 9, 0),
    (256, 4, "bf16", 16 * 6 + 2, 256),
    (256, 2, "f32", 16 * 4 + 15, 0),
    (512, 4, "bf16", 16 * 4 + 9, 512),          # projection walked from L2
    (512, 1, "f32", 16 * 2 + 1, 0),
    # widths that do not divide a byte: codes straddle bytes and dwords
    (128, 5, "bf16", 16 * 9 + 5, 64),
    (128, 3, "f32", 16 * 4 + 1, 0),
    (64, 3, "bf16", 16 * 5 + 3, 0),             # 6-byte runs per lane (16-bit accesses)
    (64, 7, "bf16", 16 * 2 + 9, 16),
    (256, 3, "bf16", 16 * 4 + 7, 256),
    (256, 6, "f32", 16 * 3, 0),
    (512, 3, "bf16", 16 * 2 + 5, 512),
    (512, 5, "bf16", 16 * 2 + 11, 0),
]


@pytest.mark.parametrize("d,bits,dtype,n,m", PACKED_CASES)
def test_packed_quantize_dequantize(d, bits, dtype, n, m):
    _case("packed d=%d bits=%d %s n=%d m=%d" % (d, bits, dtype, n, m))
    xt, x = _inputs(n, d, dtype, seed=d * 31 + bits)
    st, D = _signs(d, seed=d + 7 * bits)
    Gt, G = _proj(m, d, seed=m + 3 * d) if m else (None, None)
    packed, norms, qb, rn = pq.quantize(xt, d, bits, st, Gt, packed=True)
    codes, norms1, qb1, rn1 = pq.quantize(xt, d, bits, st, Gt)
    torch.cuda.synchronize()
    pk = packed.cpu().numpy()
    assert pk.shape == (n, d * bits // 8)
    # the same decisions as the byte-code entry point, packed as the oracle packs them
    assert np.array_equal(pk, codec.pack_codes(codes.cpu().numpy(), bits))
    assert torch.equal(norms, norms1)
    if m:
        assert torch.equal(qb, qb1) and torch.equal(rn, rn1)
    # and against the oracle directly, through the oracle's unpacker
    gc = codec.unpack_codes(pk, bits, d)
    parity.check_quantize(x, bits, D, gc, parity.f16_values(norms), G,
                          qb.cpu().numpy() if m else None, parity.f16_values(rn) if m else None,
                          label="packed quantize d=%d b=%d" % (d, bits))
    for out_dt, bf in ((torch.float32, False), (torch.bfloat16, True)):
        out = pq.dequantize(packed, norms, d, bits, st, out_dtype=out_dt, packed=True)
        ref = pq.dequantize(codes, norms, d, bits, st, out_dtype=out_dt)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        parity.check_dequantize(gc, parity.f16_values(norms), bits, D,
                                out.float().cpu().numpy().astype(np.float64), bf, label="packed dequant")


@pytest.mark.parametrize("d,bits", [(64, 1), (128, 2), (256, 4), (512, 4), (128, 8), (64, 5), (128, 3),
                                    (256, 7), (512, 6)])
def test_packed_dequantize_oracle_codes(d, bits):
    """Codes drawn and packed on the oracle side, dequantized from the packed bytes."""
    _case("packed dequantize oracle codes d=%d bits=%d" % (d, bits))
    rng = np.random.default_rng(d * 5 + bits)
    n = 16 * 9 + 5
    codes = rng.integers(0, 1 << bits, size=(n, d))
    n16 = numerics.round_fp16(np.exp(rng.uniform(-6, 6, size=n)))
    n16[0] = 0.0
    st, D = _signs(d, seed=11)
    pk = parity.u8_tensor(codec.pack_codes(codes, bits))
    nt = torch.from_numpy(n16.astype(np.float16)).cuda()
    for out_dt, bf in ((torch.float32, False), (torch.bfloat16, True)):
        out = pq.dequantize(pk, nt, d, bits, st, out_dtype=out_dt, packed=True)
        torch.cuda.synchronize()
        parity.check_dequantize(codes.astype(np.uint8), n16, bits, D, out.float().cpu().numpy().astype(np.float64),
                                bf, label="packed dequant oracle codes")


def test_packed_config3_tensor_sampled():
    """A full-size config-3 tensor (gate, 14336 x 4096 bf16) at 4 bits, packed two codes per
    byte: sampled blocks against the oracle, every block against the byte-code path."""
    layout = synth.config3_layout()
    _, layer, name, rows, cols = layout[4]
    _case("packed config3 tensor 4 (%s %dx%d), d=128, 4-bit" % (name, rows, cols))
    xu, sseed = synth.config3_tensor(4, rows, cols)
    d, bits = 128, 4
    x = parity.bf16_tensor(xu)
    st = seeded.gpu_signs(sseed, d)
    packed, norms, _, _ = pq.quantize(x, d, bits, st, packed=True)
    codes, _, _, _ = pq.quantize(x, d, bits, st)
    out = pq.dequantize(packed, norms, d, bits, st, packed=True)
    ref = pq.dequantize(codes, norms, d, bits, st)
    torch.cuda.synchronize()
    n = codes.shape[0]
    # the byte codes packed on the device side by the reference packing of nibbles
    lo = codes[:, 0::2].to(torch.int32)
    hi = codes[:, 1::2].to(torch.int32)
    assert torch.equal(packed.to(torch.int32), lo | (hi << 4))
    assert torch.equal(out, ref)
    idx = np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n),
                                    np.random.default_rng(77).integers(0, n, 1500)]))
    sel = torch.from_numpy(idx).cuda()
    xs = numerics.bf16_from_bits(xu.reshape(-1, d)[idx])
    D = seeded.oracle_D(sseed, d)
    gc = codec.unpack_codes(packed[sel].cpu().numpy(), bits, d)
    parity.check_quantize(xs, bits, D, gc, parity.f16_values(norms[sel]), label="packed config3")
    parity.check_dequantize(gc, parity.f16_values(norms[sel]), bits, D,
                            out[sel].float().cpu().numpy().astype(np.float64), True, label="packed config3 dq")
