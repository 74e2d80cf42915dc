"""The Python binding rejects caller buffers of the wrong dtype, device or size before any
launch (the C ABI receives raw pointers and cannot see a short buffer).  Needs a GPU for the
device tensors; no kernel is launched by any case here."""

import pytest
import torch

import kv_cache_quantization_amd as pq

pytestmark = pytest.mark.gpu

D, BITS, M = 128, 4, 64


def _t(n, dtype):
    return torch.zeros((n,), dtype=dtype, device="cuda")


def _qargs():
    n = 32
    return dict(x=_t(n * D, torch.bfloat16), signs=_t(D // 8, torch.uint8), proj=_t(M * D, torch.bfloat16).view(M, D),
                out=(_t(n * D, torch.uint8), _t(n, torch.float16), _t(n * M // 8, torch.uint8), _t(n, torch.float16)))


@pytest.mark.parametrize("bad", ["codes", "norms", "qjl_bits", "rnorms", "signs", "proj", "dtype"])
def test_quantize_rejects(bad):
    a = _qargs()
    codes, norms, qb, rn = a["out"]
    if bad == "codes":
        codes = codes[:-1]
    elif bad == "norms":
        norms = norms[:-1]
    elif bad == "qjl_bits":
        qb = qb[:-8]
    elif bad == "rnorms":
        rn = _t(31, torch.float16)
    elif bad == "signs":
        a["signs"] = _t(D // 16, torch.uint8)
    elif bad == "proj":
        a["proj"] = _t(M * D, torch.bfloat16).view(M * 2, D // 2)
    elif bad == "dtype":
        norms = _t(32, torch.float32)
    with pytest.raises((ValueError, TypeError)):
        pq.quantize(a["x"], D, BITS, a["signs"], a["proj"], out=(codes, norms, qb, rn))


def test_dequantize_rejects():
    n = 32
    codes, norms, signs = _t(n * D, torch.uint8), _t(n, torch.float16), _t(D // 8, torch.uint8)
    with pytest.raises(ValueError):
        pq.dequantize(codes[:-16], norms, D, BITS, signs)
    with pytest.raises(ValueError):
        pq.dequantize(codes, norms, D, BITS, signs, out=_t(n * D - 1, torch.bfloat16))
    with pytest.raises(ValueError):
        pq.dequantize(codes, norms, D, BITS, _t(D // 8 + 1, torch.uint8))


def test_sketch_score_reject():
    n, m = 48, 256
    keys, proj = _t(n * D, torch.bfloat16), _t(m * D, torch.bfloat16).view(m, D)
    with pytest.raises(ValueError):
        pq.qjl_sketch(keys, proj, out=(_t(n * m // 8 - 1, torch.uint8), _t(n, torch.float16)))
    with pytest.raises(ValueError):
        pq.qjl_sketch(keys, proj, out=(_t(n * m // 8, torch.uint8), _t(n - 1, torch.float16)))
    B, Hkv, Hq, T = 1, 2, 8, 24
    sq = _t(B * Hq * m, torch.float32).view(B * Hq, m)
    bits, norms = _t(B * Hkv * T * m // 8, torch.uint8), _t(B * Hkv * T, torch.float16)
    with pytest.raises(ValueError):
        pq.qjl_score(sq, bits[:-1], norms, B, Hkv, Hq, T)
    with pytest.raises(ValueError):
        pq.qjl_score(sq, bits, norms[:-1], B, Hkv, Hq, T)
    with pytest.raises(ValueError):
        pq.qjl_score(sq, bits, norms, B, Hkv, Hq, T, out=_t(B * Hq * T - 1, torch.float32))
    with pytest.raises(ValueError):
        pq.qjl_score(sq, bits, norms, B, Hkv, Hq + 4, T)


def test_score_and_attention_reject():
    H, n_q, T, bits = 2, 4, 40, 3
    q = _t(H * n_q * D, torch.bfloat16).view(H, n_q, D)
    signs = _t(D // 8, torch.uint8)
    prep = pq.query_prep(q, signs)
    codes, norms = _t(H * T * D, torch.uint8), _t(H * T, torch.float16)
    with pytest.raises(ValueError):
        pq.score(prep[:-4], codes, norms, D, bits, H, n_q, T)
    with pytest.raises(ValueError):
        pq.score(prep, codes, norms[:-1], D, bits, H, n_q, T)
    with pytest.raises(ValueError):
        pq.score(prep, codes, norms, D, bits, H, n_q, T, out=_t(H * n_q * T - 1, torch.float32))
    keys, vals = (codes, norms, None, None), (codes, norms)
    with pytest.raises(ValueError):
        pq.attention(prep, keys, (codes, norms[:-1]), signs, D, bits, H, n_q, T)
    with pytest.raises(ValueError):
        pq.attention(prep, keys, vals, signs, D, bits, H, n_q, T, work=_t(16, torch.uint8))
    with pytest.raises(ValueError):
        pq.attention_noalloc(prep, keys, vals, signs, D, bits, H, n_q, T, out=_t(H * n_q * D - 1, torch.float32))
    with pytest.raises(ValueError):
        pq.query_prep(q, signs, out=_t(16, torch.uint8))


@pytest.mark.parametrize("n", [1, 15, 16 * 1023 + 7, 16 * 4096 * 9 + 3])
def test_probe_stream_widens_every_byte(n):
    """The bandwidth probe writes every byte zero-extended to 16 bits, ragged tails included."""
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    out = torch.full((n + 8,), -1, dtype=torch.int16, device="cuda")
    pq.probe_stream(src, out=out[:n])
    torch.cuda.synchronize()
    assert torch.equal(out[:n], src.to(torch.int16))
    assert torch.all(out[n:] == -1)                         # nothing past the end
