"""pq_attention_noalloc, the decode attention that allocates nothing (its work buffer is the
library's fixed device array), against pq_attention with a caller-owned work buffer: identical
outputs, on two calls in a row, the second with a smaller input (needs an MI355X)."""

import math

import numpy as np
import pytest
import torch

import kv_cache_quantization_amd as pq
import synth
from oracle import codec, numerics
from tests import seeded

pytestmark = pytest.mark.gpu


def _inputs(rng, d, bits, m, n_heads, n_q, n_tok, n_win, packed):
    kc = rng.integers(0, 1 << bits, size=(n_heads, n_tok, d), dtype=np.uint8)
    vc = rng.integers(0, 1 << bits, size=(n_heads, n_tok, d), dtype=np.uint8)
    kn = numerics.round_fp16(np.exp(rng.uniform(-1, 2, size=(n_heads, n_tok))))
    vn = numerics.round_fp16(np.exp(rng.uniform(-1, 2, size=(n_heads, n_tok))))
    qb = rng.integers(0, 256, size=(n_heads, n_tok, m // 8), dtype=np.uint8)
    rn = numerics.round_fp16(kn * rng.uniform(0.0, 0.3, size=(n_heads, n_tok)))
    qu = synth.bf16_from_f32(rng.standard_normal((n_heads, n_q, d)).astype(np.float32))
    kw = synth.bf16_from_f32(rng.standard_normal((n_heads, n_win, d)).astype(np.float32))
    vw = synth.bf16_from_f32(rng.standard_normal((n_heads, n_win, d)).astype(np.float32))
    if packed:
        kc = codec.pack_codes(kc.reshape(-1, d), bits)
        vc = codec.pack_codes(vc.reshape(-1, d), bits)
    dev = "cuda"
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    f16 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float16)).to(dev)
    b16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    keys = (u8(kc), f16(kn), u8(qb) if m else None, f16(rn) if m else None)
    return keys, (u8(vc), f16(vn)), b16(qu), (b16(kw), b16(vw)) if n_win else (None, None)


@pytest.mark.parametrize("d,bits,m,packed", [(128, 4, 0, False), (256, 3, 256, False), (512, 3, 512, True)])
def test_noalloc_matches_attention_twice(d, bits, m, packed):
    rng = np.random.default_rng(d + bits + m)
    n_q = 16
    k_seed, v_seed, g_seed = d + 3, d + 4, d + 5
    v_signs = seeded.gpu_signs(v_seed, d)
    G = seeded.gpu_proj(g_seed, m, d) if m else None
    # the first call at the config-5 attention shape (8 heads x 65536 tokens: 8.4 MB of work), the
    # second smaller (fewer heads and tokens): the second must not see what the first left behind
    for n_heads, n_tok, n_win in ((8, 65536, 128), (3, 16 * 37 + 5, 17)):
        print("\n[case] noalloc d=%d bits=%d m=%d packed=%d heads=%d tokens=%d window=%d" % (
            d, bits, m, packed, n_heads, n_tok, n_win), flush=True)
        need = pq.attention_work_bytes(d, n_heads, n_tok)
        assert 0 < need <= pq.ATTN_NOALLOC_MAX_WORK
        keys, values, q, (kw, vw) = _inputs(rng, d, bits, m, n_heads, n_q, n_tok, n_win, packed)
        prep = pq.query_prep(q, seeded.gpu_signs(k_seed, d), G)
        ref = pq.attention(prep, keys, values, v_signs, d, bits, n_heads, n_q, n_tok, m=m, k_win=kw, v_win=vw,
                           q=q, packed=packed)
        out = torch.full((n_heads, n_q, d), float("nan"), dtype=torch.float32, device="cuda")
        got = pq.attention_noalloc(prep, keys, values, v_signs, d, bits, n_heads, n_q, n_tok, m=m, k_win=kw,
                                   v_win=vw, q=q, packed=packed, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.isfinite(got).all()
        assert torch.equal(got, ref), float((got - ref).abs().max())


def test_noalloc_rejects_work_beyond_the_array():
    """A request whose work exceeds the fixed array fails with PQ_ETOOBIG before any launch."""
    d, n_heads, n_tok = 512, 4096, 64
    assert pq.attention_work_bytes(d, n_heads, n_tok) > pq.ATTN_NOALLOC_MAX_WORK
    z8 = torch.zeros((n_heads * n_tok * d,), dtype=torch.uint8, device="cuda")
    z16 = torch.zeros((n_heads * n_tok,), dtype=torch.float16, device="cuda")
    prep = torch.zeros((pq.query_prep_bytes(d, 0, n_heads),), dtype=torch.uint8, device="cuda")
    with pytest.raises(pq.PQError) as e:
        pq.attention_noalloc(prep, (z8, z16, None, None), (z8, z16), torch.zeros(d // 8, dtype=torch.uint8,
                             device="cuda"), d, 3, n_heads, 1, n_tok)
    assert e.value.status == pq.PQ_ETOOBIG
