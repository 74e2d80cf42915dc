"""The C ABI: library loads, exports every declared symbol, validates arguments on
the host and reports HIP failures (CPU only: no kernel is launched)."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import kv_cache_quantization_amd as pq
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = []
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", f)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", txt, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = pq.lib()
    declared = _declared()
    assert len(declared) >= 9
    for name in declared:
        assert hasattr(lib, name), name
    assert set(pq.EXPORTS) == set(declared)


def test_abi_version_and_strerror():
    lib = pq.lib()
    assert lib.pq_abi_version() == 1
    for st in range(5):
        assert isinstance(lib.pq_strerror(st), bytes) and lib.pq_strerror(st)
    assert lib.pq_strerror(0) == b"ok"


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6])
def test_library_codebook_matches_oracle(bits):
    c, b, mse = pq.codebook(bits)
    oc, ob, om = oracle.lloyd_max.codebook(bits)
    assert np.allclose(c, oc, atol=1e-9, rtol=0)
    assert np.allclose(b, ob, atol=1e-9, rtol=0)
    assert abs(mse - om) < 1e-9
    # the fp32 tables the kernels use agree with the oracle's fp32 decision thresholds
    assert np.array_equal(np.float32(b), np.float32(ob))


def test_codebook_rejects_bad_bits():
    lib = pq.lib()
    D = ctypes.POINTER(ctypes.c_double)
    assert lib.pq_codebook(0, D(), D(), D()) == pq.PQ_EINVAL
    assert lib.pq_codebook(9, D(), D(), D()) == pq.PQ_EINVAL


# Fake device pointers: never dereferenced, because validation fails before any HIP call.
P16 = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x10002)
NUL = ctypes.c_void_p(0)


def _q(**kw):
    a = dict(d=128, bits=4, dt=pq.PQ_BF16, x=P16, n=16, signs=P16, m=0, proj=NUL, codes=P16, norms=P16,
             qb=NUL, rn=NUL)
    a.update(kw)
    return pq.lib().pq_quantize(a["d"], a["bits"], a["dt"], a["x"], a["n"], a["signs"], a["m"], a["proj"],
                                a["codes"], a["norms"], a["qb"], a["rn"], NUL)


@pytest.mark.parametrize("kw,st", [
    (dict(d=96), pq.PQ_EINVAL), (dict(d=32), pq.PQ_EUNSUPPORTED), (dict(d=1024), pq.PQ_EUNSUPPORTED),
    (dict(bits=0), pq.PQ_EINVAL), (dict(bits=9), pq.PQ_EINVAL), (dict(dt=7), pq.PQ_EINVAL),
    (dict(n=-1), pq.PQ_EINVAL), (dict(x=NUL), pq.PQ_EINVAL), (dict(codes=NUL), pq.PQ_EINVAL),
    (dict(norms=NUL), pq.PQ_EINVAL), (dict(signs=NUL), pq.PQ_EINVAL),
    (dict(x=P2), pq.PQ_EINVAL), (dict(codes=ctypes.c_void_p(0x10008)), pq.PQ_EINVAL),
    (dict(norms=ctypes.c_void_p(0x10001)), pq.PQ_EINVAL),
    (dict(m=12, proj=P16, qb=P16, rn=P16), pq.PQ_EINVAL), (dict(m=2048, proj=P16, qb=P16, rn=P16), pq.PQ_EUNSUPPORTED),
    (dict(m=64), pq.PQ_EINVAL), (dict(m=64, proj=P16, qb=P16), pq.PQ_EINVAL),
    (dict(m=0, proj=P16), pq.PQ_EINVAL), (dict(m=-8), pq.PQ_EINVAL),
    (dict(n=2 ** 62), pq.PQ_EINVAL),
])
def test_quantize_validation(kw, st):
    assert _q(**kw) == st


def test_empty_input_is_a_no_op():
    assert _q(n=0) == pq.PQ_OK
    lib = pq.lib()
    assert lib.pq_dequantize(128, 4, P16, P16, 0, P16, pq.PQ_BF16, P16, NUL) == pq.PQ_OK
    assert lib.qjl_sketch(128, 256, P16, 0, P16, P16, P16, NUL) == pq.PQ_OK
    assert lib.qjl_score(256, 4, 8, 32, 0, P16, P16, P16, P16, NUL) == pq.PQ_OK


def test_other_entry_points_validate():
    lib = pq.lib()
    assert lib.pq_dequantize(100, 4, P16, P16, 4, P16, pq.PQ_BF16, P16, NUL) == pq.PQ_EINVAL
    assert lib.pq_dequantize(128, 4, P16, P16, 4, P16, 3, P16, NUL) == pq.PQ_EINVAL
    assert lib.pq_dequantize(128, 4, P16, P16, 4, P16, pq.PQ_F32, P2, NUL) == pq.PQ_EINVAL
    assert lib.qjl_sketch(128, 12, P16, 4, P16, P16, P16, NUL) == pq.PQ_EINVAL
    assert lib.qjl_sketch(128, 256, P16, 4, NUL, P16, P16, NUL) == pq.PQ_EINVAL
    assert lib.qjl_project(128, 0, P16, 4, P16, P16, NUL) == pq.PQ_EINVAL
    assert lib.qjl_score(256, 4, 8, 30, 64, P16, P16, P16, P16, NUL) == pq.PQ_EINVAL      # 30 % 8
    assert lib.qjl_score(256, 4, 8, 64, 64, P16, P16, P16, P16, NUL) == pq.PQ_EUNSUPPORTED  # 8 q per kv
    assert lib.qjl_score(96, 4, 8, 32, 64, P16, P16, P16, P16, NUL) == pq.PQ_EUNSUPPORTED   # m % 64


def test_two_stage_entry_points_validate():
    lib = pq.lib()
    assert lib.pq_query_prep_bytes(100, 0, 1) == -1
    assert lib.pq_query_prep_bytes(128, 96, 1) == -1
    assert lib.pq_query_prep_bytes(128, 0, 2) == 2 * (112 * 128 + 256)
    assert lib.pq_query_prep_bytes(512, 512, 8) == 8 * (112 * 1024 + 256)
    # pq_query_prep(d, m, n_heads, n_q, q, signs, proj, prep, stream)
    assert lib.pq_query_prep(128, 128, 2, 17, P16, P16, P16, P16, NUL) == pq.PQ_EINVAL      # n_q > 16
    assert lib.pq_query_prep(128, 0, 2, 4, P16, P16, P16, P16, NUL) == pq.PQ_EINVAL         # proj without m
    assert lib.pq_query_prep(128, 96, 2, 4, P16, P16, P16, P16, NUL) == pq.PQ_EUNSUPPORTED  # m % 64
    assert lib.pq_query_prep(128, 128, 2, 4, P16, P16, P16, P2, NUL) == pq.PQ_EINVAL        # prep alignment
    assert lib.pq_query_prep(128, 128, 0, 4, NUL, NUL, NUL, NUL, NUL) == pq.PQ_OK           # no heads
    # pq_score(d, bits, m, n_heads, n_q, n_tok, prep, codes, norms, qbits, rnorms, scores, stream)
    args = lambda **kw: [kw.get(k, v) for k, v in (
        ("d", 256), ("bits", 3), ("m", 256), ("h", 2), ("nq", 16), ("t", 100), ("prep", P16), ("codes", P16),
        ("norms", P16), ("qb", P16), ("rn", P16), ("out", P16), ("s", NUL))]
    assert lib.pq_score(*args(bits=5)) == pq.PQ_EUNSUPPORTED
    assert lib.pq_score(*args(bits=0)) == pq.PQ_EINVAL
    assert lib.pq_score(*args(d=512, m=1024)) == pq.PQ_EUNSUPPORTED                        # d + m > 1344
    assert lib.pq_score(*args(nq=17)) == pq.PQ_EINVAL
    assert lib.pq_score(*args(m=0)) == pq.PQ_EINVAL                                         # bits without m
    assert lib.pq_score(*args(qb=NUL)) == pq.PQ_EINVAL
    assert lib.pq_score(*args(codes=ctypes.c_void_p(0x10008))) == pq.PQ_EINVAL
    assert lib.pq_score(*args(t=0, prep=NUL, codes=NUL)) == pq.PQ_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="needs a machine without a GPU")
def test_valid_call_without_gpu_reports_hip_error():
    # arguments pass validation, so the library reaches the HIP runtime, which has no device
    assert _q() == pq.PQ_EHIP
    assert pq.lib().pq_last_hip_error() != 0
    with pytest.raises(pq.PQError):
        raise pq.PQError(pq.PQ_EHIP, "pq_quantize")


def test_packed_entry_points_validate():
    """Packed codes exist at every width 1..8; bad arguments are refused before any HIP call."""
    lib = pq.lib()

    def qp(bits, n=16, **kw):
        a = dict(d=128, dt=pq.PQ_BF16, x=P16, signs=P16, m=0, proj=NUL, codes=P16, norms=P16, qb=NUL, rn=NUL)
        a.update(kw)
        return lib.pq_quantize_packed(a["d"], bits, a["dt"], a["x"], n, a["signs"], a["m"], a["proj"],
                                      a["codes"], a["norms"], a["qb"], a["rn"], NUL)

    for bits in (0, 9, -1):
        assert qp(bits) == pq.PQ_EINVAL
        assert lib.pq_dequantize_packed(128, bits, P16, P16, 16, P16, pq.PQ_BF16, P16, NUL) == pq.PQ_EINVAL
    for bits in range(1, 9):
        assert qp(bits, n=0) == pq.PQ_OK
        assert lib.pq_dequantize_packed(128, bits, P16, P16, 0, P16, pq.PQ_BF16, P16, NUL) == pq.PQ_OK
        assert qp(bits, d=96) == pq.PQ_EINVAL
        assert qp(bits, d=1024) == pq.PQ_EUNSUPPORTED
        assert qp(bits, codes=NUL) == pq.PQ_EINVAL
        assert qp(bits, codes=ctypes.c_void_p(0x10008)) == pq.PQ_EINVAL
        assert qp(bits, m=64) == pq.PQ_EINVAL
        assert lib.pq_dequantize_packed(128, bits, P16, P16, 16, P16, 3, P16, NUL) == pq.PQ_EINVAL
        assert lib.pq_dequantize_packed(128, bits, NUL, P16, 16, P16, pq.PQ_BF16, P16, NUL) == pq.PQ_EINVAL


def test_packed_score_validates_like_score():
    lib = pq.lib()
    args = (P16, P16, P16, P16, P16, P16, NUL)
    assert lib.pq_score_packed(256, 3, 256, 2, 16, 0, *args) == pq.PQ_OK                  # no tokens
    assert lib.pq_score_packed(256, 5, 256, 2, 16, 64, *args) == pq.PQ_EUNSUPPORTED       # bits > 4
    assert lib.pq_score_packed(100, 3, 0, 2, 16, 64, P16, P16, P16, NUL, NUL, P16, NUL) == pq.PQ_EINVAL
    assert lib.pq_score_packed(256, 3, 256, 2, 17, 64, *args) == pq.PQ_EINVAL             # n_q > 16


def test_outlier_entry_points_validate():
    lib = pq.lib()
    # qjl_outlier_channels(d, keys, heads, seq_len, group_size, n_out, idx, stream)
    assert lib.qjl_outlier_channels(128, P16, 0, 64, 32, 8, P16, NUL) == pq.PQ_OK
    assert lib.qjl_outlier_channels(512, P16, 2, 64, 32, 8, P16, NUL) == pq.PQ_EUNSUPPORTED
    assert lib.qjl_outlier_channels(96, P16, 2, 64, 32, 8, P16, NUL) == pq.PQ_EINVAL
    assert lib.qjl_outlier_channels(128, P16, 2, 64, 0, 8, P16, NUL) == pq.PQ_EINVAL
    assert lib.qjl_outlier_channels(128, P16, 2, 64, 32, 0, P16, NUL) == pq.PQ_EINVAL
    assert lib.qjl_outlier_channels(128, P16, 2, 64, 32, 129, P16, NUL) == pq.PQ_EINVAL
    assert lib.qjl_outlier_channels(128, NUL, 2, 64, 32, 8, P16, NUL) == pq.PQ_EINVAL
    assert lib.qjl_outlier_channels(128, P2, 2, 64, 32, 8, P16, NUL) == pq.PQ_EINVAL
    # qjl_sketch_split(d, m, keys, heads, seq_len, gs, n_out, idx, part, proj, bits, norms, stream)
    assert lib.qjl_sketch_split(128, 256, P16, 2, 0, 32, 8, P16, 0, P16, P16, P16, NUL) == pq.PQ_OK
    assert lib.qjl_sketch_split(128, 256, P16, 2, 64, 32, 8, P16, 2, P16, P16, P16, NUL) == pq.PQ_EINVAL
    assert lib.qjl_sketch_split(128, 12, P16, 2, 64, 32, 8, P16, 0, P16, P16, P16, NUL) == pq.PQ_EINVAL
    assert lib.qjl_sketch_split(512, 256, P16, 2, 64, 32, 8, P16, 0, P16, P16, P16, NUL) == pq.PQ_EUNSUPPORTED
    assert lib.qjl_sketch_split(128, 256, P16, 2, 64, 32, 8, NUL, 1, P16, P16, P16, NUL) == pq.PQ_EINVAL
    # qjl_score_add validates as qjl_score
    assert lib.qjl_score_add(256, 4, 8, 32, 0, P16, P16, P16, P16, NUL) == pq.PQ_OK
    assert lib.qjl_score_add(256, 4, 8, 30, 64, P16, P16, P16, P16, NUL) == pq.PQ_EINVAL
    assert lib.qjl_score_add(256, 4, 8, 64, 64, P16, P16, P16, P16, NUL) == pq.PQ_EUNSUPPORTED


def test_attention_entry_points_validate():
    """Decode attention: work size, and bad arguments refused before any HIP call."""
    lib = pq.lib()
    assert lib.pq_attention_work_bytes(100, 2, 64) == -1
    assert lib.pq_attention_work_bytes(128, -1, 64) == -1
    assert lib.pq_attention_work_bytes(128, 2, 0) == 0
    # one range of one tile: 16 query rows of (max, sum) and of d floats
    assert lib.pq_attention_work_bytes(128, 1, 5) == 16 * (8 + 128 * 4)
    nb = lib.pq_attention_work_bytes(256, 8, 65536)
    assert nb > 0 and nb % (16 * (8 + 256 * 4)) == 0
    F = ctypes.c_float
    names = ("d", "bits", "m", "h", "nq", "t", "prep", "kc", "kn", "kb", "kr", "vc", "vn", "vs", "w", "kw", "vw",
             "q", "scale", "work", "out", "s")
    base = dict(d=128, bits=3, m=128, h=2, nq=16, t=100, prep=P16, kc=P16, kn=P16, kb=P16, kr=P16, vc=P16,
                vn=P16, vs=P16, w=4, kw=P16, vw=P16, q=P16, scale=F(0.1), work=P16, out=P16, s=NUL)

    def att(fn=lib.pq_attention, **kw):
        a = dict(base)
        a.update(kw)
        return fn(*[a[n] for n in names])

    for fn in (lib.pq_attention, lib.pq_attention_packed):
        assert att(fn, bits=5) == pq.PQ_EUNSUPPORTED
        assert att(fn, bits=0) == pq.PQ_EINVAL
        assert att(fn, d=96) == pq.PQ_EINVAL
        assert att(fn, nq=17) == pq.PQ_EINVAL
        assert att(fn, m=0) == pq.PQ_EINVAL                          # residual bits without m
        assert att(fn, m=96) == pq.PQ_EUNSUPPORTED
        assert att(fn, kb=NUL) == pq.PQ_EINVAL
        assert att(fn, vc=NUL) == pq.PQ_EINVAL
        assert att(fn, vs=NUL) == pq.PQ_EINVAL
        assert att(fn, work=NUL) == pq.PQ_EINVAL
        assert att(fn, work=ctypes.c_void_p(0x10008)) == pq.PQ_EINVAL
        assert att(fn, kc=ctypes.c_void_p(0x10008)) == pq.PQ_EINVAL
        assert att(fn, q=NUL) == pq.PQ_EINVAL                        # window without queries
        assert att(fn, w=5000) == pq.PQ_EUNSUPPORTED
        assert att(fn, w=-1) == pq.PQ_EINVAL
        assert att(fn, t=0, w=0) == pq.PQ_EINVAL                     # softmax over no token
        assert att(fn, scale=F(float("nan"))) == pq.PQ_EINVAL
        assert att(fn, scale=F(float("inf"))) == pq.PQ_EINVAL
        assert att(fn, h=0) == pq.PQ_OK
        assert att(fn, nq=0) == pq.PQ_OK


def test_block_diagonal_entry_points_validate():
    lib = pq.lib()
    # pq_quantize_bd(d, bits, in_dtype, x, n, signs, codes, norms, stream)
    q = lambda d=192, bits=4, dt=pq.PQ_BF16, x=P16, n=16, s=P16, c=P16, nm=P16: lib.pq_quantize_bd(
        d, bits, dt, x, n, s, c, nm, NUL)
    assert q(d=100) == pq.PQ_EINVAL
    assert q(d=32) == pq.PQ_EUNSUPPORTED
    assert q(d=4128) == pq.PQ_EUNSUPPORTED
    assert q(bits=0) == pq.PQ_EINVAL and q(bits=9) == pq.PQ_EINVAL
    assert q(dt=7) == pq.PQ_EINVAL
    assert q(x=NUL) == pq.PQ_EINVAL and q(c=NUL) == pq.PQ_EINVAL
    assert q(nm=ctypes.c_void_p(0x10001)) == pq.PQ_EINVAL
    assert q(x=ctypes.c_void_p(0x10008)) == pq.PQ_EINVAL and q(c=ctypes.c_void_p(0x10008)) == pq.PQ_EINVAL
    assert q(n=-1) == pq.PQ_EINVAL
    assert q(n=0) == pq.PQ_OK
    # pq_dequantize_bd(d, bits, codes, norms, n, signs, out_dtype, out, stream)
    assert lib.pq_dequantize_bd(100, 4, P16, P16, 16, P16, pq.PQ_BF16, P16, NUL) == pq.PQ_EINVAL
    assert lib.pq_dequantize_bd(192, 4, P16, P16, 16, P16, 3, P16, NUL) == pq.PQ_EINVAL
    assert lib.pq_dequantize_bd(192, 4, NUL, P16, 16, P16, pq.PQ_BF16, P16, NUL) == pq.PQ_EINVAL
    assert lib.pq_dequantize_bd(192, 4, P16, P16, 0, P16, pq.PQ_BF16, P16, NUL) == pq.PQ_OK


@pytest.mark.parametrize("d,bits", [(64, 3), (128, 4), (16, 2), (256, 3), (512, 3), (208, 2)])
def test_library_sphere_codebook_matches_oracle(d, bits):
    c, b = pq.sphere_codebook(bits, d)
    oc, ob, _ = oracle.dense.beta_codebook(bits, d)
    np.testing.assert_allclose(c, oc, atol=1e-8)
    np.testing.assert_allclose(b, ob, atol=1e-8)


def test_dense_entry_points_validate():
    lib = pq.lib()
    q = lambda d=128, bits=4, dt=pq.PQ_BF16, x=P16, n=16, r=P16, c=P16, nm=P16: lib.pq_quantize_dense(
        d, bits, dt, x, n, r, c, nm, NUL)
    assert q(d=100) == pq.PQ_EINVAL and q(d=0) == pq.PQ_EINVAL
    assert q(d=528) == pq.PQ_EUNSUPPORTED and q(d=1024) == pq.PQ_EUNSUPPORTED
    assert q(bits=0) == pq.PQ_EINVAL and q(bits=9) == pq.PQ_EINVAL
    assert q(dt=5) == pq.PQ_EINVAL and q(r=NUL) == pq.PQ_EINVAL and q(c=NUL) == pq.PQ_EINVAL
    assert q(n=0) == pq.PQ_OK
    assert lib.pq_dequantize_dense(128, 4, P16, P16, 16, NUL, pq.PQ_BF16, P16, NUL) == pq.PQ_EINVAL
    assert lib.pq_dequantize_dense(128, 4, P16, P16, 0, P16, pq.PQ_BF16, P16, NUL) == pq.PQ_OK


def _noalloc(**kw):
    a = dict(d=256, bits=3, m=0, heads=8, nq=16, ntok=65536, prep=P16, kc=P16, kn=P16, kb=NUL, kr=NUL, vc=P16,
             vn=P16, vs=P16, nwin=0, kw=NUL, vw=NUL, q=NUL, scale=0.0625, packed=0, out=P16)
    a.update(kw)
    return pq.lib().pq_attention_noalloc(a["d"], a["bits"], a["m"], a["heads"], a["nq"], a["ntok"], a["prep"],
                                         a["kc"], a["kn"], a["kb"], a["kr"], a["vc"], a["vn"], a["vs"], a["nwin"],
                                         a["kw"], a["vw"], a["q"], a["scale"], a["packed"], a["out"], NUL)


@pytest.mark.parametrize("kw,st", [
    (dict(d=512, heads=4096, ntok=64), pq.PQ_ETOOBIG),      # 134 MB of work: beyond the fixed array
    (dict(packed=2), pq.PQ_EINVAL), (dict(prep=NUL), pq.PQ_EINVAL), (dict(out=NUL), pq.PQ_EINVAL),
    (dict(bits=5), pq.PQ_EUNSUPPORTED), (dict(ntok=0, nwin=0), pq.PQ_EINVAL), (dict(heads=0), pq.PQ_OK),
])
def test_attention_noalloc_validation(kw, st):
    """Validation and the size limit of the allocation-free attention are decided on the host,
    before any HIP call (so they run without a GPU)."""
    assert _noalloc(**kw) == st
    if st == pq.PQ_ETOOBIG:
        assert pq.attention_work_bytes(kw["d"], kw["heads"], kw["ntok"]) > pq.ATTN_NOALLOC_MAX_WORK
        assert pq.lib().pq_strerror(st) != pq.lib().pq_strerror(99)


def test_noalloc_limit_matches_the_header():
    import re
    with open(os.path.join(ROOT, "include", "pq.h")) as f:
        m = re.search(r"#define PQ_ATTN_NOALLOC_MAX_WORK \((\d+) << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == pq.ATTN_NOALLOC_MAX_WORK


@pytest.mark.parametrize("args,st", [
    ((96, 4, pq.PQ_BF16, 0, 3, P16), pq.PQ_EINVAL), ((1024, 4, pq.PQ_BF16, 0, 3, P16), pq.PQ_EUNSUPPORTED),
    ((128, 0, pq.PQ_BF16, 0, 3, P16), pq.PQ_EINVAL), ((128, 4, 7, 0, 3, P16), pq.PQ_EINVAL),
    ((128, 4, pq.PQ_BF16, 2, 3, P16), pq.PQ_EINVAL), ((128, 4, pq.PQ_BF16, 0, -1, P16), pq.PQ_EINVAL),
    ((128, 4, pq.PQ_BF16, 0, 3, NUL), pq.PQ_EINVAL), ((128, 4, pq.PQ_BF16, 0, 3, ctypes.c_void_p(0x10004)), pq.PQ_EINVAL),
    ((128, 4, pq.PQ_BF16, 1, 0, NUL), pq.PQ_OK),
])
def test_grouped_validation(args, st):
    """The grouped codec's host-side validation (no HIP call on these paths)."""
    lib = pq.lib()
    assert lib.pq_quantize_many(*args, NUL) == st
    assert lib.pq_dequantize_many(*args, NUL) == st


def test_tensor_record_layout():
    """pq_tensor is six 8-byte fields, 48 bytes: the table the binding builds."""
    import re
    with open(os.path.join(ROOT, "include", "pq.h")) as f:
        txt = f.read()
    body = re.search(r"typedef struct \{([^}]*)\} pq_tensor;", txt).group(1)
    fields = [l.strip().rstrip(";").split()[-1].lstrip("*") for l in body.strip().splitlines()]
    assert fields == ["x", "codes", "norms", "signs", "out", "n_blocks"]
