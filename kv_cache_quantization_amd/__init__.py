"""MI355X (gfx950) rotate-then-quantize block codec and QJL sketch.

Python binding of the C ABI in ``include/pq.h`` (library ``libpqhip.so`` built
in this directory by ``python kv_cache_quantization_amd/build.py``).  The
binding only marshals arguments: every step of the path runs in the library's
HIP kernels.  torch supplies device memory and the current HIP stream.

Importing works without a GPU (the library loads, compute calls then fail with
PQ_EHIP); importing fails loudly when the library has not been built.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpqhip.so")

PQ_OK, PQ_EINVAL, PQ_EUNSUPPORTED, PQ_EHIP = 0, 1, 2, 3
PQ_F32, PQ_BF16 = 0, 1


class PQError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.pq_strerror(status).decode()
        if status == PQ_EHIP:
            msg += " (hipError_t %d)" % _lib.pq_last_hip_error()
        super().__init__("%s: %s" % (where, msg))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("kv_cache_quantization_amd: %s is not built "
                          "(run python kv_cache_quantization_amd/build.py)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.POINTER(ctypes.c_double)
    sig = {
        "pq_abi_version": ([], I),
        "pq_strerror": ([I], ctypes.c_char_p),
        "pq_last_hip_error": ([], I),
        "pq_codebook": ([I, D, D, D], I),
        "pq_quantize": ([I, I, I, P, L, P, I, P, P, P, P, P, P], I),
        "pq_dequantize": ([I, I, P, P, L, P, I, P, P], I),
        "pq_quantize_packed": ([I, I, I, P, L, P, I, P, P, P, P, P, P], I),
        "pq_dequantize_packed": ([I, I, P, P, L, P, I, P, P], I),
        "qjl_sketch": ([I, I, P, L, P, P, P, P], I),
        "qjl_project": ([I, I, P, L, P, P, P], I),
        "qjl_score": ([I, I, I, I, L, P, P, P, P, P], I),
        "qjl_score_add": ([I, I, I, I, L, P, P, P, P, P], I),
        "qjl_outlier_channels": ([I, P, L, L, I, I, P, P], I),
        "qjl_sketch_split": ([I, I, P, L, L, I, I, P, I, P, P, P, P], I),
        "pq_query_prep_bytes": ([I, I, I], L),
        "pq_query_prep": ([I, I, I, I, P, P, P, P, P], I),
        "pq_score": ([I, I, I, I, I, L, P, P, P, P, P, P, P], I),
        "pq_score_packed": ([I, I, I, I, I, L, P, P, P, P, P, P, P], I),
        "pq_attention_work_bytes": ([I, I, L], L),
        "pq_quantize_bd": ([I, I, I, P, L, P, P, P, P], I),
        "pq_sphere_codebook": ([I, I, D, D], I),
        "pq_quantize_dense": ([I, I, I, P, L, P, P, P, P], I),
        "pq_dequantize_dense": ([I, I, P, P, L, P, I, P, P], I),
        "pq_dequantize_bd": ([I, I, P, P, L, P, I, P, P], I),
        "pq_attention": ([I, I, I, I, I, L, P, P, P, P, P, P, P, P, L, P, P, P, ctypes.c_float, P, P, P], I),
        "pq_attention_packed": ([I, I, I, I, I, L, P, P, P, P, P, P, P, P, L, P, P, P, ctypes.c_float, P, P, P],
                                I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()
EXPORTS = ("pq_abi_version", "pq_strerror", "pq_last_hip_error", "pq_codebook", "pq_quantize",
           "pq_dequantize", "pq_quantize_packed", "pq_dequantize_packed", "qjl_sketch", "qjl_project",
           "qjl_score", "qjl_score_add", "qjl_outlier_channels", "qjl_sketch_split", "pq_query_prep_bytes",
           "pq_query_prep", "pq_score", "pq_score_packed", "pq_attention_work_bytes", "pq_attention",
           "pq_attention_packed", "pq_quantize_bd", "pq_dequantize_bd", "pq_sphere_codebook",
           "pq_quantize_dense", "pq_dequantize_dense")


def lib():
    """The loaded ctypes library (for tests of the raw C ABI)."""
    return _lib


def _check(status, where):
    if status != PQ_OK:
        raise PQError(status, where)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dtypes):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def codebook(bits):
    """(centroids, boundaries, mse) of the library's Lloyd-Max N(0,1) quantizer (host)."""
    L = 1 << bits
    c = (ctypes.c_double * L)()
    b = (ctypes.c_double * max(L - 1, 1))()
    mse = ctypes.c_double()
    _check(_lib.pq_codebook(bits, c, b, ctypes.byref(mse)), "pq_codebook")
    return list(c), list(b)[:L - 1], mse.value


def quantize(x, d, bits, signs, proj=None, out=None, packed=False):
    """Quantize the contiguous d-element blocks of ``x`` (fp32 or bf16).

    Returns (codes uint8 [n, d], norms fp16 [n], qjl_bits uint8 [n, m/8] or None,
    rnorms fp16 [n] or None).  ``proj`` (bf16 [m, d]) turns on the QJL residual stage.
    ``out`` may hold preallocated (codes, norms, qjl_bits, rnorms).  ``packed`` calls
    pq_quantize_packed: codes are then uint8 [n, d * bits / 8], a bit stream per block.
    """
    _dev(x, "x", (torch.float32, torch.bfloat16))
    _dev(signs, "signs", (torch.uint8,))
    if x.numel() % d:
        raise ValueError("x.numel() must be a multiple of d")
    n = x.numel() // d
    m = 0
    if proj is not None:
        _dev(proj, "proj", (torch.bfloat16,))
        m = proj.shape[0]
    if out is None:
        codes = torch.empty((n, d * bits // 8 if packed else d), dtype=torch.uint8, device=x.device)
        norms = torch.empty((n,), dtype=torch.float16, device=x.device)
        qb = torch.empty((n, m // 8), dtype=torch.uint8, device=x.device) if m else None
        rn = torch.empty((n,), dtype=torch.float16, device=x.device) if m else None
    else:
        codes, norms, qb, rn = out
    dt = PQ_BF16 if x.dtype == torch.bfloat16 else PQ_F32
    fn, name = (_lib.pq_quantize_packed, "pq_quantize_packed") if packed else (_lib.pq_quantize, "pq_quantize")
    _check(fn(d, bits, dt, _ptr(x), n, _ptr(signs), m, _ptr(proj), _ptr(codes), _ptr(norms),
              _ptr(qb), _ptr(rn), _stream()), name)
    return codes, norms, qb, rn


def dequantize(codes, norms, d, bits, signs, out_dtype=torch.bfloat16, out=None, packed=False):
    """Reconstruct blocks from codes (uint8 [n, d], or [n, d * bits / 8] with ``packed``,
    which calls pq_dequantize_packed) and fp16 norms; returns [n, d]."""
    _dev(codes, "codes", (torch.uint8,))
    _dev(norms, "norms", (torch.float16,))
    _dev(signs, "signs", (torch.uint8,))
    n = norms.numel()
    if codes.numel() != n * (d * bits // 8 if packed else d):
        raise ValueError("codes do not match norms")
    if out is None:
        out = torch.empty((n, d), dtype=out_dtype, device=codes.device)
    _dev(out, "out", (torch.float32, torch.bfloat16))
    dt = PQ_BF16 if out.dtype == torch.bfloat16 else PQ_F32
    fn, name = (_lib.pq_dequantize_packed, "pq_dequantize_packed") if packed else (_lib.pq_dequantize, "pq_dequantize")
    _check(fn(d, bits, _ptr(codes), _ptr(norms), n, _ptr(signs), dt, _ptr(out), _stream()), name)
    return out


def qjl_sketch(keys, proj, out=None, split=None):
    """keys bf16 [..., d]; returns (bits uint8 [n, m/8], norms fp16 [n]).

    ``split`` = (idx, seq_len, group_size, part) sketches one part of each key split by its
    group's outlier channels (qjl_sketch_split): part 0 without them, part 1 only them;
    keys are then [heads, seq_len, d] and idx as from ``qjl_outlier_channels``."""
    _dev(keys, "keys", (torch.bfloat16,))
    _dev(proj, "proj", (torch.bfloat16,))
    m, d = proj.shape
    n = keys.numel() // d
    if out is None:
        bits = torch.empty((n, m // 8), dtype=torch.uint8, device=keys.device)
        norms = torch.empty((n,), dtype=torch.float16, device=keys.device)
    else:
        bits, norms = out
    if split is None:
        _check(_lib.qjl_sketch(d, m, _ptr(keys), n, _ptr(proj), _ptr(bits), _ptr(norms), _stream()), "qjl_sketch")
    else:
        idx, seq_len, group_size, part = split
        _dev(idx, "idx", (torch.uint8,))
        if n % seq_len:
            raise ValueError("keys are not [heads, seq_len, d]")
        _check(_lib.qjl_sketch_split(d, m, _ptr(keys), n // seq_len, seq_len, group_size, idx.shape[-1], _ptr(idx),
                                     part, _ptr(proj), _ptr(bits), _ptr(norms), _stream()), "qjl_sketch_split")
    return bits, norms


def qjl_outlier_channels(keys, group_size, n_out, out=None):
    """keys bf16 [..., seq_len, d] -> uint8 [..., ceil(seq_len / group_size), n_out]: per group of
    group_size consecutive tokens, the n_out channels of largest norm, decreasing."""
    _dev(keys, "keys", (torch.bfloat16,))
    seq_len, d = keys.shape[-2], keys.shape[-1]
    heads = keys.numel() // (seq_len * d)
    n_groups = (seq_len + group_size - 1) // group_size
    if out is None:
        out = torch.empty(tuple(keys.shape[:-2]) + (n_groups, n_out), dtype=torch.uint8, device=keys.device)
    _check(_lib.qjl_outlier_channels(d, _ptr(keys), heads, seq_len, group_size, n_out, _ptr(out), _stream()),
           "qjl_outlier_channels")
    return out


def qjl_project(q, proj, out=None):
    """Project queries q (bf16 [..., d]) through G: fp32 [n_q, m]."""
    _dev(q, "q", (torch.bfloat16,))
    _dev(proj, "proj", (torch.bfloat16,))
    m, d = proj.shape
    nq = q.numel() // d
    if out is None:
        out = torch.empty((nq, m), dtype=torch.float32, device=q.device)
    _check(_lib.qjl_project(d, m, _ptr(q), nq, _ptr(proj), _ptr(out), _stream()), "qjl_project")
    return out


def qjl_score(sq, bits, norms, batch, kv_heads, q_heads, n_keys, out=None, accumulate=False):
    """QJL scores [batch, q_heads, n_keys] fp32 from projected queries and packed key bits;
    ``accumulate`` adds them to ``out`` (qjl_score_add)."""
    _dev(sq, "sq", (torch.float32,))
    _dev(bits, "bits", (torch.uint8,))
    _dev(norms, "norms", (torch.float16,))
    m = sq.shape[-1]
    if accumulate and out is None:
        raise ValueError("accumulate needs out")
    if out is None:
        out = torch.empty((batch, q_heads, n_keys), dtype=torch.float32, device=sq.device)
    fn, name = (_lib.qjl_score_add, "qjl_score_add") if accumulate else (_lib.qjl_score, "qjl_score")
    _check(fn(m, batch, kv_heads, q_heads, n_keys, _ptr(sq), _ptr(bits), _ptr(norms), _ptr(out), _stream()), name)
    return out


def query_prep_bytes(d, m, n_heads):
    """Bytes of the prepared-query buffer of the two-stage score."""
    nb = _lib.pq_query_prep_bytes(d, m, n_heads)
    if nb < 0:
        raise PQError(PQ_EINVAL, "pq_query_prep_bytes")
    return nb


def query_prep(q, signs, proj=None, out=None):
    """Prepare queries q (bf16 [n_heads, n_q, d], n_q <= 16) for ``score``.

    Returns a uint8 device buffer; per head it starts with H(D q) as fp32 [16, d]
    and G q as fp32 [16, m] (see ``prep_views``).
    """
    _dev(q, "q", (torch.bfloat16,))
    _dev(signs, "signs", (torch.uint8,))
    n_heads, n_q, d = q.shape
    m = 0
    if proj is not None:
        _dev(proj, "proj", (torch.bfloat16,))
        m = proj.shape[0]
    if out is None:
        out = torch.empty((query_prep_bytes(d, m, n_heads),), dtype=torch.uint8, device=q.device)
    _check(_lib.pq_query_prep(d, m, n_heads, n_q, _ptr(q), _ptr(signs), _ptr(proj), _ptr(out), _stream()),
           "pq_query_prep")
    return out


def prep_views(prep, d, m, n_heads):
    """(qrot fp32 [n_heads, 16, d], sq fp32 [n_heads, 16, m]) views of a prepared-query buffer."""
    per = query_prep_bytes(d, m, 1)
    heads = prep.view(n_heads, per)
    qrot = heads[:, :16 * d * 4].contiguous().view(torch.float32).view(n_heads, 16, d)
    sq = heads[:, 16 * d * 4:16 * (d + m) * 4].contiguous().view(torch.float32).view(n_heads, 16, m)
    return qrot, sq


def score(prep, codes, norms, d, bits, n_heads, n_q, n_tok, qjl_bits=None, rnorms=None, m=0, out=None,
          packed=False):
    """Two-stage scores fp32 [n_heads, n_q, n_tok] from codes [n_heads, n_tok, d] (or bit-packed,
    d * bits / 8 bytes per token, with ``packed``: pq_score_packed), norms, and (with m > 0)
    the QJL residual bits and residual norms."""
    _dev(prep, "prep", (torch.uint8,))
    _dev(codes, "codes", (torch.uint8,))
    _dev(norms, "norms", (torch.float16,))
    if m:
        _dev(qjl_bits, "qjl_bits", (torch.uint8,))
        _dev(rnorms, "rnorms", (torch.float16,))
    if out is None:
        out = torch.empty((n_heads, n_q, n_tok), dtype=torch.float32, device=codes.device)
    _dev(out, "out", (torch.float32,))
    if codes.numel() != n_heads * n_tok * (d * bits // 8 if packed else d):
        raise ValueError("codes do not match n_heads, n_tok, d")
    fn, name = (_lib.pq_score_packed, "pq_score_packed") if packed else (_lib.pq_score, "pq_score")
    _check(fn(d, bits, m, n_heads, n_q, n_tok, _ptr(prep), _ptr(codes), _ptr(norms), _ptr(qjl_bits),
              _ptr(rnorms), _ptr(out), _stream()), name)
    return out


def attention_work_bytes(d, n_heads, n_tok):
    """Bytes of the work buffer ``attention`` needs (partial results of the fused kernel)."""
    nb = _lib.pq_attention_work_bytes(d, n_heads, n_tok)
    if nb < 0:
        raise PQError(PQ_EINVAL, "pq_attention_work_bytes")
    return nb


def attention(prep, keys, values, v_signs, d, bits, n_heads, n_q, n_tok, m=0, k_win=None, v_win=None,
              q=None, sm_scale=None, packed=False, work=None, out=None):
    """Decode attention over a quantized cache plus an unquantized recent window.

    prep: ``query_prep`` of the queries with the key signs (and G when m > 0).
    keys: (codes, norms, qjl_bits, rnorms) of the quantized keys, [n_heads, n_tok, ...]
    (qjl_bits and rnorms None when m == 0); values: (codes, norms), quantized without QJL.
    k_win, v_win: bf16 [n_heads, n_win, d] (or None); q: the bf16 queries [n_heads, n_q, d],
    needed with a window.  Returns fp32 [n_heads, n_q, d]; sm_scale defaults to 1/sqrt(d).
    ``packed``: codes bit-packed at the code width (pq_attention_packed).
    """
    k_codes, k_norms, k_bits, k_rn = keys
    v_codes, v_norms = values
    for t, name in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _dev(t, name, (torch.uint8,))
        if n_tok and t.numel() != n_heads * n_tok * (d * bits // 8 if packed else d):
            raise ValueError("%s do not match n_heads, n_tok, d" % name)
    _dev(k_norms, "k_norms", (torch.float16,))
    _dev(v_norms, "v_norms", (torch.float16,))
    _dev(v_signs, "v_signs", (torch.uint8,))
    if n_tok:
        _dev(prep, "prep", (torch.uint8,))
    if m:
        _dev(k_bits, "k_qjl_bits", (torch.uint8,))
        _dev(k_rn, "k_rnorms", (torch.float16,))
    n_win = 0
    if k_win is not None:
        _dev(k_win, "k_win", (torch.bfloat16,))
        _dev(v_win, "v_win", (torch.bfloat16,))
        _dev(q, "q", (torch.bfloat16,))
        n_win = k_win.shape[1]
        if k_win.shape != (n_heads, n_win, d) or v_win.shape != k_win.shape or q.shape != (n_heads, n_q, d):
            raise ValueError("window or query shape does not match n_heads, n_q, d")
    if sm_scale is None:
        sm_scale = 1.0 / float(d) ** 0.5
    dev = v_codes.device
    if work is None:
        work = torch.empty((max(16, attention_work_bytes(d, n_heads, n_tok)),), dtype=torch.uint8, device=dev)
    _dev(work, "work", (torch.uint8,))
    if work.numel() < attention_work_bytes(d, n_heads, n_tok):
        raise ValueError("work buffer too small")
    if out is None:
        out = torch.empty((n_heads, n_q, d), dtype=torch.float32, device=dev)
    _dev(out, "out", (torch.float32,))
    fn, name = (_lib.pq_attention_packed, "pq_attention_packed") if packed else (_lib.pq_attention, "pq_attention")
    _check(fn(d, bits, m, n_heads, n_q, n_tok, _ptr(prep), _ptr(k_codes), _ptr(k_norms), _ptr(k_bits), _ptr(k_rn),
              _ptr(v_codes), _ptr(v_norms), _ptr(v_signs), n_win, _ptr(k_win), _ptr(v_win), _ptr(q),
              float(sm_scale), _ptr(work), _ptr(out), _stream()), name)
    return out


def quantize_bd(x, d, bits, signs, out=None):
    """Codec with the block-diagonal rotation, for block sizes d that are not powers of two
    (any multiple of 32 in 64..4096): x fp32 or bf16 with numel a multiple of d.
    Returns (codes uint8 [n_blocks, d], norms fp16 [n_blocks])."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    _dev(signs, "signs", (torch.uint8,))
    if x.numel() % d:
        raise ValueError("x.numel() must be a multiple of d")
    n = x.numel() // d
    if out is None:
        out = (torch.empty((n, d), dtype=torch.uint8, device=x.device),
               torch.empty((n,), dtype=torch.float16, device=x.device))
    codes, norms = out
    _check(_lib.pq_quantize_bd(d, bits, PQ_BF16 if x.dtype == torch.bfloat16 else PQ_F32, _ptr(x), n,
                               _ptr(signs), _ptr(codes), _ptr(norms), _stream()), "pq_quantize_bd")
    return codes, norms


def dequantize_bd(codes, norms, d, bits, signs, out_dtype=torch.bfloat16, out=None):
    """Inverse of ``quantize_bd``: [n_blocks, d] of out_dtype (fp32 or bf16)."""
    _dev(codes, "codes", (torch.uint8,))
    _dev(norms, "norms", (torch.float16,))
    _dev(signs, "signs", (torch.uint8,))
    n = norms.numel()
    if codes.numel() != n * d:
        raise ValueError("codes do not match norms and d")
    if out is None:
        out = torch.empty((n, d), dtype=out_dtype, device=codes.device)
    _dev(out, "out", (torch.float32, torch.bfloat16))
    _check(_lib.pq_dequantize_bd(d, bits, _ptr(codes), _ptr(norms), n, _ptr(signs),
                                 PQ_BF16 if out.dtype == torch.bfloat16 else PQ_F32, _ptr(out), _stream()),
           "pq_dequantize_bd")
    return out


def sphere_codebook(bits, d):
    """(centroids, boundaries) float64 of the Lloyd-Max quantizer of one sphere coordinate in R^d."""
    c = (ctypes.c_double * (1 << bits))()
    b = (ctypes.c_double * max(1, (1 << bits) - 1))()
    _check(_lib.pq_sphere_codebook(bits, d, c, b), "pq_sphere_codebook")
    return list(c), list(b)[: (1 << bits) - 1]


def quantize_dense(x, d, bits, rot, out=None):
    """Codec with a dense rotation rot (fp32 [d, d], row-major, device) and the sphere-coordinate
    codebook.  Returns (codes uint8 [n_blocks, d], norms fp16 [n_blocks])."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    _dev(rot, "rot", (torch.float32,))
    if x.numel() % d or rot.numel() != d * d:
        raise ValueError("x.numel() must be a multiple of d and rot must be d x d")
    n = x.numel() // d
    if out is None:
        out = (torch.empty((n, d), dtype=torch.uint8, device=x.device),
               torch.empty((n,), dtype=torch.float16, device=x.device))
    codes, norms = out
    _check(_lib.pq_quantize_dense(d, bits, PQ_BF16 if x.dtype == torch.bfloat16 else PQ_F32, _ptr(x), n, _ptr(rot),
                                  _ptr(codes), _ptr(norms), _stream()), "pq_quantize_dense")
    return codes, norms


def dequantize_dense(codes, norms, d, bits, rot, out_dtype=torch.bfloat16, out=None):
    """Inverse of ``quantize_dense``: [n_blocks, d] of out_dtype (fp32 or bf16)."""
    _dev(codes, "codes", (torch.uint8,))
    _dev(norms, "norms", (torch.float16,))
    _dev(rot, "rot", (torch.float32,))
    n = norms.numel()
    if codes.numel() != n * d:
        raise ValueError("codes do not match norms and d")
    if out is None:
        out = torch.empty((n, d), dtype=out_dtype, device=codes.device)
    _dev(out, "out", (torch.float32, torch.bfloat16))
    _check(_lib.pq_dequantize_dense(d, bits, _ptr(codes), _ptr(norms), n, _ptr(rot),
                                    PQ_BF16 if out.dtype == torch.bfloat16 else PQ_F32, _ptr(out), _stream()),
           "pq_dequantize_dense")
    return out
