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

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpqhip.so")

PQ_OK, PQ_EINVAL, PQ_EUNSUPPORTED, PQ_EHIP, PQ_ETOOBIG = 0, 1, 2, 3, 4
ATTN_NOALLOC_MAX_WORK = 16 << 20      # PQ_ATTN_NOALLOC_MAX_WORK of include/pq.h
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
        "pq_make_signs": ([ctypes.c_uint64, I, P], I),
        "qjl_make_projection": ([ctypes.c_uint64, I, I, P], I),
        "pq_quantize": ([I, I, I, P, L, P, I, P, P, P, P, P, P], I),
        "pq_dequantize": ([I, I, P, P, L, P, I, P, P], I),
        "pq_quantize_packed": ([I, I, I, P, L, P, I, P, P, P, P, P, P], I),
        "pq_quantize_many": ([I, I, I, I, I, P, P], I),
        "pq_dequantize_many": ([I, I, I, I, I, P, P], I),
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
        "pq_attention_noalloc": ([I, I, I, I, I, L, P, P, P, P, P, P, P, P, L, P, P, P, ctypes.c_float, I, P, P],
                                 I),
        "pq_probe_stream": ([P, P, L, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()
EXPORTS = ("pq_abi_version", "pq_strerror", "pq_last_hip_error", "pq_codebook", "pq_make_signs",
           "qjl_make_projection", "pq_quantize", "pq_quantize_many", "pq_dequantize_many",
           "pq_dequantize", "pq_quantize_packed", "pq_dequantize_packed", "qjl_sketch", "qjl_project",
           "qjl_score", "qjl_score_add", "qjl_outlier_channels", "qjl_sketch_split", "pq_query_prep_bytes",
           "pq_query_prep", "pq_score", "pq_score_packed", "pq_attention_work_bytes", "pq_attention",
           "pq_attention_packed", "pq_quantize_bd", "pq_dequantize_bd", "pq_sphere_codebook",
           "pq_quantize_dense", "pq_dequantize_dense", "pq_attention_noalloc", "pq_probe_stream")


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


def _dev(t, name, dtypes, numel=None, device=None, min_numel=None):
    """Check a caller tensor before its pointer reaches a kernel: a contiguous device tensor of
    one of ``dtypes`` on ``device``, with exactly ``numel`` (or at least ``min_numel``)
    elements.  A buffer of the wrong size would become an out-of-bounds device access, which
    the C ABI (raw pointers) cannot see."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if numel is not None and t.numel() != numel:
        raise ValueError("%s has %d elements, expected %d" % (name, t.numel(), numel))
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError("%s has %d elements, needs at least %d" % (name, t.numel(), min_numel))
    return t


def _proj_shape(proj, d, name="proj"):
    """m of a JL matrix proj (bf16 [m, d])."""
    if proj.dim() != 2 or proj.shape[1] != d:
        raise ValueError("%s must be [m, %d], got %s" % (name, d, tuple(proj.shape)))
    return proj.shape[0]


def codebook(bits):
    """(centroids, boundaries, mse) of the library's Lloyd-Max N(0,1) quantizer (host)."""
    L = 1 << bits
    c = (ctypes.c_double * L)()
    b = (ctypes.c_double * max(L - 1, 1))()
    mse = ctypes.c_double()
    _check(_lib.pq_codebook(bits, c, b, ctypes.byref(mse)), "pq_codebook")
    return list(c), list(b)[:L - 1], mse.value


def make_signs(seed, d):
    """Rotation sign mask of ``seed`` (pq_make_signs): numpy uint8 [d/8], bit j set <=> D_j = -1."""
    mask = np.zeros(d // 8 if d > 0 else 0, dtype=np.uint8)
    _check(_lib.pq_make_signs(int(seed) & 0xFFFFFFFFFFFFFFFF, d, mask.ctypes.data_as(ctypes.c_void_p)),
           "pq_make_signs")
    return mask


def make_projection(seed, m, d):
    """Gaussian JL matrix G of ``seed`` (qjl_make_projection): numpy uint16 [m, d] of bf16 bits."""
    g = np.zeros((max(m, 0), max(d, 0)), dtype=np.uint16)
    _check(_lib.qjl_make_projection(int(seed) & 0xFFFFFFFFFFFFFFFF, m, d, g.ctypes.data_as(ctypes.c_void_p)),
           "qjl_make_projection")
    return g


def signs_tensor(seed, d, device="cuda"):
    """``make_signs`` as a uint8 tensor on ``device``."""
    return torch.from_numpy(make_signs(seed, d)).to(device)


def projection_tensor(seed, m, d, device="cuda"):
    """``make_projection`` as a bfloat16 tensor [m, d] on ``device``."""
    return torch.from_numpy(make_projection(seed, m, d).view("int16")).view(torch.bfloat16).to(device)


def quantize(x, d, bits, signs, proj=None, out=None, packed=False):
    """Quantize the contiguous d-element blocks of ``x`` (fp32 or bf16).

    Returns (codes uint8 [n, d], norms fp16 [n], qjl_bits uint8 [n, m/8] or None,
    rnorms fp16 [n] or None).  ``proj`` (bf16 [m, d]) turns on the QJL residual stage.
    ``out`` may hold preallocated (codes, norms, qjl_bits, rnorms).  ``packed`` calls
    pq_quantize_packed: codes are then uint8 [n, d * bits / 8], a bit stream per block.
    """
    _dev(x, "x", (torch.float32, torch.bfloat16))
    dev = x.device
    _dev(signs, "signs", (torch.uint8,), numel=d // 8, device=dev)
    if d <= 0 or x.numel() % d:
        raise ValueError("x.numel() must be a multiple of d")
    n = x.numel() // d
    m = 0
    if proj is not None:
        _dev(proj, "proj", (torch.bfloat16,), device=dev)
        m = _proj_shape(proj, d)
    cb = d * bits // 8 if packed else d
    if out is None:
        codes = torch.empty((n, cb), dtype=torch.uint8, device=dev)
        norms = torch.empty((n,), dtype=torch.float16, device=dev)
        qb = torch.empty((n, m // 8), dtype=torch.uint8, device=dev) if m else None
        rn = torch.empty((n,), dtype=torch.float16, device=dev) if m else None
    else:
        codes, norms, qb, rn = out
    _dev(codes, "codes", (torch.uint8,), numel=n * cb, device=dev)
    _dev(norms, "norms", (torch.float16,), numel=n, device=dev)
    if m:
        _dev(qb, "qjl_bits", (torch.uint8,), numel=n * (m // 8), device=dev)
        _dev(rn, "rnorms", (torch.float16,), numel=n, device=dev)
    elif qb is not None or rn is not None:
        raise ValueError("qjl_bits and rnorms need proj")
    dt = PQ_BF16 if x.dtype == torch.bfloat16 else PQ_F32
    fn, name = (_lib.pq_quantize_packed, "pq_quantize_packed") if packed else (_lib.pq_quantize, "pq_quantize")
    _check(fn(d, bits, dt, _ptr(x), n, _ptr(signs), m, _ptr(proj), _ptr(codes), _ptr(norms),
              _ptr(qb), _ptr(rn), _stream()), name)
    return codes, norms, qb, rn


def dequantize(codes, norms, d, bits, signs, out_dtype=torch.bfloat16, out=None, packed=False):
    """Reconstruct blocks from codes (uint8 [n, d], or [n, d * bits / 8] with ``packed``,
    which calls pq_dequantize_packed) and fp16 norms; returns [n, d]."""
    _dev(norms, "norms", (torch.float16,))
    dev = norms.device
    n = norms.numel()
    _dev(codes, "codes", (torch.uint8,), numel=n * (d * bits // 8 if packed else d), device=dev)
    _dev(signs, "signs", (torch.uint8,), numel=d // 8, device=dev)
    if out is None:
        out = torch.empty((n, d), dtype=out_dtype, device=dev)
    _dev(out, "out", (torch.float32, torch.bfloat16), numel=n * d, device=dev)
    dt = PQ_BF16 if out.dtype == torch.bfloat16 else PQ_F32
    fn, name = (_lib.pq_dequantize_packed, "pq_dequantize_packed") if packed else (_lib.pq_dequantize, "pq_dequantize")
    _check(fn(d, bits, _ptr(codes), _ptr(norms), n, _ptr(signs), dt, _ptr(out), _stream()), name)
    return out


def _tensor_table(rows, device):
    """Device table of pq_tensor records (x, codes, norms, signs, out, n_blocks), 48 bytes each."""
    tab = np.zeros((len(rows), 6), dtype=np.int64)
    for i, (x, codes, norms, signs, out, n) in enumerate(rows):
        tab[i] = [t.data_ptr() if t is not None else 0 for t in (x, codes, norms, signs, out)] + [n]
    return torch.from_numpy(tab).to(device)


def quantize_many(xs, d, bits, signs, packed=False, outs=None):
    """Quantize many tensors (same codec, no QJL stage) in one launch (pq_quantize_many).

    xs: list of fp32 or bf16 device tensors (one dtype), each of numel a multiple of d;
    signs: list of uint8 [d/8] sign masks, one per tensor.  Returns [(codes, norms)], codes
    uint8 [n, d] (or [n, d * bits / 8] with ``packed``), norms fp16 [n]; ``outs`` may hold them
    preallocated."""
    if len(xs) != len(signs) or (outs is not None and len(outs) != len(xs)):
        raise ValueError("one sign mask (and output pair) per tensor")
    if not xs:
        return []
    dev, dt = xs[0].device, xs[0].dtype
    cb = d * bits // 8 if packed else d
    rows, res = [], []
    for i, x in enumerate(xs):
        _dev(x, "xs[%d]" % i, (dt,), device=dev)
        if dt not in (torch.float32, torch.bfloat16):
            raise TypeError("xs must be fp32 or bf16")
        if d <= 0 or x.numel() % d:
            raise ValueError("xs[%d].numel() must be a multiple of d" % i)
        n = x.numel() // d
        _dev(signs[i], "signs[%d]" % i, (torch.uint8,), numel=d // 8, device=dev)
        if outs is None:
            codes = torch.empty((n, cb), dtype=torch.uint8, device=dev)
            norms = torch.empty((n,), dtype=torch.float16, device=dev)
        else:
            codes, norms = outs[i]
        _dev(codes, "codes[%d]" % i, (torch.uint8,), numel=n * cb, device=dev)
        _dev(norms, "norms[%d]" % i, (torch.float16,), numel=n, device=dev)
        rows.append((x, codes, norms, signs[i], None, n))
        res.append((codes, norms))
    tab = _tensor_table(rows, dev)
    _check(_lib.pq_quantize_many(d, bits, PQ_BF16 if dt == torch.bfloat16 else PQ_F32, 1 if packed else 0, len(xs),
                                 _ptr(tab), _stream()), "pq_quantize_many")
    return res


def dequantize_many(codes, norms, d, bits, signs, out_dtype=torch.bfloat16, packed=False, outs=None):
    """Dequantize many tensors in one launch (pq_dequantize_many): lists of codes, norms and sign
    masks, one entry per tensor; returns a list of [n, d] tensors of out_dtype (or fills ``outs``)."""
    if not (len(codes) == len(norms) == len(signs)) or (outs is not None and len(outs) != len(codes)):
        raise ValueError("one codes, norms and sign mask (and output) per tensor")
    if not codes:
        return []
    dev = norms[0].device
    cb = d * bits // 8 if packed else d
    rows, res = [], []
    for i in range(len(codes)):
        _dev(norms[i], "norms[%d]" % i, (torch.float16,), device=dev)
        n = norms[i].numel()
        _dev(codes[i], "codes[%d]" % i, (torch.uint8,), numel=n * cb, device=dev)
        _dev(signs[i], "signs[%d]" % i, (torch.uint8,), numel=d // 8, device=dev)
        out = torch.empty((n, d), dtype=out_dtype, device=dev) if outs is None else outs[i]
        _dev(out, "out[%d]" % i, (out_dtype,), numel=n * d, device=dev)
        if out_dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("out_dtype must be fp32 or bf16")
        rows.append((None, codes[i], norms[i], signs[i], out, n))
        res.append(out)
    tab = _tensor_table(rows, dev)
    _check(_lib.pq_dequantize_many(d, bits, PQ_BF16 if out_dtype == torch.bfloat16 else PQ_F32, 1 if packed else 0,
                                   len(codes), _ptr(tab), _stream()), "pq_dequantize_many")
    return res


def qjl_sketch(keys, proj, out=None, split=None):
    """keys bf16 [..., d]; returns (bits uint8 [n, m/8], norms fp16 [n]).

    ``split`` = (idx, seq_len, group_size, part) sketches one part of each key split by its
    group's outlier channels (qjl_sketch_split): part 0 without them, part 1 only them;
    keys are then [heads, seq_len, d] and idx as from ``qjl_outlier_channels``."""
    _dev(keys, "keys", (torch.bfloat16,))
    dev = keys.device
    _dev(proj, "proj", (torch.bfloat16,), device=dev)
    if proj.dim() != 2:
        raise ValueError("proj must be [m, d]")
    m, d = proj.shape
    if keys.numel() % d:
        raise ValueError("keys.numel() must be a multiple of d")
    n = keys.numel() // d
    if out is None:
        bits = torch.empty((n, m // 8), dtype=torch.uint8, device=dev)
        norms = torch.empty((n,), dtype=torch.float16, device=dev)
    else:
        bits, norms = out
    _dev(bits, "bits", (torch.uint8,), numel=n * (m // 8), device=dev)
    _dev(norms, "norms", (torch.float16,), numel=n, device=dev)
    if split is None:
        _check(_lib.qjl_sketch(d, m, _ptr(keys), n, _ptr(proj), _ptr(bits), _ptr(norms), _stream()), "qjl_sketch")
    else:
        idx, seq_len, group_size, part = split
        if seq_len <= 0 or n % seq_len or group_size <= 0:
            raise ValueError("keys are not [heads, seq_len, d]")
        heads = n // seq_len
        n_out = idx.shape[-1]
        _dev(idx, "idx", (torch.uint8,), numel=heads * (-(-seq_len // group_size)) * n_out, device=dev)
        _check(_lib.qjl_sketch_split(d, m, _ptr(keys), heads, seq_len, group_size, n_out, _ptr(idx),
                                     part, _ptr(proj), _ptr(bits), _ptr(norms), _stream()), "qjl_sketch_split")
    return bits, norms


def qjl_outlier_channels(keys, group_size, n_out, out=None):
    """keys bf16 [..., seq_len, d] -> uint8 [..., ceil(seq_len / group_size), n_out]: per group of
    group_size consecutive tokens, the n_out channels of largest norm, decreasing."""
    _dev(keys, "keys", (torch.bfloat16,))
    if keys.dim() < 2 or group_size <= 0:
        raise ValueError("keys must be [..., seq_len, d] and group_size positive")
    seq_len, d = keys.shape[-2], keys.shape[-1]
    heads = keys.numel() // (seq_len * d) if seq_len * d else 0
    n_groups = (seq_len + group_size - 1) // group_size
    if out is None:
        out = torch.empty(tuple(keys.shape[:-2]) + (n_groups, n_out), dtype=torch.uint8, device=keys.device)
    _dev(out, "out", (torch.uint8,), numel=heads * n_groups * n_out, device=keys.device)
    _check(_lib.qjl_outlier_channels(d, _ptr(keys), heads, seq_len, group_size, n_out, _ptr(out), _stream()),
           "qjl_outlier_channels")
    return out


def qjl_project(q, proj, out=None):
    """Project queries q (bf16 [..., d]) through G: fp32 [n_q, m]."""
    _dev(q, "q", (torch.bfloat16,))
    _dev(proj, "proj", (torch.bfloat16,), device=q.device)
    if proj.dim() != 2:
        raise ValueError("proj must be [m, d]")
    m, d = proj.shape
    if q.numel() % d:
        raise ValueError("q.numel() must be a multiple of d")
    nq = q.numel() // d
    if out is None:
        out = torch.empty((nq, m), dtype=torch.float32, device=q.device)
    _dev(out, "out", (torch.float32,), numel=nq * m, device=q.device)
    _check(_lib.qjl_project(d, m, _ptr(q), nq, _ptr(proj), _ptr(out), _stream()), "qjl_project")
    return out


def qjl_score(sq, bits, norms, batch, kv_heads, q_heads, n_keys, out=None, accumulate=False):
    """QJL scores [batch, q_heads, n_keys] fp32 from projected queries and packed key bits;
    ``accumulate`` adds them to ``out`` (qjl_score_add)."""
    _dev(sq, "sq", (torch.float32,))
    dev = sq.device
    m = sq.shape[-1]
    _dev(sq, "sq", (torch.float32,), numel=batch * q_heads * m)
    _dev(bits, "bits", (torch.uint8,), numel=batch * kv_heads * n_keys * (m // 8), device=dev)
    _dev(norms, "norms", (torch.float16,), numel=batch * kv_heads * n_keys, device=dev)
    if accumulate and out is None:
        raise ValueError("accumulate needs out")
    if out is None:
        out = torch.empty((batch, q_heads, n_keys), dtype=torch.float32, device=dev)
    _dev(out, "out", (torch.float32,), numel=batch * q_heads * n_keys, device=dev)
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
    if q.dim() != 3:
        raise ValueError("q must be [n_heads, n_q, d]")
    n_heads, n_q, d = q.shape
    dev = q.device
    _dev(signs, "signs", (torch.uint8,), numel=d // 8, device=dev)
    m = 0
    if proj is not None:
        _dev(proj, "proj", (torch.bfloat16,), device=dev)
        m = _proj_shape(proj, d)
    need = query_prep_bytes(d, m, n_heads)
    if out is None:
        out = torch.empty((need,), dtype=torch.uint8, device=dev)
    _dev(out, "out", (torch.uint8,), min_numel=need, device=dev)
    _check(_lib.pq_query_prep(d, m, n_heads, n_q, _ptr(q), _ptr(signs), _ptr(proj), _ptr(out), _stream()),
           "pq_query_prep")
    return out


def prep_views(prep, d, m, n_heads):
    """(qrot fp32 [n_heads, 16, d], sq fp32 [n_heads, 16, m]) views of a prepared-query buffer."""
    per = query_prep_bytes(d, m, 1)
    heads = prep[:per * n_heads].view(n_heads, per)
    qrot = heads[:, :16 * d * 4].contiguous().view(torch.float32).view(n_heads, 16, d)
    sq = heads[:, 16 * d * 4:16 * (d + m) * 4].contiguous().view(torch.float32).view(n_heads, 16, m)
    return qrot, sq


def score(prep, codes, norms, d, bits, n_heads, n_q, n_tok, qjl_bits=None, rnorms=None, m=0, out=None,
          packed=False):
    """Two-stage scores fp32 [n_heads, n_q, n_tok] from codes [n_heads, n_tok, d] (or bit-packed,
    d * bits / 8 bytes per token, with ``packed``: pq_score_packed), norms, and (with m > 0)
    the QJL residual bits and residual norms."""
    _dev(codes, "codes", (torch.uint8,), numel=n_heads * n_tok * (d * bits // 8 if packed else d))
    dev = codes.device
    _dev(prep, "prep", (torch.uint8,), min_numel=query_prep_bytes(d, m, n_heads), device=dev)
    _dev(norms, "norms", (torch.float16,), numel=n_heads * n_tok, device=dev)
    if m:
        _dev(qjl_bits, "qjl_bits", (torch.uint8,), numel=n_heads * n_tok * (m // 8), device=dev)
        _dev(rnorms, "rnorms", (torch.float16,), numel=n_heads * n_tok, device=dev)
    if out is None:
        out = torch.empty((n_heads, n_q, n_tok), dtype=torch.float32, device=dev)
    _dev(out, "out", (torch.float32,), numel=n_heads * n_q * n_tok, device=dev)
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


def _attention_inputs(prep, keys, values, v_signs, d, bits, n_heads, n_q, n_tok, m, k_win, v_win, q, packed, out):
    """Checks shared by ``attention`` and ``attention_noalloc``; returns (n_win, out)."""
    k_codes, k_norms, k_bits, k_rn = keys
    v_codes, v_norms = values
    _dev(v_codes, "v_codes", (torch.uint8,))
    dev = v_codes.device
    cb = d * bits // 8 if packed else d
    for t, name in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _dev(t, name, (torch.uint8,), numel=n_heads * n_tok * cb, device=dev)
    _dev(k_norms, "k_norms", (torch.float16,), numel=n_heads * n_tok, device=dev)
    _dev(v_norms, "v_norms", (torch.float16,), numel=n_heads * n_tok, device=dev)
    _dev(v_signs, "v_signs", (torch.uint8,), numel=d // 8, device=dev)
    if n_tok:
        _dev(prep, "prep", (torch.uint8,), min_numel=query_prep_bytes(d, m, n_heads), device=dev)
    if m:
        _dev(k_bits, "k_qjl_bits", (torch.uint8,), numel=n_heads * n_tok * (m // 8), device=dev)
        _dev(k_rn, "k_rnorms", (torch.float16,), numel=n_heads * n_tok, device=dev)
    n_win = 0
    if k_win is not None:
        _dev(k_win, "k_win", (torch.bfloat16,), device=dev)
        _dev(v_win, "v_win", (torch.bfloat16,), device=dev)
        _dev(q, "q", (torch.bfloat16,), device=dev)
        if k_win.dim() != 3:
            raise ValueError("k_win must be [n_heads, n_win, d]")
        n_win = k_win.shape[1]
        if k_win.shape != (n_heads, n_win, d) or v_win.shape != k_win.shape or q.shape != (n_heads, n_q, d):
            raise ValueError("window or query shape does not match n_heads, n_q, d")
    if out is None:
        out = torch.empty((n_heads, n_q, d), dtype=torch.float32, device=dev)
    _dev(out, "out", (torch.float32,), numel=n_heads * n_q * d, device=dev)
    return n_win, out


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
    n_win, out = _attention_inputs(prep, keys, values, v_signs, d, bits, n_heads, n_q, n_tok, m, k_win, v_win, q,
                                   packed, out)
    k_codes, k_norms, k_bits, k_rn = keys
    v_codes, v_norms = values
    if sm_scale is None:
        sm_scale = 1.0 / float(d) ** 0.5
    need = attention_work_bytes(d, n_heads, n_tok)
    if work is None:
        work = torch.empty((max(16, need),), dtype=torch.uint8, device=out.device)
    _dev(work, "work", (torch.uint8,), min_numel=need, device=out.device)
    fn, name = (_lib.pq_attention_packed, "pq_attention_packed") if packed else (_lib.pq_attention, "pq_attention")
    _check(fn(d, bits, m, n_heads, n_q, n_tok, _ptr(prep), _ptr(k_codes), _ptr(k_norms), _ptr(k_bits), _ptr(k_rn),
              _ptr(v_codes), _ptr(v_norms), _ptr(v_signs), n_win, _ptr(k_win), _ptr(v_win), _ptr(q),
              float(sm_scale), _ptr(work), _ptr(out), _stream()), name)
    return out


def attention_noalloc(prep, keys, values, v_signs, d, bits, n_heads, n_q, n_tok, m=0, k_win=None, v_win=None,
                      q=None, sm_scale=None, packed=False, out=None):
    """``attention`` through pq_attention_noalloc: no work buffer is allocated or passed; the
    library's fixed device array serves (calls overlapping on one device race).  ``out`` may be
    preallocated (fp32 [n_heads, n_q, d]); nothing else is allocated when it is."""
    n_win, out = _attention_inputs(prep, keys, values, v_signs, d, bits, n_heads, n_q, n_tok, m, k_win, v_win, q,
                                   packed, out)
    k_codes, k_norms, k_bits, k_rn = keys
    v_codes, v_norms = values
    if sm_scale is None:
        sm_scale = 1.0 / float(d) ** 0.5
    _check(_lib.pq_attention_noalloc(d, bits, m, n_heads, n_q, n_tok, _ptr(prep), _ptr(k_codes), _ptr(k_norms),
                                     _ptr(k_bits), _ptr(k_rn), _ptr(v_codes), _ptr(v_norms), _ptr(v_signs), n_win,
                                     _ptr(k_win), _ptr(v_win), _ptr(q), float(sm_scale), 1 if packed else 0,
                                     _ptr(out), _stream()), "pq_attention_noalloc")
    return out


def quantize_bd(x, d, bits, signs, out=None):
    """Codec with the block-diagonal rotation, for block sizes d that are not powers of two
    (any multiple of 32 in 64..4096): x fp32 or bf16 with numel a multiple of d.
    Returns (codes uint8 [n_blocks, d], norms fp16 [n_blocks])."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    dev = x.device
    _dev(signs, "signs", (torch.uint8,), numel=d // 8, device=dev)
    if d <= 0 or x.numel() % d:
        raise ValueError("x.numel() must be a multiple of d")
    n = x.numel() // d
    if out is None:
        out = (torch.empty((n, d), dtype=torch.uint8, device=dev), torch.empty((n,), dtype=torch.float16, device=dev))
    codes, norms = out
    _dev(codes, "codes", (torch.uint8,), numel=n * d, device=dev)
    _dev(norms, "norms", (torch.float16,), numel=n, device=dev)
    _check(_lib.pq_quantize_bd(d, bits, PQ_BF16 if x.dtype == torch.bfloat16 else PQ_F32, _ptr(x), n,
                               _ptr(signs), _ptr(codes), _ptr(norms), _stream()), "pq_quantize_bd")
    return codes, norms


def dequantize_bd(codes, norms, d, bits, signs, out_dtype=torch.bfloat16, out=None):
    """Inverse of ``quantize_bd``: [n_blocks, d] of out_dtype (fp32 or bf16)."""
    _dev(norms, "norms", (torch.float16,))
    dev = norms.device
    n = norms.numel()
    _dev(codes, "codes", (torch.uint8,), numel=n * d, device=dev)
    _dev(signs, "signs", (torch.uint8,), numel=d // 8, device=dev)
    if out is None:
        out = torch.empty((n, d), dtype=out_dtype, device=dev)
    _dev(out, "out", (torch.float32, torch.bfloat16), numel=n * d, device=dev)
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
    dev = x.device
    _dev(rot, "rot", (torch.float32,), numel=d * d, device=dev)
    if d <= 0 or x.numel() % d:
        raise ValueError("x.numel() must be a multiple of d")
    n = x.numel() // d
    if out is None:
        out = (torch.empty((n, d), dtype=torch.uint8, device=dev), torch.empty((n,), dtype=torch.float16, device=dev))
    codes, norms = out
    _dev(codes, "codes", (torch.uint8,), numel=n * d, device=dev)
    _dev(norms, "norms", (torch.float16,), numel=n, device=dev)
    _check(_lib.pq_quantize_dense(d, bits, PQ_BF16 if x.dtype == torch.bfloat16 else PQ_F32, _ptr(x), n, _ptr(rot),
                                  _ptr(codes), _ptr(norms), _stream()), "pq_quantize_dense")
    return codes, norms


def dequantize_dense(codes, norms, d, bits, rot, out_dtype=torch.bfloat16, out=None):
    """Inverse of ``quantize_dense``: [n_blocks, d] of out_dtype (fp32 or bf16)."""
    _dev(norms, "norms", (torch.float16,))
    dev = norms.device
    n = norms.numel()
    _dev(codes, "codes", (torch.uint8,), numel=n * d, device=dev)
    _dev(rot, "rot", (torch.float32,), numel=d * d, device=dev)
    if out is None:
        out = torch.empty((n, d), dtype=out_dtype, device=dev)
    _dev(out, "out", (torch.float32, torch.bfloat16), numel=n * d, device=dev)
    _check(_lib.pq_dequantize_dense(d, bits, _ptr(codes), _ptr(norms), n, _ptr(rot),
                                    PQ_BF16 if out.dtype == torch.bfloat16 else PQ_F32, _ptr(out), _stream()),
           "pq_dequantize_dense")
    return out


def probe_stream(src, out=None):
    """Bandwidth probe (pq_probe_stream): ``src`` uint8 [n] -> int16 [n], each byte
    zero-extended; the memory traffic of dequantize with none of its arithmetic."""
    _dev(src, "src", (torch.uint8,))
    n = src.numel()
    if out is None:
        out = torch.empty((n,), dtype=torch.int16, device=src.device)
    _dev(out, "out", (torch.int16,), numel=n, device=src.device)
    _check(_lib.pq_probe_stream(_ptr(src), _ptr(out), n, _stream()), "pq_probe_stream")
    return out
