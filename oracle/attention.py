"""Decode attention over a quantized KV cache with an unquantized recent window, plain float64.

Test infrastructure (see the package docstring).

eliza quantization README, "TurboQuant": the cache keeps codes and norms per key and value
vector; at attention time the codes go through centroid lookup and the inverse rotation; the
most recent residual_length tokens are kept unquantized.  "Fused TurboQuant (Triton)": Q K^T is
scored straight from the stored codes.  glq 0.7.2 README, "Inline-dequant E8 KV": decoding the
compressed K/V inside the attention kernel, each vector read once, instead of into a workspace.

What is computed, for one KV head and one query row q (length d):
    s_t = estimate of <q, k_t>   for the T quantized tokens (the codec's first stage, plus the
                                 QJL residual term when the keys carry one: ``qjl.two_stage``),
    s_w = <q, k_w>               for the W window tokens (exact),
    p   = softmax(scale . [s_t ; s_w]),
    o   = sum_t p_t vhat_t + sum_w p_w v_w,   vhat_t = ``codec.dequantize`` of the value codes.

Readings where the pages leave a step open:
  * one code width for keys and values (the pages' cache takes a single nbits); values carry no
    QJL residual (only the inner products with keys use it);
  * keys and values of a head use their own sign masks D_k and D_v;
  * the window is held in the cache's input dtype (bf16 values here);
  * scale defaults to 1/sqrt(d);
  * token order does not matter to the result (softmax pairs each key with its value): the
    quantized tokens come first, the window after them.
"""

import numpy as np

from . import codec, qjl


def key_scores(q, k_codes, k_n16, bits, D_k, k_qbits=None, k_rn16=None, G=None):
    """Scores of queries q (nq, d) against T quantized keys: (est (nq, T), L1 scale (nq, T)).

    With a QJL residual (k_qbits, k_rn16, G given) the two-stage estimate, else <q, xhat>."""
    q = np.asarray(q, dtype=np.float64)
    if G is not None:
        return qjl.two_stage(k_codes, k_n16, k_qbits, k_rn16, q, bits, D_k, G)
    khat = codec.dequantize(k_codes, k_n16, bits, D_k)
    return q @ khat.T, np.abs(q) @ np.abs(khat).T


def decode_attention(q, k_codes, k_n16, v_codes, v_n16, bits, D_k, D_v, k_win=None, v_win=None,
                     scale=None, k_qbits=None, k_rn16=None, G=None):
    """Attention output of the query rows q (nq, d) of one KV head.

    k_codes, v_codes (T, d) codes; k_n16, v_n16 (T,) fp16 norms as float64; k_win, v_win (W, d)
    float64 (None for W = 0).  Returns a dict with ``out`` (nq, d), the probabilities ``p``
    (nq, T + W), the logits ``z`` (nq, T + W), the L1 scale of the quantized scores
    ``score_l1`` (nq, T) and the value rows ``v`` (T + W, d) in the order of ``p``.
    """
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    T = np.asarray(k_codes).shape[0]
    W = 0 if k_win is None else np.asarray(k_win).shape[0]
    if T + W == 0:
        raise ValueError("attention over an empty cache")
    if T:
        s_q, l1 = key_scores(q, k_codes, k_n16, bits, D_k, k_qbits, k_rn16, G)
        vhat = codec.dequantize(v_codes, v_n16, bits, D_v)
    else:
        s_q, l1 = np.zeros((q.shape[0], 0)), np.zeros((q.shape[0], 0))
        vhat = np.zeros((0, d))
    if W:
        k_win = np.asarray(k_win, dtype=np.float64)
        s_w = q @ k_win.T
        values = np.concatenate([vhat, np.asarray(v_win, dtype=np.float64)], axis=0)
    else:
        s_w = np.zeros((q.shape[0], 0))
        values = vhat
    z = scale * np.concatenate([s_q, s_w], axis=1)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    return {"out": p @ values, "p": p, "z": z, "score_l1": l1, "v": values}
