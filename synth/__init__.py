"""Seeded synthetic inputs for the codec, shared by the oracle side and the GPU side.

This module holds none of the method's arithmetic: it only draws random
numbers and casts them to the storage dtypes.  The random quantities the
method itself draws (the +-1 rotation signs D and the Gaussian JL matrix G) are
not drawn here: a config names their seeds, and each side rebuilds them with
its own implementation of the same counter-based generator (the library's
pq_make_signs / qjl_make_projection for the GPU side, ``oracle.seeds`` for the
oracle side).

Every data array comes from numpy's PCG64 seeded with ``SeedSequence([seed, tag])``,
so each (seed, purpose) pair is an independent, reproducible stream.

Workload recipes (sizes and distributions of the pages' workloads):
  config 1  one fp32 weight 256x512, N(0, 0.02^2), data seed 0, d=128, 4-bit.
  config 2  one bf16 weight 4096x4096, N(0, 0.02^2) with 0.1% of the entries
            (floor(0.001 N) distinct seeded positions) multiplied by 10, d=128,
            5-bit, QJL m=64.
  config 3  a 7B-style decoder weight set: 32 layers x {q 4096x4096,
            k 1024x4096, v 1024x4096, o 4096x4096, gate 14336x4096,
            up 14336x4096, down 4096x14336}, bf16 N(0, 0.02^2), 8 seeded input
            columns per tensor multiplied by 8, d=128, 4-bit; tensor t (model
            order, layer-major) uses rotation seed base+t.
  config 4  bf16 keys [4][8][32768][128], N(0,1) with 4 seeded channels per KV
            head multiplied by 20 (same channels for every batch row and token),
            G with m=256, one query token with 32 heads (GQA 4:1), N(0,1).
  config 5  bf16 KV vectors [8][65536][256] and [8][65536][512], N(0,1) times a
            per-(head, channel) scale exp(z), z ~ N(0,1); 3-bit, QJL m=d; 16
            N(0,1) queries per KV head per tensor.
Keys and weights stand in for model activations and checkpoints; no dataset
or trained weight is read.
"""

import numpy as np

TAG_DATA, TAG_SIGNS, TAG_PROJ, TAG_OUTLIER, TAG_QUERY, TAG_SCALE = 1, 2, 3, 4, 5, 6
BASE_SEED = 42          # rotation / projection seed base; tensor t uses BASE_SEED + t
OUTLIER_PROJ_SEED = BASE_SEED + 1000    # the outlier channels' own projection (config-4 shape)


def rng(seed, tag):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tag)])))


def bf16_from_f32(a):
    """float32 array -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(u):
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gaussian_bf16(seed, tag, shape, std=1.0):
    g = rng(seed, tag).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        g *= np.float32(std)
    return bf16_from_f32(g)


# ----------------------------------------------------------------------------- configs

def config1(seed=0):
    x = rng(seed, TAG_DATA).standard_normal((256, 512), dtype=np.float32) * np.float32(0.02)
    return {"name": "config1", "x": x, "dtype": "f32", "d": 128, "bits": 4, "m": 0,
            "sign_seed": BASE_SEED}


def weight_with_outlier_entries(seed, rows, cols, frac=0.001, factor=10.0, std=0.02):
    g = rng(seed, TAG_DATA).standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    n = rows * cols
    k = int(np.floor(frac * n))
    pos = rng(seed, TAG_OUTLIER).choice(n, size=k, replace=False)
    flat = g.reshape(-1)
    flat[pos] *= np.float32(factor)
    return bf16_from_f32(g), np.sort(pos)


def config2(seed=0, rows=4096, cols=4096):
    x, pos = weight_with_outlier_entries(seed, rows, cols)
    return {"name": "config2", "x": x, "dtype": "bf16", "d": 128, "bits": 5, "m": 64,
            "sign_seed": BASE_SEED, "proj_seed": BASE_SEED,
            "outlier_positions": pos}


CONFIG3_SHAPES = (("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
                  ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336))


def config3_layout(n_layers=32):
    """[(tensor index, layer, name, rows, cols)] in model order."""
    out = []
    t = 0
    for layer in range(n_layers):
        for name, r, c in CONFIG3_SHAPES:
            out.append((t, layer, name, r, c))
            t += 1
    return out


def config3_tensor(t, rows, cols, seed=0, n_cols_out=8, factor=8.0):
    """Tensor t of config 3: bf16 N(0, 0.02^2), 8 seeded input columns scaled by 8.
    Returns (bf16 bits, rotation sign seed)."""
    s = seed * 1000 + t
    g = rng(s, TAG_DATA).standard_normal((rows, cols), dtype=np.float32) * np.float32(0.02)
    colsel = rng(s, TAG_OUTLIER).choice(cols, size=n_cols_out, replace=False)
    g[:, colsel] *= np.float32(factor)
    return bf16_from_f32(g), BASE_SEED + t


def config4(seed=0, batch=4, kv_heads=8, tokens=32768, head_dim=128, q_heads=32, m=256):
    keys = rng(seed, TAG_DATA).standard_normal((batch, kv_heads, tokens, head_dim), dtype=np.float32)
    chans = np.stack([rng(seed * 100 + h, TAG_OUTLIER).choice(head_dim, size=4, replace=False)
                      for h in range(kv_heads)])
    for h in range(kv_heads):
        keys[:, h, :, chans[h]] *= np.float32(20.0)
    q = rng(seed, TAG_QUERY).standard_normal((batch, q_heads, head_dim), dtype=np.float32)
    return {"name": "config4", "keys": bf16_from_f32(keys), "q": bf16_from_f32(q),
            "proj_seed": BASE_SEED, "d": head_dim, "m": m,
            "outlier_channels": chans}


def config5_tensor(d, seed=0, kv_heads=8, tokens=65536, n_q=16):
    """One of the two config-5 tensors: [kv_heads][tokens][d] bf16 with log-normal channel scales."""
    s = seed * 10 + d
    x = rng(s, TAG_DATA).standard_normal((kv_heads, tokens, d), dtype=np.float32)
    scale = np.exp(rng(s, TAG_SCALE).standard_normal((kv_heads, 1, d))).astype(np.float32)
    x *= scale
    q = rng(s, TAG_QUERY).standard_normal((kv_heads, n_q, d), dtype=np.float32)
    return {"x": bf16_from_f32(x), "q": bf16_from_f32(q), "d": d, "bits": 3, "m": d,
            "sign_seed": BASE_SEED + d, "proj_seed": BASE_SEED + d}


def config5_attention(d, seed=0, kv_heads=8, tokens=65536, n_q=16, window=128):
    """Decode-attention inputs on the config-5 recipe: keys and values are two tensors of that
    recipe (seeds ``seed`` and ``seed + 1``, so each has its own channel scales) of
    tokens + window rows per head; the first ``tokens`` rows go to the quantized cache, the last
    ``window`` rows stay unquantized.  Values get their own sign mask."""
    keys = config5_tensor(d, seed, kv_heads, tokens + window, n_q)
    vals = config5_tensor(d, seed + 1, kv_heads, tokens + window, n_q)
    return {"k": np.ascontiguousarray(keys["x"][:, :tokens]), "v": np.ascontiguousarray(vals["x"][:, :tokens]),
            "k_win": np.ascontiguousarray(keys["x"][:, tokens:]), "v_win": np.ascontiguousarray(vals["x"][:, tokens:]),
            "q": keys["q"], "d": d, "bits": keys["bits"], "m": keys["m"], "k_sign_seed": keys["sign_seed"],
            "proj_seed": keys["proj_seed"], "v_sign_seed": BASE_SEED + d + 1}
