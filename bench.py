"""Benchmark of the codec hot path on one MI355X.

One step = quantize (rotate, Lloyd-Max codes, fp16 norms, QJL residual signs
and norms) + dequantize of one 4096 x 4096 bf16 weight (d = 128, 5-bit codes,
m = 64 residual projections), all inputs resident in HBM.  Eight buffer sets
are rotated so that no step finds its data in the 256 MB Infinity Cache.

Prints one JSON line.  ``value`` is input bytes / (quantize + dequantize
kernel time), in GB/s.  ``parts`` adds the QJL half of the metric on the
config-4 key cache: sketch and score rates in keys/s.  The roofline entry is for the quantize kernel:
algorithmic bytes per launch (input read + codes, norms, sign bits and residual
norms written) over its average duration measured with HIP events on the
stream the kernels run on.  ``cpu_baseline`` times the oracle on the host on a
bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
N_SETS = 8


def _args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-sample-blocks", type=int, default=131072,
                    help="blocks of the workload the oracle baseline processes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-qjl", action="store_true", help="skip the config-4 QJL sketch/score leg")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    return ap.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("pq_kernels.hip", "pq_device.h", "pq_internal.h", "pq_api.cpp"):
        with open(os.path.join(ROOT, "kv_cache_quantization_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel_name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when
    the summary is missing or was taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", "pq_quantize_config2_counters.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel_name)
    return None if k is None else k.get("hbm_bytes_per_launch")


def cpu_baseline(n_blocks):
    """Time the oracle (quantize + QJL residual + dequantize) on the first n_blocks of
    the workload, on the host cores; returns the record for the JSON line."""
    import synth
    import oracle
    from oracle import numerics, hadamard
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    c = synth.config2()
    d, bits = c["d"], c["bits"]
    x = numerics.bf16_from_bits(c["x"].reshape(-1, d)[:n_blocks])
    D = hadamard.signs_from_mask(c["signs"], d)
    G = numerics.bf16_from_bits(c["G"])
    t0 = time.perf_counter()
    q = oracle.codec.quantize(x, bits, D)
    r = oracle.codec.qjl_residual(x, q["codes"], q["n16"], bits, D, G)
    xh = oracle.codec.dequantize(q["codes"], q["n16"], bits, D)
    dt = time.perf_counter() - t0
    assert r["bits"].shape[0] == n_blocks and xh.shape == x.shape
    in_bytes = n_blocks * d * 2
    return {"value": round(in_bytes / dt / 1e9, 6), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": "first %d of 131072 blocks of the 4096x4096 weight (%.1f MB of bf16 input), "
                      "quantize + QJL residual + dequantize, %.2f s" % (n_blocks, in_bytes / 1e6, dt)}


def qjl_leg(pq, synth, torch, steps, warmup):
    """Config 4: QJL sketch of the 4x8x32768x128 bf16 key cache (m=256), then the
    GQA score of one query token (32 heads) against every key.  Returns the timings
    and rates for the JSON line."""
    c = synth.config4()
    B, Hkv, T, d = c["keys"].shape
    Hq, m = c["q"].shape[1], c["m"]
    n_keys = B * Hkv * T
    dev = torch.device("cuda:0")
    keys_host = torch.from_numpy(c["keys"].view(np.int16)).view(torch.bfloat16)
    G = torch.from_numpy(c["G"].view(np.int16)).view(torch.bfloat16).to(dev)
    q = torch.from_numpy(c["q"].view(np.int16)).view(torch.bfloat16).to(dev)
    key_sets = [keys_host.to(dev) for _ in range(2)]          # 2 x 256 MiB: beyond the last-level cache
    bits0, norms0 = pq.qjl_sketch(key_sets[0], G)
    sketch_out = [(torch.empty_like(bits0), torch.empty_like(norms0)) for _ in range(2)]
    score_in = [(bits0.clone(), norms0.clone()) for _ in range(N_SETS)]   # 8 x 34 MiB of bits and norms
    sq = pq.qjl_project(q, G)
    scores = [torch.empty((B, Hq, T), dtype=torch.float32, device=dev) for _ in range(2)]
    for k in range(warmup):
        pq.qjl_sketch(key_sets[k % 2], G, out=sketch_out[k % 2])
        pq.qjl_score(pq.qjl_project(q, G, out=sq), *score_in[k % N_SETS], B, Hkv, Hq, T, out=scores[k % 2])
    big = torch.randn(8192, 8192, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    _ = big @ big
    for k in range(steps):
        ev[k][0].record()
        pq.qjl_sketch(key_sets[k % 2], G, out=sketch_out[k % 2])
        ev[k][1].record()
        pq.qjl_project(q, G, out=sq)
        ev[k][2].record()
        pq.qjl_score(sq, *score_in[k % N_SETS], B, Hkv, Hq, T, out=scores[k % 2])
        ev[k][3].record()
    torch.cuda.synchronize()
    t_sk = float(np.mean([ev[k][0].elapsed_time(ev[k][1]) for k in range(steps)])) * 1e-3
    t_pr = float(np.mean([ev[k][1].elapsed_time(ev[k][2]) for k in range(steps)])) * 1e-3
    t_sc = float(np.mean([ev[k][2].elapsed_time(ev[k][3]) for k in range(steps)])) * 1e-3
    sk_bytes = n_keys * d * 2 + n_keys * (m // 8) + n_keys * 2
    sc_bytes = n_keys * (m // 8) + n_keys * 2 + B * Hq * T * 4 + B * Hq * m * 4
    sk_flops = 2.0 * n_keys * d * m
    return {
        "qjl_config": "config4: keys 4x8x32768x128 bf16, m=256, 32 query heads (GQA 4:1)",
        "qjl_sketch_us": round(t_sk * 1e6, 3), "qjl_sketch_keys_per_s": round(n_keys / t_sk, 1),
        "qjl_sketch_hbm_frac": round(sk_bytes / t_sk / 1e9 / HBM_PEAK_GBS, 4),
        "qjl_sketch_mfma_frac": round(sk_flops / t_sk / 1e12 / BF16_PEAK_TFLOPS, 4),
        "qjl_project_us": round(t_pr * 1e6, 3),
        "qjl_score_us": round(t_sc * 1e6, 3), "qjl_score_keys_per_s": round(n_keys / t_sc, 1),
        "qjl_score_hbm_frac": round(sc_bytes / t_sc / 1e9 / HBM_PEAK_GBS, 4),
        "qjl_sketch_algorithmic_bytes": sk_bytes, "qjl_score_algorithmic_bytes": sc_bytes,
    }


def main():
    args = _args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported "
              "(the codec shards by blocks with no exchange, see DESIGN.md)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_cache_quantization_amd as pq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        nbytes = 512 << 20
        a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": nbytes, "bytes_written": nbytes,
                          "launches": 5}))
        return

    c = synth.config2()
    d, bits, m = c["d"], c["bits"], c["m"]
    n_blocks = c["x"].size // d
    x_host = torch.from_numpy(c["x"].view(np.int16)).view(torch.bfloat16)
    signs = torch.from_numpy(c["signs"]).to(dev)
    proj = torch.from_numpy(c["G"].view(np.int16)).view(torch.bfloat16).to(dev)

    sets = []
    for _ in range(N_SETS):
        x = x_host.to(dev)
        codes = torch.empty((n_blocks, d), dtype=torch.uint8, device=dev)
        norms = torch.empty((n_blocks,), dtype=torch.float16, device=dev)
        qb = torch.empty((n_blocks, m // 8), dtype=torch.uint8, device=dev)
        rn = torch.empty((n_blocks,), dtype=torch.float16, device=dev)
        out = torch.empty((n_blocks, d), dtype=torch.bfloat16, device=dev)
        sets.append((x, codes, norms, qb, rn, out))

    def step(k, evs=None):
        x, codes, norms, qb, rn, out = sets[k % N_SETS]
        if evs is not None:
            evs[0].record()
        pq.quantize(x, d, bits, signs, proj, out=(codes, norms, qb, rn))
        if evs is not None:
            evs[1].record()
        pq.dequantize(codes, norms, d, bits, signs, out=out)
        if evs is not None:
            evs[2].record()

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    # keep the GPU busy while the timed steps are enqueued, so that no kernel waits for its launch
    big = torch.randn(8192, 8192, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    _ = big @ big
    for k in range(args.steps):
        step(k, evs[k])
    torch.cuda.synchronize()

    tq = np.array([evs[k][0].elapsed_time(evs[k][1]) for k in range(args.steps)]) * 1e-3   # s
    td = np.array([evs[k][1].elapsed_time(evs[k][2]) for k in range(args.steps)]) * 1e-3
    total = evs[0][0].elapsed_time(evs[-1][2]) * 1e-3
    t_q, t_d = float(np.mean(tq)), float(np.mean(td))

    in_bytes = n_blocks * d * 2
    q_bytes = in_bytes + n_blocks * d + n_blocks * 2 + n_blocks * (m // 8) + n_blocks * 2
    dq_bytes = n_blocks * d + n_blocks * 2 + in_bytes
    value = in_bytes / (t_q + t_d) / 1e9
    q_gbs = q_bytes / t_q / 1e9
    traffic = counter_traffic("pq_quantize_kernel")

    rec = {
        "metric": "quantize+dequantize GB/s and % HBM peak; QJL score keys/s at 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0, 0.02^2) weight with 0.1% outlier entries x10",
        "config": {"workload": "config2: one 4096x4096 bf16 weight, d=128 blocks, 5-bit Lloyd-Max codes, "
                               "QJL residual m=64; quantize then dequantize",
                   "n_blocks": n_blocks, "d": d, "bits": bits, "m": m, "buffer_sets": N_SETS},
        "parts": {
            "quantize_us": round(t_q * 1e6, 3), "dequantize_us": round(t_d * 1e6, 3),
            "quantize_hbm_frac": round(q_gbs / HBM_PEAK_GBS, 4),
            "dequantize_hbm_frac": round(dq_bytes / t_d / 1e9 / HBM_PEAK_GBS, 4),
            "quantize_algorithmic_bytes": q_bytes, "dequantize_algorithmic_bytes": dq_bytes,
        },
        "roofline": {"bound": "hbm", "achieved": round(q_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(q_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "pq_quantize_kernel<128, bf16, qjl>",
                     "algorithmic_bytes_per_launch": q_bytes},
        "kernel_source": kernel_source_hash(),
    }
    if not args.no_qjl:
        rec["parts"].update(qjl_leg(pq, synth, torch, args.steps, args.warmup))
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(args.cpu_sample_blocks)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
