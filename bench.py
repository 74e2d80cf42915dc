"""Benchmark of the codec hot path on one MI355X.

One step = quantize (rotate, Lloyd-Max codes, fp16 norms, QJL residual signs
and norms) + dequantize of one 4096 x 4096 bf16 weight (d = 128, 5-bit codes,
m = 64 residual projections), all inputs resident in HBM.  Eight buffer sets
are rotated so that no step finds its data in the 256 MB Infinity Cache.

Prints one JSON line.  ``value`` is input bytes / (quantize + dequantize
kernel time), in GB/s.  ``parts`` adds the QJL half of the metric on the
config-4 key cache (sketch and score rates in keys/s), the config-5 two-stage
path (quantize, dequantize, query preparation, score) and the config-3 grouped
pass over 224 tensors, each with its fraction of the HBM (or matrix-core) peak.  The roofline entry is for the quantize kernel:
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
FP16_PEAK_TFLOPS = 2500.0
N_SETS = 8


def _args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-sample-blocks", type=int, default=32768,
                    help="blocks of the workload the oracle baseline processes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-qjl", action="store_true", help="skip the config-4 QJL sketch/score leg")
    ap.add_argument("--no-tsq", action="store_true", help="skip the config-5 two-stage leg")
    ap.add_argument("--no-grouped", action="store_true", help="skip the config-3 grouped pass")
    ap.add_argument("--no-attn", action="store_true", help="skip the config-5 decode-attention leg")
    ap.add_argument("--no-bd", action="store_true", help="skip the block-diagonal rotation leg (d=2688)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-rotation leg (d=128)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="write the profiles/ summaries from rocprofv3 output under DIR, then exit")
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


def _cpu_model():
    """The host CPU's model name (from /proc/cpuinfo, as lscpu reports it)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(n_blocks, min_seconds=6.0):
    """Time the oracle (quantize + QJL residual + dequantize) on the first n_blocks of the
    workload on the host, twice: with numpy's BLAS held to one thread, then with all of its
    threads (every host core it sees), each pass repeated until min_seconds have elapsed;
    returns the record for the JSON line (value = the all-core rate)."""
    import synth
    import oracle
    from oracle import numerics, seeds
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    c = synth.config2()
    d, bits = c["d"], c["bits"]
    x = numerics.bf16_from_bits(c["x"].reshape(-1, d)[:n_blocks])
    D = seeds.signs(c["sign_seed"], d)
    G = seeds.projection_values(c["proj_seed"], c["m"], d)

    def run():
        reps, dt = 0, 0.0
        while dt < min_seconds:
            t0 = time.perf_counter()
            q = oracle.codec.quantize(x, bits, D)
            r = oracle.codec.qjl_residual(x, q["codes"], q["n16"], bits, D, G)
            xh = oracle.codec.dequantize(q["codes"], q["n16"], bits, D)
            dt += time.perf_counter() - t0
            reps += 1
            assert r["bits"].shape[0] == n_blocks and xh.shape == x.shape
        return reps, dt

    with threadpool_limits(limits=1):
        r1, t1 = run()
    ra, ta = run()
    in_bytes = n_blocks * d * 2
    return {"value": round(in_bytes * ra / ta / 1e9, 6), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "value_1thread": round(in_bytes * r1 / t1 / 1e9, 6), "cpu_model": _cpu_model(),
            "host_cpus": os.cpu_count(),
            "sample": "first %d of 131072 blocks of the 4096x4096 weight (%.1f MB of bf16 input), quantize + QJL "
                      "residual + dequantize in the float64 oracle: %d passes in %.2f s on %d BLAS threads "
                      "(value), %d passes in %.2f s on 1 thread (value_1thread)" % (
                          n_blocks, in_bytes / 1e6, ra, ta, threads, r1, t1)}


def summarize(run_dir):
    """Write the committed profile summaries from the rocprofv3 output of the commands
    listed in them (run_dir holds prof_trace/, pmc_q_fetch/, pmc_q_write/, pmc_c_fetch/,
    pmc_c_write/ as written there)."""
    import csv
    out_dir = os.path.join(ROOT, "profiles")

    def rows(sub, name):
        with open(os.path.join(run_dir, sub, name)) as fh:
            return list(csv.DictReader(fh))

    def short(name):
        return name.replace("void ", "").replace("(anonymous namespace)::", "").split("(pqi::")[0]

    trace_cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/prof_trace -o trace -- "
                 "python3 bench.py --steps 50 --warmup 5 --no-cpu-baseline --no-grouped")
    lines = ["# Kernel durations of the benchmark (config 2 codec, config 4 QJL leg, config 5 two-stage and "
             "decode-attention legs, block-diagonal leg), one MI355X",
             "", "command: " + trace_cmd, "kernel source hash: " + kernel_source_hash(), "",
             "average_ns is rocprofv3's average over every call; median_ns and timed_avg_ns come from the "
             "per-dispatch trace, timed_avg_ns over the calls within 25% of the median (the benchmark's set-up "
             "launches the same kernels at other sizes, e.g. the attention leg quantizes its keys with the "
             "config-2 instantiation)", "",
             "%-58s %6s %12s %10s %12s %10s %10s" % ("kernel", "calls", "average_ns", "median_ns", "timed_avg_ns",
                                                      "min_ns", "max_ns")]
    durs = {}
    for r in rows("prof_trace", "trace_kernel_trace.csv"):
        durs.setdefault(short(r["Kernel_Name"]), []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    for r in rows("prof_trace", "trace_kernel_stats.csv"):
        n = short(r["Name"])
        if any(k in n for k in ("pq_", "qjl_")):
            ds = sorted(durs.get(n, [0]))
            med = ds[len(ds) // 2]
            kept = [x for x in ds if abs(x - med) <= 0.25 * med] or ds
            lines.append("%-58s %6s %12.1f %10d %12.1f %10s %10s" % (n, r["Calls"], float(r["AverageNs"]), med,
                                                                     sum(kept) / len(kept), r["MinNs"], r["MaxNs"]))
    with open(os.path.join(out_dir, "bench_kernels_config2_config4_config5_trace.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")

    def counter(sub, prefix, kernel):
        vals = [float(r["Counter_Value"]) for r in rows(sub, prefix + "_counter_collection.csv")
                if kernel in r["Kernel_Name"]]
        return sum(vals) / len(vals), len(vals)

    copy_bytes = 512 << 20
    cf, _ = counter("pmc_c_fetch", "c_fetch", "__amd_rocclr_copyBuffer")
    cw, _ = counter("pmc_c_write", "c_write", "__amd_rocclr_copyBuffer")
    f_fetch, f_write = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    rec = {"source_hash": kernel_source_hash(),
           "commands": [
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/pmc_q_fetch -o q_fetch -- "
               "python3 bench.py --steps 8 --warmup 2 --no-cpu-baseline --no-qjl --no-tsq --no-grouped --no-attn",
               "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/pmc_q_write -o q_write -- "
               "python3 bench.py --steps 8 --warmup 2 --no-cpu-baseline --no-qjl --no-tsq --no-grouped --no-attn",
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/pmc_a_fetch -o a_fetch -- "
               "python3 bench.py --steps 8 --warmup 2 --no-cpu-baseline --no-qjl --no-tsq --no-grouped",
               "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/pmc_a_write -o a_write -- "
               "python3 bench.py --steps 8 --warmup 2 --no-cpu-baseline --no-qjl --no-tsq --no-grouped",
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/pmc_c_fetch -o c_fetch -- "
               "python3 bench.py --calibrate-copy",
               "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/pmc_c_write -o c_write -- "
               "python3 bench.py --calibrate-copy"],
           "calibration": {"copy_bytes": copy_bytes, "fetch_size_kib": cf, "write_size_kib": cw,
                           "fetch_factor": f_fetch, "write_factor": f_write},
           "kernels": {}}
    # the byte-code instantiations the roofline is quoted on (the same run also times the
    # packed-code kernels, whose traffic differs)
    for kname, key in (("pq_quantize_kernel<128, true, true, false, 1, 1024, true>", "pq_quantize_kernel"),
                       ("pq_dequantize_kernel<128, true, 0>", "pq_dequantize_kernel")):
        fk, nf = counter("pmc_q_fetch", "q_fetch", kname)
        wk, nw = counter("pmc_q_write", "q_write", kname)
        rec["kernels"][key] = {"instantiation": kname, "dispatches": [nf, nw], "fetch_size_kib": fk,
                               "write_size_kib": wk,
                               "hbm_bytes_per_launch": round(fk * 1024 * f_fetch + wk * 1024 * f_write)}
    # the fused decode-attention kernels of the config-5 attention leg (byte codes)
    for kname, key in (("pq_attend_kernel<256, 3, 4, false>", "pq_attend_kernel_d256"),
                       ("pq_attend_kernel<512, 3, 8, false>", "pq_attend_kernel_d512"),
                       ("pq_attend_kernel<128, 3, 2, false>", "pq_attend_kernel_d128"),
                       ("pq_attend_combine_kernel<512>", "pq_attend_combine_kernel_d512")):
        fk, nf = counter("pmc_a_fetch", "a_fetch", kname)
        wk, nw = counter("pmc_a_write", "a_write", kname)
        rec["kernels"][key] = {"instantiation": kname, "dispatches": [nf, nw], "fetch_size_kib": fk,
                               "write_size_kib": wk,
                               "hbm_bytes_per_launch": round(fk * 1024 * f_fetch + wk * 1024 * f_write)}
    with open(os.path.join(out_dir, "pq_quantize_config2_counters.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print("\n".join(lines))
    print(json.dumps(rec["kernels"]))
    if os.path.isdir(os.path.join(run_dir, "pmc_sq_a")):
        summarize_sq(run_dir)


# the kernels whose instruction mix and matrix-core use the benchmark reports, with the units
# (tiles of 16 blocks or keys) one launch processes in the benchmark's workload
SQ_KERNELS = (
    ("pq_quantize_kernel<128, true, true, false, 1, 1024, true>", "config-2 quantize + QJL (m=64)", 131072 // 16),
    ("pq_dequantize_kernel<128, true, 0>", "config-2 dequantize", 131072 // 16),
    ("pq_quantize_kernel<256, true, true, true, 1, 512, false>", "config-5 d=256 quantize + QJL (m=256)", 524288 // 16),
    ("pq_quantize_chunked_kernel<512, true, 1>", "config-5 d=512 quantize + QJL (m=512)", 524288 // 16),
    ("qjl_sketch_rows_kernel<128, false>", "config-4 QJL sketch (m=256)", 1048576 // 16),
    ("qjl_score_kernel<4, false>", "config-4 QJL score (4 query heads per KV head)", 1048576 // 16),
    ("pq_score_kernel<256, 3, 4, false>", "config-5 d=256 two-stage score (16 queries)", 524288 // 16),
    ("pq_score_kernel<512, 3, 8, false>", "config-5 d=512 two-stage score (16 queries)", 524288 // 16),
    ("pq_attend_kernel<256, 3, 4, false>", "config-5 d=256 decode attention", 524288 // 16),
    ("pq_attend_kernel<512, 3, 8, false>", "config-5 d=512 decode attention", 524288 // 16),
)
SQ_SET_A = "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_BUSY_CU_CYCLES SQ_WAVES GRBM_GUI_ACTIVE GRBM_COUNT"
SQ_SET_B = ("SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_LDS SQ_WAVE_CYCLES "
            "SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_I8 GRBM_GUI_ACTIVE")
SQ_BENCH_ARGS = "python3 bench.py --steps 8 --warmup 2 --no-cpu-baseline --no-grouped --no-bd --no-dense"


def summarize_sq(run_dir):
    """profiles/sq_counters_bench_kernels.{json,txt} from two rocprofv3 --pmc runs of the
    benchmark (run_dir/pmc_sq_a, run_dir/pmc_sq_b).  Derived figures follow rocprofv3's own
    metric definitions: MfmaUtil = sum SQ_VALU_MFMA_BUSY_CYCLES / (max-per-XCC GRBM_GUI_ACTIVE x
    1024 SIMDs), VALUBusy = sum SQ_ACTIVE_INST_VALU / 256 CUs / max-per-XCC GRBM_GUI_ACTIVE; the
    per-dispatch GRBM_GUI_ACTIVE rows are sums over the 8 XCCs, so max-per-XCC is taken as 1/8 of
    them (the XCCs run the kernel together)."""
    import csv
    out_dir = os.path.join(ROOT, "profiles")

    def load(sub, key):
        # per kernel, per dispatch, per counter; the benchmark also launches some of these kernels
        # at other sizes while setting up its legs (the attention leg quantizes its keys with the
        # config-2 instantiation), so only the dispatches whose `key` counter lies within 25% of
        # that kernel's median are kept: the timed workload's launches
        per = {}
        with open(os.path.join(run_dir, sub, "pmc_counter_collection.csv")) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"].replace("void ", "").replace("(anonymous namespace)::", "").split("(pqi::")[0]
                per.setdefault(name, {}).setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
        vals = {}
        for name, disp in per.items():
            ks = sorted(d[key] for d in disp.values() if key in d)
            med = ks[len(ks) // 2] if ks else 0.0
            for d in disp.values():
                if key in d and abs(d[key] - med) <= 0.25 * med:
                    for c, v in d.items():
                        vals.setdefault(name, {}).setdefault(c, []).append(v)
        return vals

    a, b = load("pmc_sq_a", "SQ_INSTS_VALU"), load("pmc_sq_b", "SQ_ACTIVE_INST_VALU")
    rec = {"source_hash": kernel_source_hash(),
           "commands": ["rocprofv3 --pmc %s --output-format csv -d <dir>/pmc_sq_a -o pmc -- %s" % (SQ_SET_A, SQ_BENCH_ARGS),
                        "rocprofv3 --pmc %s --output-format csv -d <dir>/pmc_sq_b -o pmc -- %s" % (SQ_SET_B, SQ_BENCH_ARGS)],
           "definitions": {"valu_insts_per_tile": "SQ_INSTS_VALU / tiles of 16 blocks (keys) per launch",
                           "mfma_insts_per_tile": "SQ_INSTS_MFMA / tiles per launch",
                           "mfma_util": "sum SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs)",
                           "valu_busy": "sum SQ_ACTIVE_INST_VALU / 256 CUs / (GRBM_GUI_ACTIVE / 8)",
                           "mfma_mops_per_launch": "(SQ_INSTS_VALU_MFMA_MOPS_F16 + _BF16 + _I8) x 512 flops (or int ops)",
                           "dispatches": "launches of the timed workload: those whose SQ_INSTS_VALU (SQ_ACTIVE_INST_VALU in the "
                                         "second run) lies within 25% of the kernel's median; set-up launches at other "
                                         "sizes are left out"},
           "kernels": {}}
    lines = ["# SQ counters of the benchmark's hot kernels, one MI355X (per launch, means over dispatches)", "",
             "commands:"] + ["  " + c for c in rec["commands"]] + ["kernel source hash: " + rec["source_hash"], "",
             "%-58s %8s %9s %8s %9s %9s %12s" % ("kernel", "tiles", "VALU/tile", "MFMA/tl", "MfmaUtil", "VALUBusy",
                                                "MFMA Mops")]
    mean = lambda d, k: sum(d[k]) / len(d[k]) if k in d and d[k] else float("nan")
    for kname, what, tiles in SQ_KERNELS:
        if kname not in a or kname not in b:
            continue
        ka, kb = a[kname], b[kname]
        grbm_a, grbm_b = mean(ka, "GRBM_GUI_ACTIVE") / 8.0, mean(kb, "GRBM_GUI_ACTIVE") / 8.0
        mops = sum(mean(kb, c) for c in ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                                         "SQ_INSTS_VALU_MFMA_MOPS_I8") if c in kb) * 512
        e = {"workload": what, "tiles_per_launch": tiles, "dispatches": len(ka.get("SQ_INSTS_VALU", [])),
             "raw": {k: mean(ka, k) for k in ka} | {k: mean(kb, k) for k in kb},
             "valu_insts_per_tile": mean(ka, "SQ_INSTS_VALU") / tiles,
             "mfma_insts_per_tile": mean(ka, "SQ_INSTS_MFMA") / tiles,
             "mfma_util": mean(kb, "SQ_VALU_MFMA_BUSY_CYCLES") / (grbm_b * 1024),
             "valu_busy": mean(kb, "SQ_ACTIVE_INST_VALU") / 256 / grbm_b,
             "mfma_ops_per_launch": mops}
        rec["kernels"][kname] = e
        lines.append("%-58s %8d %9.1f %8.1f %9.3f %9.3f %12.4g" % (
            kname, tiles, e["valu_insts_per_tile"], e["mfma_insts_per_tile"], e["mfma_util"], e["valu_busy"], mops))
    with open(os.path.join(out_dir, "sq_counters_bench_kernels.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    with open(os.path.join(out_dir, "sq_counters_bench_kernels.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def sq_counters():
    """Counter figures for the JSON line from the committed summary, or None when it is missing
    or was taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", "sq_counters_bench_kernels.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return {k: {f: round(v[f], 4) for f in ("valu_insts_per_tile", "mfma_insts_per_tile", "mfma_util", "valu_busy")}
            for k, v in rec["kernels"].items()}


_BIG = {}


def timed(torch, fn, steps):
    """Average duration (s) of fn(k), k = 0..steps-1, launched back to back on the current
    stream with HIP events recorded only before the first and after the last launch.  A
    large matmul queued first keeps the GPU busy while the launches are enqueued."""
    if "m" not in _BIG:
        _BIG["m"] = torch.randn(8192, 8192, device="cuda")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    _ = _BIG["m"] @ _BIG["m"]
    e0.record()
    for k in range(steps):
        fn(k)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / steps


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
    G = pq.projection_tensor(c["proj_seed"], m, d, dev)
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
    def sketch(k):
        pq.qjl_sketch(key_sets[k % 2], G, out=sketch_out[k % 2])

    def project(k):
        pq.qjl_project(q, G, out=sq)

    def score(k):
        pq.qjl_score(sq, *score_in[k % N_SETS], B, Hkv, Hq, T, out=scores[k % 2])

    t_sk = timed(torch, sketch, steps)
    t_pr = timed(torch, project, steps)
    t_sc = timed(torch, score, steps)
    sk_bytes = n_keys * d * 2 + n_keys * (m // 8) + n_keys * 2
    sc_bytes = n_keys * (m // 8) + n_keys * 2 + B * Hq * T * 4 + B * Hq * m * 4
    sk_flops = 2.0 * n_keys * d * m

    # outlier channels (group of 32 tokens, top 8, their own 256-row projection): channel
    # selection, the inlier and outlier sketches, and the two-term score
    gs, n_out, m_o = 32, 8, 256
    Go = pq.projection_tensor(synth.OUTLIER_PROJ_SEED, m_o, d, dev)
    kv = [k.view(B * Hkv, T, d) for k in key_sets]
    oidx = [pq.qjl_outlier_channels(kv[i], gs, n_out) for i in range(2)]
    sp_in = [(torch.empty_like(bits0), torch.empty_like(norms0)) for _ in range(2)]
    sp_out = [(torch.empty((n_keys, m_o // 8), dtype=torch.uint8, device=dev), torch.empty_like(norms0))
              for _ in range(2)]
    sqo = pq.qjl_project(q, Go)

    def outliers(k):
        pq.qjl_outlier_channels(kv[k % 2], gs, n_out, out=oidx[k % 2])

    def split_sketch(k):
        pq.qjl_sketch(kv[k % 2], G, out=sp_in[k % 2], split=(oidx[k % 2], T, gs, 0))
        pq.qjl_sketch(kv[k % 2], Go, out=sp_out[k % 2], split=(oidx[k % 2], T, gs, 1))

    def split_score(k):
        pq.qjl_score(sq, *sp_in[k % 2], B, Hkv, Hq, T, out=scores[k % 2])
        pq.qjl_score(sqo, *sp_out[k % 2], B, Hkv, Hq, T, out=scores[k % 2], accumulate=True)

    outliers(0), split_sketch(0), split_score(0)
    t_oc = timed(torch, outliers, steps)
    t_ss = timed(torch, split_sketch, steps)
    t_so = timed(torch, split_score, steps)
    return {
        "qjl_outlier_config": "config4 keys, outlier channels: groups of 32 tokens, top 8 channels, "
                              "256-row outlier projection; inlier and outlier sketch, two-term score",
        "qjl_outlier_channels_us": round(t_oc * 1e6, 3),
        "qjl_split_sketch_us": round(t_ss * 1e6, 3), "qjl_split_score_us": round(t_so * 1e6, 3),
        "qjl_split_score_keys_per_s": round(n_keys / t_so, 1),
        "qjl_config": "config4: keys 4x8x32768x128 bf16, m=256, 32 query heads (GQA 4:1)",
        "qjl_sketch_us": round(t_sk * 1e6, 3), "qjl_sketch_keys_per_s": round(n_keys / t_sk, 1),
        "qjl_sketch_hbm_frac": round(sk_bytes / t_sk / 1e9 / HBM_PEAK_GBS, 4),
        "qjl_sketch_mfma_frac": round(sk_flops / t_sk / 1e12 / BF16_PEAK_TFLOPS, 4),
        "qjl_project_us": round(t_pr * 1e6, 3),
        "qjl_score_us": round(t_sc * 1e6, 3), "qjl_score_keys_per_s": round(n_keys / t_sc, 1),
        "qjl_score_hbm_frac": round(sc_bytes / t_sc / 1e9 / HBM_PEAK_GBS, 4),
        "qjl_sketch_algorithmic_bytes": sk_bytes, "qjl_score_algorithmic_bytes": sc_bytes,
    }


def tsq_leg(pq, synth, torch, steps, warmup):
    """Config 5: per tensor ([8][65536][256] and [8][65536][512] bf16, 3-bit codes, QJL m=d),
    quantize, dequantize, query preparation (16 queries per KV head) and the two-stage
    score of every query against every vector."""
    dev = torch.device("cuda:0")
    out = {"tsq_config": "config5: bf16 KV vectors [8][65536][256] and [8][65536][512], log-normal channel "
                         "scales, 3-bit codes, QJL m=d, 16 queries per KV head"}
    for d in (256, 512):
        c = synth.config5_tensor(d)
        H, T, _ = c["x"].shape
        n_q, bits, m = c["q"].shape[1], c["bits"], c["m"]
        st = pq.signs_tensor(c["sign_seed"], d, dev)
        G = pq.projection_tensor(c["proj_seed"], m, d, dev)
        xs = [torch.from_numpy(c["x"].view(np.int16)).view(torch.bfloat16).to(dev) for _ in range(2)]
        q = torch.from_numpy(c["q"].view(np.int16)).view(torch.bfloat16).to(dev)
        del c
        enc = [pq.quantize(xs[i], d, bits, st, G) for i in range(2)]
        pk = [pq.quantize(xs[i], d, bits, st, G, packed=True) for i in range(2)]   # 3-bit codes bit-packed
        deq = [torch.empty((H * T, d), dtype=torch.bfloat16, device=dev) for _ in range(2)]
        prep = pq.query_prep(q, st, G)
        sc = torch.empty((H, n_q, T), dtype=torch.float32, device=dev)

        def quant(k):
            pq.quantize(xs[k % 2], d, bits, st, G, out=enc[k % 2])

        def dequant(k):
            pq.dequantize(enc[k % 2][0], enc[k % 2][1], d, bits, st, out=deq[k % 2])

        def score_packed(k):
            e = pk[k % 2]
            pq.score(prep, e[0], e[1], d, bits, H, n_q, T, e[2], e[3], m=m, out=sc, packed=True)

        def quant_packed(k):
            pq.quantize(xs[k % 2], d, bits, st, G, out=pk[k % 2], packed=True)

        def dequant_packed(k):
            pq.dequantize(pk[k % 2][0], pk[k % 2][1], d, bits, st, out=deq[k % 2], packed=True)

        def prepare(k):
            pq.query_prep(q, st, G, out=prep)

        def score(k):
            e = enc[k % 2]
            pq.score(prep, e[0], e[1], d, bits, H, n_q, T, e[2], e[3], m=m, out=sc)

        for k in range(warmup):
            quant(k), dequant(k), prepare(k), score(k)
        t = {name: timed(torch, fn, steps) for name, fn in
             (("quantize", quant), ("dequantize", dequant), ("query_prep", prepare), ("score", score),
              ("quantize_packed", quant_packed), ("dequantize_packed", dequant_packed),
              ("score_packed", score_packed))}
        nb = H * T
        qb = nb * d * 2 + nb * d + nb * 2 + nb * (m // 8) + nb * 2
        db = nb * d + nb * 2 + nb * d * 2
        pcb = nb * d * bits // 8                         # packed code bytes
        sb = nb * (d + 2 + m // 8 + 2) + H * n_q * T * 4
        out.update({
            "tsq_d%d_quantize_us" % d: round(t["quantize"] * 1e6, 2),
            "tsq_d%d_quantize_hbm_frac" % d: round(qb / t["quantize"] / 1e9 / HBM_PEAK_GBS, 4),
            "tsq_d%d_quantize_mfma_frac" % d: round(2.0 * 2 * nb * d * m / t["quantize"] / 1e12 / FP16_PEAK_TFLOPS, 4),
            "tsq_d%d_dequantize_us" % d: round(t["dequantize"] * 1e6, 2),
            "tsq_d%d_dequantize_hbm_frac" % d: round(db / t["dequantize"] / 1e9 / HBM_PEAK_GBS, 4),
            "tsq_d%d_query_prep_us" % d: round(t["query_prep"] * 1e6, 2),
            "tsq_d%d_score_us" % d: round(t["score"] * 1e6, 2),
            "tsq_d%d_score_vectors_per_s" % d: round(nb / t["score"], 1),
            "tsq_d%d_score_hbm_frac" % d: round(sb / t["score"] / 1e9 / HBM_PEAK_GBS, 4),
            "tsq_d%d_quantize_packed_us" % d: round(t["quantize_packed"] * 1e6, 2),
            "tsq_d%d_dequantize_packed_us" % d: round(t["dequantize_packed"] * 1e6, 2),
            "tsq_d%d_dequantize_packed_hbm_frac" % d: round((db - nb * d + pcb) / t["dequantize_packed"] / 1e9
                                                            / HBM_PEAK_GBS, 4),
            "tsq_d%d_score_packed_us" % d: round(t["score_packed"] * 1e6, 2),
            "tsq_d%d_score_packed_vectors_per_s" % d: round(nb / t["score_packed"], 1),
            "tsq_d%d_score_packed_hbm_frac" % d: round((sb - nb * d + pcb) / t["score_packed"] / 1e9 / HBM_PEAK_GBS, 4),
        })
        del xs, enc, pk, deq, prep, sc
        torch.cuda.empty_cache()
    return out


def attn_leg(pq, synth, torch, steps, warmup):
    """Decode attention on the config-5 shapes: per KV head 65536 quantized tokens (keys 3-bit with
    QJL m=d, values 3-bit without) plus a 128-token bf16 window, 16 queries per head, for d=256
    and d=512; and at the config-4 decode shape, d=128 with 32 heads of 32768 tokens and 4
    queries per head; byte codes and bit-packed codes.  Algorithmic bytes: every key and value
    code, norm and residual bit read once, the window and queries read once, the output written."""
    dev = torch.device("cuda:0")
    out = {"attn_config": "config5 shapes: 8 KV heads x 65536 quantized tokens + 128-token bf16 window, "
                          "16 queries per head, keys 3-bit + QJL m=d, values 3-bit, softmax scale 1/sqrt(d); "
                          "d128: the config-4 decode shape (batch 4 x 8 KV heads = 32 heads x 32768 tokens, "
                          "4 queries per KV head) on the same recipe"}
    t16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    for d, kv, toks, nq in ((256, 8, 65536, 16), (512, 8, 65536, 16), (128, 32, 32768, 4)):
        c = synth.config5_attention(d, kv_heads=kv, tokens=toks, n_q=nq)
        H, T, _ = c["k"].shape
        W, n_q, bits, m = c["k_win"].shape[1], c["q"].shape[1], c["bits"], c["m"]
        kst = pq.signs_tensor(c["k_sign_seed"], d, dev)
        vst = pq.signs_tensor(c["v_sign_seed"], d, dev)
        G = pq.projection_tensor(c["proj_seed"], m, d, dev)
        kx, vx = t16(c["k"]), t16(c["v"])
        kw, vw, q = t16(c["k_win"]), t16(c["v_win"]), t16(c["q"])
        del c
        keys = pq.quantize(kx, d, bits, kst, G)
        vals = pq.quantize(vx, d, bits, vst)[:2]
        kp = pq.quantize(kx, d, bits, kst, G, packed=True)[0]
        vp = pq.quantize(vx, d, bits, vst, packed=True)[0]
        del kx, vx
        prep = pq.query_prep(q, kst, G)
        work = torch.empty((pq.attention_work_bytes(d, H, T),), dtype=torch.uint8, device=dev)
        o = torch.empty((H, n_q, d), dtype=torch.float32, device=dev)

        def attend(k):
            pq.attention(prep, keys, vals, vst, d, bits, H, n_q, T, m=m, k_win=kw, v_win=vw, q=q, work=work, out=o)

        def attend_packed(k):
            pq.attention(prep, (kp,) + tuple(keys[1:]), (vp, vals[1]), vst, d, bits, H, n_q, T, m=m, k_win=kw,
                         v_win=vw, q=q, work=work, out=o, packed=True)

        for k in range(warmup):
            attend(k), attend_packed(k)
        ta, tp = timed(torch, attend, steps), timed(torch, attend_packed, steps)
        nb = H * T
        side = nb * (2 + m // 8 + 2 + 2) + 2 * H * W * d * 2 + H * n_q * d * 2 + H * n_q * d * 4
        ab = 2 * nb * d + side
        apb = 2 * nb * d * bits // 8 + side
        out.update({
            "attn_d%d_us" % d: round(ta * 1e6, 2),
            "attn_d%d_hbm_frac" % d: round(ab / ta / 1e9 / HBM_PEAK_GBS, 4),
            "attn_d%d_tokens_per_s" % d: round(nb / ta, 1),
            "attn_d%d_packed_us" % d: round(tp * 1e6, 2),
            "attn_d%d_packed_hbm_frac" % d: round(apb / tp / 1e9 / HBM_PEAK_GBS, 4),
            "attn_d%d_algorithmic_bytes" % d: ab,
            "attn_d%d_packed_algorithmic_bytes" % d: apb,
            "attn_d%d_work_bytes" % d: work.numel(),
            "attn_d%d_fused_kernel_hbm_bytes" % d: counter_traffic("pq_attend_kernel_d%d" % d),
        })
        del keys, vals, kp, vp, prep, work, o
        torch.cuda.empty_cache()
    return out


def bd_leg(pq, synth, torch, steps, warmup):
    """Block-diagonal rotation for a block size that is not a power of two: a 16384 x 2688 bf16
    weight (the config-2 recipe at the pages' 2688 width) in blocks of d = 2688 = 2048 + 512 +
    128, 4-bit codes; quantize and dequantize (bf16 out)."""
    dev = torch.device("cuda:0")
    d, bits, rows = 2688, 4, 16384
    xu, _ = synth.weight_with_outlier_entries(5, rows, d)
    x = torch.from_numpy(xu.view(np.int16)).view(torch.bfloat16).to(dev)
    del xu
    st = pq.signs_tensor(synth.BASE_SEED + d, d, dev)
    codes, norms = pq.quantize_bd(x, d, bits, st)
    out = torch.empty((rows, d), dtype=torch.bfloat16, device=dev)

    def quant(k):
        pq.quantize_bd(x, d, bits, st, out=(codes, norms))

    def dequant(k):
        pq.dequantize_bd(codes, norms, d, bits, st, out=out)

    for k in range(warmup):
        quant(k), dequant(k)
    tq, td = timed(torch, quant, steps), timed(torch, dequant, steps)
    n = rows * d
    qb = n * 2 + n + rows * 2
    db = n + rows * 2 + n * 2
    return {"bd_config": "16384 x 2688 bf16 weight (config-2 recipe), blocks of d=2688 = 2048+512+128, 4-bit",
            "bd_quantize_us": round(tq * 1e6, 2), "bd_quantize_hbm_frac": round(qb / tq / 1e9 / HBM_PEAK_GBS, 4),
            "bd_dequantize_us": round(td * 1e6, 2), "bd_dequantize_hbm_frac": round(db / td / 1e9 / HBM_PEAK_GBS, 4),
            "bd_quantize_algorithmic_bytes": qb, "bd_dequantize_algorithmic_bytes": db}


def dense_leg(pq, synth, torch, steps, warmup):
    """Dense random rotation with the sphere-coordinate codebook on a KV-cache tensor of the
    config-5 recipe at head size 128: [8][65536][128] bf16, 3-bit; the rotation is a Haar matrix
    (QR of a seeded Gaussian with the sign fix), an input of the codec."""
    dev = torch.device("cuda:0")
    d, bits = 128, 3
    c = synth.config5_tensor(d)
    x = torch.from_numpy(c["x"].view(np.int16)).view(torch.bfloat16).to(dev).reshape(-1, d)
    del c
    G = np.random.default_rng(synth.BASE_SEED + d).standard_normal((d, d))
    Q, R = np.linalg.qr(G)
    rot = torch.from_numpy((Q * np.sign(np.diag(R))[None, :]).astype(np.float32)).to(dev)
    n = x.shape[0]
    codes, norms = pq.quantize_dense(x, d, bits, rot)
    out = torch.empty((n, d), dtype=torch.bfloat16, device=dev)

    def quant(k):
        pq.quantize_dense(x, d, bits, rot, out=(codes, norms))

    def dequant(k):
        pq.dequantize_dense(codes, norms, d, bits, rot, out=out)

    for k in range(warmup):
        quant(k), dequant(k)
    tq, td = timed(torch, quant, steps), timed(torch, dequant, steps)
    qb = n * d * 2 + n * d + n * 2
    db = n * d + n * 2 + n * d * 2
    # matrix-core work as issued: quantize two bf16 products per K step (the hi and mid parts
    # of Pi), dequantize three fp16 products (hi hi, hi lo, lo hi); both against the 2.5 PFLOP/s
    # dense bf16 / fp16 peak
    flops = 2.0 * n * d * d
    return {"dense_config": "[8][65536][128] bf16 (config-5 recipe at d=128), 3-bit sphere-coordinate codebook, "
                            "Haar rotation",
            "dense_quantize_us": round(tq * 1e6, 2), "dense_quantize_hbm_frac": round(qb / tq / 1e9 / HBM_PEAK_GBS, 4),
            "dense_quantize_bf16_mfma_tflops": round(2 * flops / tq / 1e12, 2),
            "dense_quantize_bf16_mfma_frac": round(2 * flops / tq / 1e12 / BF16_PEAK_TFLOPS, 4),
            "dense_dequantize_us": round(td * 1e6, 2), "dense_dequantize_hbm_frac": round(db / td / 1e9 / HBM_PEAK_GBS, 4),
            "dense_dequantize_f16_mfma_tflops": round(3 * flops / td / 1e12, 2),
            "dense_dequantize_f16_mfma_frac": round(3 * flops / td / 1e12 / FP16_PEAK_TFLOPS, 4)}


def config3_weights(synth, torch, dev):
    """The 224 distinct bf16 tensors of config 3 (32 layers x q, k, v, o, gate, up, down; 14 GB),
    generated on the GPU from torch's seeded generator on the recipe of synth.config3_tensor:
    N(0, 0.02^2) and 8 seeded input columns per tensor scaled by 8 (7e9 values are too many to
    draw on the host within the benchmark's time)."""
    gen = torch.Generator(device=dev)
    xs = []
    for t, _, _, rows, cols in synth.config3_layout():
        gen.manual_seed(1000 + t)
        x = torch.randn((rows, cols), generator=gen, device=dev, dtype=torch.float32).mul_(0.02)
        cols_out = torch.randperm(cols, generator=gen, device=dev)[:8]
        x[:, cols_out] *= 8.0
        xs.append(x.to(torch.bfloat16))
        del x
    return xs


def grouped_leg(pq, synth, torch, reps, packed=False, xs=None):
    """Config 3: one streamed quantize pass and one dequantize pass over the 224 distinct tensors
    of a 32-layer 7B-style decoder (4-bit codes, d=128), each tensor with its own rotation signs
    (seed 42 + t), as ONE grouped launch per pass (pq_quantize_many / pq_dequantize_many over a
    device table of the 224 tensors).  ``packed``: codes bit-packed two to a byte."""
    dev = torch.device("cuda:0")
    layout = synth.config3_layout()
    d, bits = 128, 4
    cb = d * bits // 8 if packed else d                   # code bytes per block
    if xs is None:
        xs = config3_weights(synth, torch, dev)
    signs = [pq.signs_tensor(synth.BASE_SEED + t, d, dev) for t, _, _, _, _ in layout]
    enc = [(torch.empty((x.numel() // d, cb), dtype=torch.uint8, device=dev),
            torch.empty((x.numel() // d,), dtype=torch.float16, device=dev)) for x in xs]
    outs = [torch.empty((x.numel() // d, d), dtype=torch.bfloat16, device=dev) for x in xs]
    codes, norms = [c for c, _ in enc], [n for _, n in enc]
    total = sum(r * c for _, _, _, r, c in layout)
    assert total == sum(x.numel() for x in xs)

    def qpass(k):
        pq.quantize_many(xs, d, bits, signs, packed=packed, outs=enc)

    def dpass(k):
        pq.dequantize_many(codes, norms, d, bits, signs, packed=packed, outs=outs)

    qpass(0), dpass(0)
    tq, td = timed(torch, qpass, reps), timed(torch, dpass, reps)
    nb = total // d
    code_bytes = nb * cb
    q_bytes = total * 2 + code_bytes + nb * 2
    d_bytes = code_bytes + nb * 2 + total * 2
    del outs, enc
    key = "grouped_packed" if packed else "grouped"
    return {key + "_config": "config3: 224 distinct bf16 tensors (32 layers x q,k,v,o,gate,up,down), "
                             "6,979,321,856 values, d=128, 4-bit%s, one grouped launch per pass" % (
                                 ", codes packed two per byte" if packed else ""),
            key + "_quantize_ms": round(tq * 1e3, 3), key + "_quantize_hbm_frac": round(q_bytes / tq / 1e9 / HBM_PEAK_GBS, 4),
            key + "_dequantize_ms": round(td * 1e3, 3), key + "_dequantize_hbm_frac": round(d_bytes / td / 1e9 / HBM_PEAK_GBS, 4),
            key + "_input_gb_per_s": round(total * 2 / (tq + td) / 1e9, 1)}


def main():
    args = _args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1:
        print("bench.py: runs on one GPU only; --gpus %d is not supported "
              "(the codec would shard by blocks, with no exchange between GPUs)" % args.gpus, file=sys.stderr)
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
    signs = pq.signs_tensor(c["sign_seed"], d, dev)
    proj = pq.projection_tensor(c["proj_seed"], m, d, dev)

    sets = []
    for _ in range(N_SETS):
        x = x_host.to(dev)
        codes = torch.empty((n_blocks, d), dtype=torch.uint8, device=dev)
        norms = torch.empty((n_blocks,), dtype=torch.float16, device=dev)
        qb = torch.empty((n_blocks, m // 8), dtype=torch.uint8, device=dev)
        rn = torch.empty((n_blocks,), dtype=torch.float16, device=dev)
        out = torch.empty((n_blocks, d), dtype=torch.bfloat16, device=dev)
        pcodes = torch.empty((n_blocks, d * bits // 8), dtype=torch.uint8, device=dev)
        sets.append((x, codes, norms, qb, rn, out, pcodes))

    def quant(k):
        x, codes, norms, qb, rn, _, _ = sets[k % N_SETS]
        pq.quantize(x, d, bits, signs, proj, out=(codes, norms, qb, rn))

    def dequant(k):
        _, codes, norms, _, _, out, _ = sets[k % N_SETS]
        pq.dequantize(codes, norms, d, bits, signs, out=out)

    def quant_packed(k):
        x, _, norms, qb, rn, _, pcodes = sets[k % N_SETS]
        pq.quantize(x, d, bits, signs, proj, out=(pcodes, norms, qb, rn), packed=True)

    def dequant_packed(k):
        _, _, norms, _, _, out, pcodes = sets[k % N_SETS]
        pq.dequantize(pcodes, norms, d, bits, signs, out=out, packed=True)

    def step(k):
        quant(k)
        dequant(k)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t_q = timed(torch, quant, args.steps)
    t_d = timed(torch, dequant, args.steps)
    t_step = timed(torch, step, args.steps)
    quant_packed(0), dequant_packed(0)
    t_qp = timed(torch, quant_packed, args.steps)
    t_dp = timed(torch, dequant_packed, args.steps)

    # the ceiling of a dequantize-shaped stream on this GPU, measured in the same run: the
    # library's bandwidth probe reads 1 byte and writes 2 per value, the traffic of dequantize
    # without its arithmetic (over the same 8 rotating buffer sets)
    st_in = [bs[1].view(-1) for bs in sets]          # codes, uint8 [n d]
    st_out = [bs[5].view(torch.int16).view(-1) for bs in sets]   # output buffer, 2 bytes a value

    def stream(k):
        pq.probe_stream(st_in[k % N_SETS], out=st_out[k % N_SETS])

    stream(0)
    t_stream = timed(torch, stream, args.steps)

    in_bytes = n_blocks * d * 2
    q_bytes = in_bytes + n_blocks * d + n_blocks * 2 + n_blocks * (m // 8) + n_blocks * 2
    dq_bytes = n_blocks * d + n_blocks * 2 + in_bytes
    value = in_bytes / t_step / 1e9
    q_gbs = q_bytes / t_q / 1e9
    traffic = counter_traffic("pq_quantize_kernel")

    rec = {
        "metric": "quantize+dequantize GB/s and % HBM peak; QJL score keys/s at 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
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
            "quantize_packed_us": round(t_qp * 1e6, 3), "dequantize_packed_us": round(t_dp * 1e6, 3),
            "packed_input_gb_per_s": round(in_bytes / (t_qp + t_dp) / 1e9, 1),
            "stream_1B_in_2B_out_us": round(t_stream * 1e6, 3),
            "stream_1B_in_2B_out_hbm_frac": round(3 * n_blocks * d / t_stream / 1e9 / HBM_PEAK_GBS, 4),
        },
        "roofline": {"bound": "hbm", "achieved": round(q_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(q_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "pq_quantize_kernel<128, bf16, qjl>",
                     "algorithmic_bytes_per_launch": q_bytes},
        "kernel_source": kernel_source_hash(),
        "counters": sq_counters(),
    }
    def progress(what):
        print("[bench] %s done" % what, file=sys.stderr, flush=True)

    progress("config-2 codec")
    if not args.no_qjl:
        rec["parts"].update(qjl_leg(pq, synth, torch, args.steps, args.warmup))
        progress("config-4 QJL leg")
    if not args.no_tsq:
        rec["parts"].update(tsq_leg(pq, synth, torch, max(5, args.steps // 10), min(args.warmup, 3)))
        progress("config-5 two-stage leg")
    if not args.no_dense:
        rec["parts"].update(dense_leg(pq, synth, torch, max(5, args.steps // 10), min(args.warmup, 3)))
        progress("dense-rotation leg")
    if not args.no_bd:
        rec["parts"].update(bd_leg(pq, synth, torch, max(5, args.steps // 10), min(args.warmup, 3)))
        progress("block-diagonal leg")
    if not args.no_attn:
        rec["parts"].update(attn_leg(pq, synth, torch, max(5, args.steps // 10), min(args.warmup, 3)))
        progress("attention leg")
    if not args.no_grouped:
        w3 = config3_weights(synth, torch, dev)
        rec["parts"].update(grouped_leg(pq, synth, torch, max(3, args.steps // 50), xs=w3))
        rec["parts"].update(grouped_leg(pq, synth, torch, max(3, args.steps // 50), packed=True, xs=w3))
        del w3
        progress("config-3 grouped leg")
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(args.cpu_sample_blocks)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
