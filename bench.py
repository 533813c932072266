#!/usr/bin/env python3
"""Benchmark of the ternary projection path on one MI355X.

Headline (`value`): one decode token through every ternary projection of the
28-layer, 1536-hidden decoder -- 196 matrices (q, k, v, o, gate, up, down per
layer) at M = 1 -- as one grouped launch per step: per-row int8 quantization of
each projection's activations, the ternary x int8 contraction and the fp32
dequantization, all inside one kernel.  `value` is packed-weight GB/s.  The
weights (seeded fp32 masters ~N(0, 0.02)) are ternarized and packed on the GPU
once before timing, as the format ships pre-ternarized weights.  Two copies of
the 327.5 MB packed set alternate between steps so the reads come from HBM
rather than the 256 MB last-level cache.  Before the warm-up and the timed
steps the device is settled: a freshly started GPU runs its first seconds of
work much slower, so untimed batches run until two in a row agree (`settle`).
`step_stats` times the same launches one by one afterwards (median, minimum,
interquartile range).

`roofline` describes that decode kernel: algorithmic bytes per launch (packed
codes + fp32 activations + fp32 outputs + scales) over the launch duration
timed with HIP events on the launch stream.  `traffic` comes from the counter
summary in profiles/ when it was taken on the current kernel source.

`configs` reports the other workloads (single 1536x1536 GEMV, one decoder
layer, each projection shape alone and grouped over its 28 layers, the launch
floor, the sweep with all-zero codes against random ones, the dependent
per-token chain, the I8_S encoder layers, the lookup-table sweep, the sweep at
M = 4 and 16 (each projection with its own input, and with the inputs a decoder
shares: q, k, v one, gate and up another), prefill at M = 256 and 1800 over the
196 matrices and at M = 256
over one layer, prefill on each projection shape alone (its 28 matrices
grouped, and one matrix per call), batched decode at M = 32 and 64);
`cpu_baseline` times the CPU oracle on a bounded sample of the headline
workload on this host, its ternarize + pack step on its own, and (in
`other_rows`) its prefill and I8_S contractions on row samples.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0       # MI355X dense int8 MFMA
METRIC = "ternary matmul: decode weight GB/s (% HBM peak); prefill int8 TOPS (% MFMA peak)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_grouped_decode_sweep_m1_pmc.txt")
DECODE_SOURCES = ("gemv.hip", "bitnet_device.hpp", "bitnet_internal.hpp")


SWEEP_WEIGHTS = "0.02 N(0,1) fp32 masters, seed 10000+7l+p (the decode sweep's)"
OVERLAP_CHUNKS = (4, 7, 14, 28)
LONGFORM_WEIGHTS = "Student-t(3) fp32 masters scaled to std 0.01, seed 50000+7l+p"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--layers", type=int, default=28)
    ap.add_argument("--only",
                    choices=("all", "decode", "prefill", "chain", "lut", "i8", "lmhead", "copy",
                             "vendor"),
                    default="all",
                    help="decode: headline only; prefill: one prefill step size (--prefill-m) "
                         "only; chain: the dependent per-token chain only (graph of grouped "
                         "launches, and the staged call); lut: the lookup-table variant of "
                         "the M=1 sweep only; i8: the int8 x int8 encoder layers only; lmhead: the "
                         "8-bit embedding / lm_head table only; copy: 1 GiB copy probe used to calibrate the byte counters; "
                         "vendor: the vendor int8 GEMM (torch._int_mm) on the prefill shapes, "
                         "a reference point for the int8 MFMA rate these shapes allow")
    ap.add_argument("--prefill-m", type=int, default=256)
    ap.add_argument("--prefill-shapes", action="store_true",
                    help="with --only prefill: also each projection shape alone")
    ap.add_argument("--decode-m", type=int, default=1,
                    help="rows of the headline decode sweep (1 unless profiling other sizes)")
    ap.add_argument("--decode-subset", choices=("all", "gate_down"), default="all",
                    help="matrices of the decode sweep (gate_down: the 28 gate + 28 down)")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads")
    ap.add_argument("--settle-seconds", type=float, default=3.0,
                    help="minimum untimed settling before the headline warm-up (0: none, for "
                         "profiler runs that count every dispatch)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the timed CPU-oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gen-workers", type=int, default=0,
                    help="host processes drawing the workloads' arrays (0: one per CPU, at "
                         "most 16; 1: in this process, as profiler runs need)")
    ap.add_argument("--cache-dir", default="",
                    help="keep drawn arrays as .npy files here and reuse them (profiler runs "
                         "that repeat one workload)")
    return ap.parse_args()


def host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip() + f" ({os.cpu_count()} logical CPUs)"
    except OSError:
        pass
    return "unknown"


def decode_source_hash() -> str:
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "ternary_weight_decoder_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Timer:
    """HIP events on the launch stream around a block of launches."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def time(self, fn, steps, warmup=50):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for i in range(steps):
            fn(i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps   # ms per step

    def settle(self, fn, batch=100, agree=0.02, min_s=3.0, max_s=30.0):
        """Untimed work until the device reaches its steady state: batches of
        `batch` steps until two in a row agree within `agree` (after at least
        `min_s`, at most `max_s` seconds).  A freshly started GPU runs its
        first seconds of work much slower (the same decode sweep measured
        97.5 us per step in the first process on a box and 55.5 us in the
        next).  Returns the seconds spent and the last two batch times."""
        t0 = time.perf_counter()
        prev = first = None
        while True:
            ms = self.time(fn, batch, warmup=0)
            first = ms if first is None else first
            el = time.perf_counter() - t0
            if prev is not None and abs(ms - prev) <= agree * prev and el >= min_s:
                break
            if el >= max_s:
                break
            prev = ms
        return {"seconds": round(el, 2), "first_batch_us_per_step": round(first * 1e3, 2),
                "last_batches_us_per_step":
                [round(prev * 1e3, 2) if prev else None, round(ms * 1e3, 2)]}

    def graph_time(self, fn, calls, replays=20):
        """Device time per call: `calls` calls captured once in a HIP graph and
        the graph replayed back to back, so the host's launch rate (Python,
        ctypes, one enqueue per kernel) drops out of the figure.  Returns ms
        per call."""
        torch = self.torch
        fn(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(calls):
                    fn(i)
        torch.cuda.current_stream().wait_stream(cap)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(replays):
            g.replay()
        e1.record(self.stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (replays * calls)
        g.reset()
        cap.synchronize()
        del g
        return ms

    def per_step(self, fn, steps, warmup=3):
        """Device time of each step on its own (an event pair around every
        launch): median, minimum and interquartile range in microseconds."""
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(self.stream)
        for i in range(steps):
            fn(i)
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        us = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps)])
        q1, med, q3 = np.percentile(us, [25, 50, 75])
        return {"steps": steps, "median_us": round(float(med), 2), "min_us": round(float(us.min()), 2),
                "p25_us": round(float(q1), 2), "p75_us": round(float(q3), 2)}


def copy_probe(torch):
    """A plain 1 GiB elementwise copy (negation), five times: the byte-counter
    reference (1 GiB read and 1 GiB written per launch)."""
    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": 4 * n, "launches": 5}), flush=True)


def vendor_reference(torch):
    """torch._int_mm (the vendor int8 GEMM library) on the prefill projection
    shapes: int8 x int8 -> int32, no quantization, no dequantization."""
    dev = "cuda:0"
    out = []
    for M, N, K in ((256, 8960, 1536), (256, 1536, 8960), (1800, 8960, 1536), (1800, 1536, 8960),
                    (8192, 8192, 8192)):
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev)
        b = torch.randint(0, 3, (N, K), dtype=torch.int8, device=dev).t()   # column-major [K, N]
        for _ in range(3):
            torch._int_mm(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            torch._int_mm(a, b)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / 20 * 1e3
        out.append({"M": M, "N": N, "K": K, "us": round(us, 1),
                    "int8_TOPS": round(2.0 * M * N * K / us / 1e6, 1)})
    print(json.dumps({"vendor_int8_gemm": out}), flush=True)


def main():
    args = parse()
    GEN["workers"], GEN["cache"] = args.gen_workers, args.cache_dir
    if args.gpus != 1:
        print(f"bench.py: this implementation runs on one GPU; --gpus {args.gpus} is not "
              "supported (multi-GPU operation would replicate the packed weights per GPU "
              "and give each GPU its own requests or token shard)", file=sys.stderr)
        sys.exit(2)

    import torch
    from ternary_weight_decoder_amd import binding as tb, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.only == "copy":
        copy_probe(torch)
        return
    if args.only == "vendor":
        vendor_reference(torch)
        return
    dev = torch.device("cuda:0")
    tb.lib()
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream)
    if args.only == "i8":
        log("[bench] I8_S encoder layers only")
        res = i8_configs(torch, tb, synth, timer, dev, steps=args.steps)
        res["i8_dwconv_encoder"] = dwconv_config(torch, tb, synth, timer, dev, steps=args.steps)
        print(json.dumps(res), flush=True)
        return
    if args.only == "lmhead":
        log("[bench] embedding / lm_head table only")
        print(json.dumps(lmhead_configs(torch, tb, synth, timer, dev, steps=args.steps)),
              flush=True)
        return

    problems = synth.sweep_problems(args.layers)
    n_mat = len(problems)
    log(f"[bench] generating and ternarizing {n_mat} matrices on the GPU")

    # ---- offline: ternarize + pack every matrix on the GPU -------------------
    packed, w_scales = [], []
    ws_t = torch.empty(tb.bitnet_ternarize_workspace_bytes(synth.INTERMEDIATE), dtype=torch.uint8,
                       device=dev)
    tern_ms, w_bytes = 0.0, 0
    for p in problems:
        W = torch.from_numpy(synth.problem_weights(p)).to(dev)
        pk = torch.empty(p.N * p.K // 4, dtype=torch.uint8, device=dev)
        sc = torch.empty(1, dtype=torch.float32, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        tb.bitnet_ternarize_pack_into(W, p.N, p.K, pk, sc, ws_t)
        e1.record(stream)
        e1.synchronize()
        tern_ms += e0.elapsed_time(e1)
        w_bytes += W.numel() * 4
        packed.append(pk)
        w_scales.append(sc)
        del W
    packed_bytes = sum(p.N * p.K // 4 for p in problems)
    copy_b = [t.clone() for t in packed]
    Ns = [p.N for p in problems]
    Ks = [p.K for p in problems]

    def alg_bytes(M, probs):
        return (sum(p.N * p.K // 4 for p in probs) + sum(M * p.K * 4 for p in probs) +
                sum(M * p.N * 4 for p in probs) + 4 * len(probs))

    def decode_plans(M, probs=problems, xs_host=None, copies=(packed, copy_b)):
        idx = [problems.index(p) for p in probs] if probs is not problems else range(n_mat)
        if xs_host is None:
            xs = [torch.from_numpy(synth.problem_activations(p, M)).to(dev) for p in probs]
        else:
            xs = [torch.from_numpy(x).to(dev) for x in xs_host]
        ys = [torch.empty((M, p.N), dtype=torch.float32, device=dev) for p in probs]
        plans = [tb.GroupedPlan(M, xs, [c[i] for i in idx], [w_scales[i] for i in idx], ys,
                                [p.N for p in probs], [p.K for p in probs]) for c in copies]
        return plans, xs, ys

    if args.only == "chain":
        log("[bench] dependent per-token chain only")
        res = chain_configs(torch, tb, synth, timer, problems, packed, w_scales, alg_bytes,
                            decode_plans, dev)
        print(json.dumps(res), flush=True)
        return

    if args.only == "lut":
        log("[bench] lookup-table decode sweep only")
        res = lut_config(torch, tb, synth, timer, problems, packed, copy_b, w_scales, alg_bytes,
                         decode_plans, dev, steps=args.steps)
        print(json.dumps(res), flush=True)
        return

    if args.only == "prefill":
        M = args.prefill_m
        log(f"[bench] prefill M={M} only")
        if M == synth.PREFILL_M_LONG:
            lf = synth.longform_problems(args.layers)
            lf_packed, lf_scales = pack_set(torch, tb, synth, lf, True, dev)
            res = prefill_config(torch, tb, synth, timer, lf, lf_packed, lf_scales, M, dev,
                                 LONGFORM_WEIGHTS)
        else:
            res = prefill_config(torch, tb, synth, timer, synth.prefill_problems(args.layers),
                                 packed, w_scales, M, dev, SWEEP_WEIGHTS)
        if args.prefill_shapes:
            res["per_shape"] = prefill_shapes_config(torch, tb, timer, problems, packed,
                                                      w_scales, M, dev)
        print(json.dumps({"workload": f"prefill M={M} over {n_mat} matrices", **res}), flush=True)
        return

    # ---- headline: decode sweep, M = 1 ------------------------------------------
    M = args.decode_m
    if args.decode_subset == "gate_down":
        sweep = [p for p in problems if p.proj in (4, 6)]
    else:
        sweep = problems
    xs_host = [synth.problem_activations(p, M) for p in sweep]
    plans, xs, ys = decode_plans(M, probs=sweep, xs_host=xs_host)
    packed_bytes = sum(p.N * p.K // 4 for p in sweep)
    steps = args.steps
    log(f"[bench] decode sweep M={M} over {len(sweep)} matrices: settling the device, then "
        f"warmup {args.warmup}, timed {steps} steps")
    settle = (timer.settle(lambda i=0: plans[i % 2].run(), min_s=args.settle_seconds)
              if args.settle_seconds > 0 else None)
    if settle:
        log(f"[bench] settled after {settle['seconds']} s "
            f"(first batch {settle['first_batch_us_per_step']}, last batches "
            f"{settle['last_batches_us_per_step']} us/step)")
    ms_step = timer.time(lambda i=0: plans[i % 2].run(), steps, warmup=args.warmup)
    weight_gbps = packed_bytes / (ms_step * 1e-3) / 1e9
    bytes_launch = alg_bytes(M, sweep)
    achieved = bytes_launch / (ms_step * 1e-3) / 1e9
    log(f"[bench] decode {ms_step * 1e3:.1f} us/step, weight {weight_gbps:.0f} GB/s, "
        f"all bytes {achieved:.0f} GB/s")
    # The same launches timed one by one (outside the timed block above).
    step_stats = timer.per_step(lambda i=0: plans[i % 2].run(), 200)

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            recs = [json.loads(s) for s in f if s.startswith("{")]
        if recs and recs[-1].get("source_hash") == decode_source_hash():
            traffic = recs[-1].get("bytes_per_launch")

    configs = {}
    if args.only == "all" and not args.no_configs:
        configs = other_configs(torch, tb, synth, timer, problems, packed, copy_b, w_scales,
                                alg_bytes, decode_plans, dev)

    # ---- CPU oracle on a bounded sample of the headline workload -------------
    cpu = None
    if args.only == "all" and not args.no_cpu_baseline:
        import oracle
        cores = oracle.num_threads()
        t_spent, bytes_done, mats, max_rel, packed_equal = 0.0, 0, 0, 0.0, 0
        t_tern, tern_bytes = 0.0, 0
        plans[0].run()
        torch.cuda.synchronize()
        refs = []
        for i, p in enumerate(sweep):
            W = synth.problem_weights(p)
            t0 = time.perf_counter()
            pk_ref, s_ref = oracle.ternarize_pack(W)      # offline step, timed on its own
            t_tern += time.perf_counter() - t0
            tern_bytes += W.nbytes
            refs.append((pk_ref, s_ref))
            t0 = time.perf_counter()
            ref = oracle.ternary_matmul(xs_host[i], pk_ref, s_ref, p.N)
            t_spent += time.perf_counter() - t0
            bytes_done += p.N * p.K // 4
            mats += 1
            packed_equal += int(np.array_equal(packed[problems.index(p)].cpu().numpy(), pk_ref))
            y_gpu = ys[i].cpu().numpy()
            rel = np.abs(y_gpu - ref["y"]) / np.maximum(np.abs(ref["y"]), 1e-30)
            max_rel = max(max_rel, float(rel.max()))
            if t_spent >= args.cpu_seconds:
                break
        # The same oracle on one thread, over the first layer's 7 projections.
        oracle.set_num_threads(1)
        t1, b1 = 0.0, 0
        for i, p in enumerate(sweep[:min(7, mats)]):
            t0 = time.perf_counter()
            oracle.ternary_matmul(xs_host[i], refs[i][0], refs[i][1], p.N)
            t1 += time.perf_counter() - t0
            b1 += p.N * p.K // 4
        oracle.set_num_threads(cores)
        # The oracle on the other contraction rows, each on a bounded row sample.
        other = {}
        t_pf, ops_pf = 0.0, 0.0
        for i, p in enumerate(sweep[:min(7, mats)]):
            xp = synth.activations(32, p.K, seed=33000 + i)
            t0 = time.perf_counter()
            oracle.ternary_matmul(xp, refs[i][0], refs[i][1], p.N)
            t_pf += time.perf_counter() - t0
            ops_pf += 2.0 * 32 * p.N * p.K
        if t_pf > 0:
            other["prefill"] = {"value": round(ops_pf / t_pf / 1e12, 5), "unit": "int8 TOPS",
                                "sample": "layer 0's 7 projections, 32 rows each"}
        t_i8, ops_i8 = 0.0, 0.0
        for name in sorted(synth.I8_LAYERS):
            _, K8, N8, relu8 = synth.I8_LAYERS[name]
            x8, W8, b8 = synth.i8_layer_inputs(name)
            q8, s8 = oracle.i8_quant_weights(W8)
            t0 = time.perf_counter()
            oracle.i8_linear(x8[:1024], q8, s8, b8, relu8)
            t_i8 += time.perf_counter() - t0
            ops_i8 += 2.0 * 1024 * N8 * K8
        other["i8_linear"] = {"value": round(ops_i8 / t_i8 / 1e12, 5), "unit": "int8 TOPS",
                              "sample": "first 1024 rows of each I8_S encoder layer"}
        cpu = {"value": round(bytes_done / t_spent / 1e9, 4), "unit": "GB/s", "cores": cores,
               "kind": "oracle",
               "sample": f"first {mats} of {len(sweep)} decode projections (layers in order, "
                         f"M={M}): "
                         f"per-row quantize, unpack, int32 add/sub contraction, dequantize; "
                         f"{t_spent:.1f} s of oracle time on {cores} threads; GPU-packed codes "
                         f"equal to the oracle's in {packed_equal}/{mats} matrices; GPU outputs "
                         f"agree to max relative error {max_rel:.2e}",
               "ternarize_pack": {"value": round(tern_bytes / t_tern / 1e9, 4),
                                  "unit": "GB/s of fp32 masters", "matrices": mats,
                                  "seconds": round(t_tern, 2),
                                  "note": "offline step, outside the decode figure"},
               "single_thread": {"value": round(b1 / t1 / 1e9, 4), "unit": "GB/s",
                                 "sample": "layer 0's 7 projections, M=1, 1 thread"},
               "other_rows": other,
               "host_cpu": host_cpu()}
        log(f"[bench] cpu oracle {cpu['value']} GB/s on {cores} threads ({mats} matrices)")

    line = {
        "metric": METRIC,
        "value": round(weight_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "step_stats": step_stats,
        "settle": settle,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"decode sweep: all {len(sweep)} ternary projections of a "
                               f"{args.layers}-layer decoder (q,k,v,o 1536->1536/256; gate,up "
                               f"1536->8960; down 8960->1536), M={M}, one grouped launch per step",
                   "M": M, "matrices": len(sweep), "packed_weight_bytes": packed_bytes,
                   "weight_copies_rotated": 2},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": bytes_launch,
                     "kernel": "gemv_grouped_kernel<fused quantization>"},
        "cpu_baseline": cpu,
        "ternarize_pack": {"workload": f"{n_mat} matrices, fp32 masters read once",
                           "ms_total": round(tern_ms, 3),
                           "fp32_read_GBps": round(w_bytes / (tern_ms * 1e-3) / 1e9, 1)},
        "configs": configs,
    }
    print(json.dumps(line), flush=True)


GEN = {"workers": 0, "cache": ""}


def gen_workers() -> int:
    """Host processes for drawing the workloads' arrays (the machine's CPU share)."""
    if GEN["workers"] > 0:
        return GEN["workers"]
    return max(1, min(16, os.cpu_count() or 1))


def cached(kind, items, draw):
    """draw(items) -> iterator of arrays, one per item, unless --cache-dir holds
    them (file per item, named by kind and the item's key)."""
    d = GEN["cache"]
    if not d:
        yield from draw(items)
        return
    os.makedirs(d, exist_ok=True)
    paths = [os.path.join(d, f"{kind}_{k}.npy") for k, _ in items]
    if all(os.path.exists(p) for p in paths):
        for p in paths:
            yield np.load(p)
        return
    for p, a in zip(paths, draw(items)):
        np.save(p, a)
        yield a


def pack_set(torch, tb, synth, problems, heavy_tail, dev):
    """Draw the problems' fp32 masters on the host (worker processes), ternarize
    and pack each on the GPU; returns (packed, w_scales)."""
    packed, w_scales = [], []
    ws_t = torch.empty(tb.bitnet_ternarize_workspace_bytes(synth.INTERMEDIATE),
                       dtype=torch.uint8, device=dev)
    items = [(f"{p.w_seed}_{p.N}x{p.K}_{int(heavy_tail)}", p) for p in problems]
    draw = lambda it: synth.problem_weights_iter([p for _, p in it], heavy_tail, gen_workers())
    for i, (p, W) in enumerate(zip(problems, cached("w", items, draw))):
        if i % 28 == 0:
            log(f"[bench] packing matrix {i} of {len(problems)}")
        Wd = torch.from_numpy(W).to(dev)
        pk = torch.empty(p.N * p.K // 4, dtype=torch.uint8, device=dev)
        sc = torch.empty(1, dtype=torch.float32, device=dev)
        tb.bitnet_ternarize_pack_into(Wd, p.N, p.K, pk, sc, ws_t)
        packed.append(pk)
        w_scales.append(sc)
        del Wd
    torch.cuda.synchronize()
    return packed, w_scales


def zero_code_fraction(torch, packed) -> float:
    """Share of codes equal to 0 (2-bit field value 1) over packed buffers."""
    zeros = total = 0
    for t in packed:
        v = t.to(torch.int32)
        for sh in (0, 2, 4, 6):
            zeros += int(((v >> sh) & 3).eq(1).sum().item())
        total += 4 * t.numel()
    return zeros / total


def host_activations(torch, synth, problems, M, dev):
    """problem_activations(p, M) for each problem (drawn on the host in worker
    processes: N(0,1), round(0.01 K) channels x20), copied to the device."""
    log(f"[bench] drawing activations for {len(problems)} problems, M={M}")
    items = [(f"{p.x_seed}_{M}x{p.K}", p) for p in problems]
    draw = lambda it: synth.problem_activations_iter([p for _, p in it], M, gen_workers())
    return [torch.from_numpy(x).to(dev) for x in cached("x", items, draw)]


def gpu_activations(torch, g, M, K, dev):
    """~N(0,1) rows with 1% of the channels scaled by 20, drawn on the GPU."""
    x = torch.randn((M, K), generator=g, device=dev)
    cols = torch.randperm(K, generator=g, device=dev)[:max(1, K // 100)]
    x[:, cols] *= 20.0
    return x


def prefill_config(torch, tb, synth, timer, problems, packed, w_scales, M, dev, weights,
                   zero_codes_check=False):
    """Prefill at M rows over all the problems in one grouped call per step
    (quantization launch + GEMM launch); activations drawn per problem from its
    own seed.  zero_codes_check: also time the same step with every code 0."""
    xs = host_activations(torch, synth, problems, M, dev)
    ys = [torch.empty((M, p.N), device=dev) for p in problems]
    plan = tb.GroupedPlan(M, xs, packed, w_scales, ys, [p.N for p in problems],
                          [p.K for p in problems])
    steps = 30 if M > 1000 else 100
    ms = timer.time(lambda i=0: plan.run(), steps, warmup=10 if M > 1000 else 20)
    ops = 2.0 * M * sum(p.N * p.K for p in problems)
    res = {"ms_per_step": round(ms, 4), "int8_TOPS": round(ops / (ms * 1e-3) / 1e12, 1),
           "frac_of_int8_peak": round(ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
           "step": "quantization launch + int8 MFMA GEMM launch over all matrices",
           "weights": weights,
           "activations": f"host numpy, seed {problems[0].x_seed - 7 * problems[0].layer - problems[0].proj}"
                          "+7l+p: N(0,1), round(0.01 K) channels x20"}
    # The same step with the inputs a decoder shares: a layer's q, k and v read
    # one buffer and its gate and up another, so the grouped call quantizes
    # each such input once (112 inputs instead of 196).
    first = {}
    xs_sh = []
    for p, x in zip(problems, xs):
        xs_sh.append(first.setdefault((p.layer, (0, 0, 0, 1, 2, 2, 3)[p.proj]), x))
    plan_sh = tb.GroupedPlan(M, xs_sh, packed, w_scales, ys, [p.N for p in problems],
                             [p.K for p in problems])
    ms_s = timer.time(lambda i=0: plan_sh.run(), steps, warmup=10 if M > 1000 else 20)
    res["shared_inputs"] = {"ms_per_step": round(ms_s, 4), "distinct_inputs": len(first),
                            "int8_TOPS": round(ops / (ms_s * 1e-3) / 1e12, 1),
                            "frac_of_int8_peak": round(ops / (ms_s * 1e-3) / 1e12 /
                                                       INT8_PEAK_TOPS, 4)}
    del plan_sh, xs_sh, first
    # The same step with the quantization of later chunks of problems on a
    # second stream, overlapping the contraction of earlier ones.
    aux = torch.cuda.Stream()
    overlap = {}
    for nch in OVERLAP_CHUNKS:
        ms_o = timer.time(lambda i=0: plan.run_overlap(aux, nch), steps, warmup=5)
        overlap[str(nch)] = round(ms_o, 4)
    best = min(overlap, key=overlap.get)
    ms_b = overlap[best]
    res["overlapped"] = {"ms_per_step_by_chunks": overlap, "best_chunks": int(best),
                         "ms_per_step": ms_b,
                         "int8_TOPS": round(ops / (ms_b * 1e-3) / 1e12, 1),
                         "frac_of_int8_peak": round(ops / (ms_b * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                         "step": "bitnet_ternary_matmul_grouped_overlap: quantization launches "
                                 "on a second stream, GEMM launches on the timed stream"}
    aux.synchronize()
    if zero_codes_check:
        zc = [torch.full_like(t, 0x55) for t in packed]
        zplan = tb.GroupedPlan(M, xs, zc, w_scales, ys, [p.N for p in problems],
                               [p.K for p in problems])
        ms_z = timer.time(lambda i=0: zplan.run(), steps, warmup=5)
        ms_r = timer.time(lambda i=0: plan.run(), steps, warmup=5)
        res["code_independence"] = {"ms_per_step_all_zero_codes": round(ms_z, 4),
                                    "ms_per_step_these_codes": round(ms_r, 4)}
        del zc, zplan
    del xs, ys, plan
    torch.cuda.empty_cache()
    return res


def prefill_layer_config(torch, tb, synth, timer, problems, packed, w_scales, M, dev):
    """One layer's 7 projections at prefill in one grouped call (quantization +
    GEMM); step i runs layer i % 28, so every step reads its codes from HBM."""
    layer = problems[:7]
    xs = host_activations(torch, synth, layer, M, dev)
    ys = [torch.empty((M, p.N), device=dev) for p in layer]
    layers = len(problems) // 7
    plans = [tb.GroupedPlan(M, xs, packed[7 * l:7 * l + 7], w_scales[7 * l:7 * l + 7], ys,
                            [p.N for p in layer], [p.K for p in layer]) for l in range(layers)]
    ms = timer.time(lambda i=0: plans[i % layers].run(), 280, warmup=56)
    ops = 2.0 * M * sum(p.N * p.K for p in layer)
    return {"us_per_layer": round(ms * 1e3, 2), "int8_TOPS": round(ops / (ms * 1e-3) / 1e12, 1),
            "frac_of_int8_peak": round(ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
            "step": "one grouped call (quantization + GEMM launch) over q,k,v,o,gate,up,down "
                    "of one layer, layers rotated"}


def prefill_shapes_config(torch, tb, timer, problems, packed, w_scales, M, dev):
    """Each projection shape alone: its 28 matrices (one per layer) in one
    grouped call per step (quantization + GEMM launch), and one matrix per call
    through bitnet_ternary_matmul_q8 from pre-quantized rows (a row-sum pass and
    the GEMM launch; K-split launches add a zero fill and a finishing pass), the
    28 layers' matrices in turn."""
    g = torch.Generator(device=dev)
    g.manual_seed(32000 + M)
    out = {}
    for proj, name in ((0, "q_o_1536x1536"), (1, "k_v_256x1536"), (4, "gate_up_8960x1536"),
                       (6, "down_1536x8960")):
        idx = [i for i, p in enumerate(problems) if p.proj == proj]
        n = len(idx)
        N, K = problems[idx[0]].N, problems[idx[0]].K
        ops = 2.0 * M * N * K
        xs = [gpu_activations(torch, g, M, K, dev) for _ in idx]
        ys = [torch.empty((M, N), device=dev) for _ in idx]
        plan = tb.GroupedPlan(M, xs, [packed[i] for i in idx], [w_scales[i] for i in idx], ys,
                              [N] * n, [K] * n)
        ms_g = timer.time(lambda i=0: plan.run(), 30 if M > 1000 else 100, warmup=10)
        xq, xsc = tb.bitnet_quant_act(xs[0])
        ws = torch.empty(tb.bitnet_matmul_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
        ms_1 = timer.time(lambda i=0: tb.bitnet_ternary_matmul_q8_into(
            M, N, K, xq, xsc, packed[idx[i % n]], w_scales[idx[i % n]], ys[0], ws), 5 * n,
            warmup=2 * n)
        out[name] = {"grouped_28_us": round(ms_g * 1e3, 2),
                     "grouped_28_int8_TOPS": round(n * ops / (ms_g * 1e-3) / 1e12, 1),
                     "grouped_28_frac_of_int8_peak": round(
                         n * ops / (ms_g * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                     "single_call_q8_us": round(ms_1 * 1e3, 2),
                     "single_call_q8_frac_of_int8_peak": round(
                         ops / (ms_1 * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)}
        del xs, ys, plan, xq, xsc, ws
        torch.cuda.empty_cache()
    return out


def chain_configs(torch, tb, synth, timer, problems, packed, w_scales, alg_bytes, decode_plans,
                  dev):
    """One decode token with the layer dependencies kept, two ways."""
    out = {}
    layers = len(problems) // 7
    # One token through the decoder with the data dependencies of a layer kept:
    # per layer four grouped launches in order (q,k,v | o | gate,up | down), 112
    # launches per token, captured once in a HIP graph and replayed.  Graph
    # replays are checked bit-exact against the eager launches first.
    chain, chain_ys = [], []
    for l in range(layers):
        for grp in ((0, 1, 2), (3,), (4, 5), (6,)):
            probs = [problems[7 * l + j] for j in grp]
            plans, _, ys_c = decode_plans(1, probs, copies=(packed,))
            chain.append(plans[0])
            chain_ys.extend(ys_c)

    def run_chain(i=0):
        for pl in chain:
            pl.run()
    run_chain()
    torch.cuda.synchronize()
    eager = [y.clone() for y in chain_ys]
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            run_chain()
    torch.cuda.current_stream().wait_stream(cap)
    replay_ok = True
    for _ in range(3):
        for y in chain_ys:
            y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        replay_ok &= all(torch.equal(a, b) for a, b in zip(chain_ys, eager))
    ms = timer.time(lambda i=0: graph.replay(), 100)
    ms_eager = timer.time(run_chain, 20)
    out["decode_token_chain_m1"] = {
        "us_per_token": round(ms * 1e3, 2), "launches": len(chain),
        "weight_GBps": round(sum(p.N * p.K // 4 for p in problems) / (ms * 1e-3) / 1e9, 1),
        "us_per_token_eager_launches": round(ms_eager * 1e3, 2),
        "graph_replays_match_eager": bool(replay_ok),
        "note": "28 layers x 4 dependent grouped launches (qkv, o, gate+up, down), HIP graph"}
    # Tear the graph down here, while the process is fully alive: free its
    # executable and its private memory pool, and drain the capture stream.
    graph.reset()
    cap.synchronize()
    torch.cuda.synchronize()
    del chain, chain_ys, eager, graph, cap
    torch.cuda.empty_cache()

    # The same token as one staged call: 112 stages in one cooperative launch,
    # each stage reading what the one before it wrote (q,k,v read h; o reads
    # y_q; gate and up read y_o; down reads y_up; the next layer's h is
    # y_down).  Checked bit-exact against the same flow run as 112 grouped
    # launches over the same buffers.
    h = torch.from_numpy(synth.activations(1, synth.HIDDEN, seed=4242)).to(dev)
    stages, flow_ys = [], []
    for l in range(layers):
        P = problems[7 * l:7 * l + 7]
        yl = [torch.empty((1, p.N), dtype=torch.float32, device=dev) for p in P]

        def pr(j, x, l=l, P=P, yl=yl):
            return (x, packed[7 * l + j], w_scales[7 * l + j], yl[j], P[j].N, P[j].K)
        stages += [[pr(0, h), pr(1, h), pr(2, h)], [pr(3, yl[0])], [pr(4, yl[3]), pr(5, yl[3])],
                   [pr(6, yl[5])]]
        flow_ys += yl
        h = yl[6]
    staged = tb.StagedPlan(1, stages)
    launches = [tb.GroupedPlan(1, [t[0] for t in st], [t[1] for t in st], [t[2] for t in st],
                               [t[3] for t in st], [t[4] for t in st], [t[5] for t in st])
                for st in stages]
    for pl in launches:
        pl.run()
    torch.cuda.synchronize()
    ref = [y.clone() for y in flow_ys]
    for y in flow_ys:
        y.fill_(float("nan"))
    staged.run()
    torch.cuda.synchronize()
    staged_ok = all(torch.equal(a, b) for a, b in zip(flow_ys, ref)) and not staged.timed_out()
    ms = timer.time(lambda i=0: staged.run(), 100)
    timed_out = staged.timed_out()
    # every call of this plan so far (checks, warm-up, timed): calls in which
    # some wait between stages ran out
    timeouts_total = staged.timeouts_total()
    out["decode_token_staged_m1"] = {
        "us_per_token": round(ms * 1e3, 2), "launches": 1, "stages": len(stages),
        "weight_GBps": round(sum(p.N * p.K // 4 for p in problems) / (ms * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round(alg_bytes(1, problems) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "matches_grouped_launches": bool(staged_ok), "wait_timed_out": bool(timed_out),
        "calls_with_a_wait_timed_out": int(timeouts_total),
        "note": "one token, 28 layers x 4 dependent stages, one cooperative launch"}
    del staged, launches, stages, flow_ys, ref

    return out


def i8_configs(torch, tb, synth, timer, dev, steps=100):
    """The I8_S encoder layers (int8 weights x int8 activations, fused bias and
    ReLU): one call = the row quantization launch + the int8 GEMM launch.  Four
    (x, y) buffer sets rotate so each call reads and writes HBM, not the MALL."""
    out = {}
    for name in sorted(synth.I8_LAYERS):
        M, K, N, relu = synth.I8_LAYERS[name]
        x, W, b = synth.i8_layer_inputs(name)
        q, s = tb.bitnet_i8_quant_weights(torch.from_numpy(W).to(dev))
        bd = torch.from_numpy(b).to(dev)
        x0 = torch.from_numpy(x).to(dev)
        xs = [x0] + [x0.clone() for _ in range(3)]
        ys = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in range(4)]
        ws = torch.empty(tb.bitnet_i8_linear_workspace_bytes(M, K), dtype=torch.uint8,
                         device=dev)
        call = lambda i=0: tb.bitnet_i8_linear_into(M, N, K, xs[i % 4], q, s, bd, relu,
                                                     ys[i % 4], ws)
        ms_host = timer.time(call, steps, warmup=100)
        ms = timer.graph_time(call, 40)
        moved = M * K * 4 + N * K + N * 4 + M * N * 4
        out[f"i8_linear_{name}"] = {
            "shape": {"M": M, "K": K, "N": N, "bias": True, "relu": relu},
            "us_per_call": round(ms * 1e3, 2),
            "us_per_call_python_launches": round(ms_host * 1e3, 2),
            "GBps_moved": round(moved / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "int8_TOPS": round(2 * M * N * K / (ms * 1e-3) / 1e12, 1),
            "bytes_moved": moved,
            "step": "row quantization launch + int8 MFMA GEMM launch (bias, ReLU in epilogue); "
                    "us_per_call is device time (40 calls in a HIP graph, replayed)"}
        del xs, ys, ws
    return out


def dwconv_config(torch, tb, synth, timer, dev, steps=100):
    """The encoder block's causal depthwise convolution (I8_S: per-channel int8
    kernel, per-channel activation scales) over 8192 frames x 512 channels, 7
    taps, with bias: the column-maximum launch and the convolution launch.
    Four (x, y) buffer sets rotate."""
    B, T, C, k = 1, synth.I8_FRAMES, 512, 7
    x0 = torch.from_numpy(synth.activations(B * T, C, 70100).reshape(B, T, C)).to(dev)
    W = torch.from_numpy(synth.normal_weights(C, k, 70101, std=0.1)).to(dev)
    b = torch.from_numpy(synth.normal_weights(1, C, 70102, std=0.1)[0]).to(dev)
    q, s = tb.bitnet_i8_dwconv_quant_weights(W)
    xs = [x0] + [x0.clone() for _ in range(3)]
    ys = [torch.empty_like(x0) for _ in range(4)]
    ws = torch.empty(tb.bitnet_i8_dwconv_workspace_bytes(B, T, C), dtype=torch.uint8, device=dev)
    call = lambda i=0: tb.bitnet_i8_dwconv_into(B, T, C, k, xs[i % 4], q, s, b, False,
                                                 ys[i % 4], ws)
    ms_host = timer.time(call, steps, warmup=50)
    ms = timer.graph_time(call, 40)
    alg = 2 * B * T * C * 4 + C * k + 2 * C * 4
    return {"shape": {"B": B, "T": T, "C": C, "k": k, "bias": True},
            "us_per_call": round(ms * 1e3, 2),
            "us_per_call_python_launches": round(ms_host * 1e3, 2),
            "GBps_moved": round(alg / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes": alg,
            "step": "column-maximum and convolution launches (x read twice); "
                    "us_per_call is device time (40 calls in a HIP graph, replayed)"}


def lmhead_configs(torch, tb, synth, timer, dev, steps=200):
    """The decoder's 8-bit table (151,936 x 1536, one scale per row): the
    lm_head at M = 1, 4 and 16 (one launch each: per-row activation
    quantization fused, int8 MFMA, exact per-column dequantization), three
    table copies rotated (702 MB) so each call reads HBM, not the MALL; and the
    embedding lookup of a 256-token prompt."""
    V, K = synth.VOCAB, synth.HIDDEN
    W = torch.from_numpy(synth.table_weights()).to(dev)
    q, s = tb.bitnet_table_quant(W)
    del W
    qs = [q] + [q.clone() for _ in range(2)]
    out = {}
    for M in (1, 4, 16):
        x = torch.from_numpy(synth.activations(M, K, synth.TABLE_SEED + 2)).to(dev)
        y = torch.empty((M, V), dtype=torch.float32, device=dev)
        ms = timer.time(lambda i=0: tb.bitnet_lm_head_into(M, V, K, x, qs[i % 3], s, y),
                        steps, warmup=100)
        alg = V * K + V * 4 + M * K * 4 + M * V * 4
        out[f"lm_head_m{M}"] = {
            "shape": {"M": M, "V": V, "K": K},
            "us_per_call": round(ms * 1e3, 2),
            "table_GBps": round(V * K / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes": alg,
            "kernel": "lm_head_kernel (one launch)"}
    ids = torch.from_numpy(synth.token_ids(256)).to(dev)
    e = torch.empty((256, K), dtype=torch.float32, device=dev)
    ms = timer.time(lambda i=0: tb.bitnet_embed_lookup_into(ids, 256, qs[i % 3], s, V, K, e),
                    steps, warmup=50)
    out["embed_lookup_t256"] = {
        "us_per_call": round(ms * 1e3, 2),
        "note": "256 token rows gathered and dequantized (1.6 MB written): launch-bound"}
    del qs, q, s
    return out


def lut_config(torch, tb, synth, timer, problems, packed, copy_b, w_scales, alg_bytes,
               decode_plans, dev, steps=1000):
    """The lookup-table variant over the M=1 decode sweep, timed like the headline
    (two packed copies alternate), with its outputs compared to the grouped
    call's on the same inputs."""
    xs_host = [synth.problem_activations(p, 1) for p in problems]
    xs = [torch.from_numpy(x).to(dev) for x in xs_host]
    ys = [torch.empty((1, p.N), dtype=torch.float32, device=dev) for p in problems]
    Ns, Ks = [p.N for p in problems], [p.K for p in problems]
    plans = [tb.LutPlan(xs, c, w_scales, ys, Ns, Ks) for c in (packed, copy_b)]
    ms = timer.time(lambda i=0: plans[i % 2].run(), steps, warmup=200)
    ref_plans, _, ref_ys = decode_plans(1, xs_host=xs_host, copies=(packed,))
    plans[0].run()
    ref_plans[0].run()
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(ys, ref_ys))
    pbytes = sum(p.N * p.K // 4 for p in problems)
    return {"us_per_step": round(ms * 1e3, 2),
            "weight_GBps": round(pbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(alg_bytes(1, problems) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                      4),
            "outputs_equal_grouped_call": bool(same),
            "kernel": "lut_gemv_grouped_kernel (16-entry tables per pair of codes in LDS)"}


def other_configs(torch, tb, synth, timer, problems, packed, copy_b, w_scales, alg_bytes,
                  decode_plans, dev):
    out = {}
    # The dependent per-token chain first.  Measured after the single-launch and
    # per-shape configs below, the staged call took 690 us per token instead of
    # 585 (host time per call unchanged at 35 us; the chain graph unchanged;
    # extra streams, HIP graphs, prior decode load or shifted allocations did
    # not reproduce it), so it runs on a fresh state.
    out.update(chain_configs(torch, tb, synth, timer, problems, packed, w_scales, alg_bytes,
                             decode_plans, dev))
    # Single 1536x1536 GEMV at M=1 (weights seed 0), 600 packed copies rotated
    # (354 MB) so each launch reads from HBM; this size is launch-latency bound.
    W, x = synth.single_gemv(seed=0)
    pk, sc = tb.bitnet_ternarize_pack(torch.from_numpy(W).to(dev))
    copies = [pk.clone() for _ in range(600)]
    xd = torch.from_numpy(x).to(dev)
    y = torch.empty((1, 1536), device=dev)
    ws = torch.empty(tb.bitnet_matmul_workspace_bytes(1, 1536), dtype=torch.uint8, device=dev)
    call = lambda i=0: tb.bitnet_ternary_matmul_into(1, 1536, 1536, xd, copies[i % 600], sc, y, ws)
    ms_host = timer.time(call, 600)
    ms = timer.graph_time(call, 600)
    out["single_gemv_1536x1536_m1"] = {
        "us_per_call": round(ms * 1e3, 2),
        "weight_GBps": round(1536 * 1536 / 4 / (ms * 1e-3) / 1e9, 1),
        "us_per_call_python_launches": round(ms_host * 1e3, 2),
        "note": "one 590 KB matrix per launch, latency bound; us_per_call is device time "
                "(600 calls in a HIP graph, replayed); the other figure is bound by the "
                "host's Python launch rate"}
    del copies

    # One decoder layer (7 projections, M=1) per grouped launch; steps walk the 28
    # layers so each launch reads fresh weights.
    layers = len(problems) // 7
    layer_plans = []
    for l in range(layers):
        probs = problems[7 * l:7 * l + 7]
        plans, _, _ = decode_plans(1, probs, copies=(packed,))
        layer_plans.append(plans[0])
    ms = timer.time(lambda i=0: layer_plans[i % layers].run(), 4 * layers)
    lb = sum(p.N * p.K // 4 for p in problems[:7])
    out["one_layer_m1"] = {"us_per_layer": round(ms * 1e3, 2),
                           "weight_GBps": round(lb / (ms * 1e-3) / 1e9, 1),
                           "frac_of_hbm_peak": round(alg_bytes(1, problems[:7]) /
                                                     (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    del layer_plans

    # Each projection shape on its own: single launches walking the 28 layers'
    # instances (two copies of each, so a launch rarely finds its matrix in
    # the last-level cache; the small shapes still fit there), and one grouped
    # launch over the 28 instances.
    per_shape = {}
    ws1 = torch.empty(tb.bitnet_matmul_workspace_bytes(1, synth.INTERMEDIATE), dtype=torch.uint8,
                      device=dev)
    for j, (name, K, N) in enumerate(synth.PROJECTIONS):
        idx = [i for i, p in enumerate(problems) if p.proj == j]
        inst = [(c[i], w_scales[i]) for c in (packed, copy_b) for i in idx]
        xd = torch.from_numpy(synth.problem_activations(problems[idx[0]], 1)).to(dev)
        yd = torch.empty((1, N), device=dev)
        call = lambda i=0: tb.bitnet_ternary_matmul_into(
            1, N, K, xd, inst[i % len(inst)][0], inst[i % len(inst)][1], yd, ws1)
        ms1_host = timer.time(call, 4 * len(inst))
        ms1 = timer.graph_time(call, 2 * len(inst))
        plans, _, _ = decode_plans(1, [problems[i] for i in idx])
        msg = timer.time(lambda i=0: plans[i % 2].run(), 100)
        b1 = N * K // 4
        per_shape[name] = {
            "K": K, "N": N,
            "single_us_per_call": round(ms1 * 1e3, 2),
            "single_weight_GBps": round(b1 / (ms1 * 1e-3) / 1e9, 1),
            "single_us_per_call_python_launches": round(ms1_host * 1e3, 2),
            "grouped28_us_per_launch": round(msg * 1e3, 2),
            "grouped28_weight_GBps": round(28 * b1 / (msg * 1e-3) / 1e9, 1)}
        del plans
    out["per_shape_m1"] = per_shape

    # Launch floor: the smallest call (M=1, N=64, K=128).
    pk0, sc0 = tb.bitnet_ternarize_pack(torch.ones((64, 128), device=dev))
    x0 = torch.ones((1, 128), device=dev)
    y0 = torch.empty((1, 64), device=dev)
    call = lambda i=0: tb.bitnet_ternary_matmul_into(1, 64, 128, x0, pk0, sc0, y0, ws1)
    ms0_host = timer.time(call, 500)
    ms0 = timer.graph_time(call, 200)
    out["launch_floor_m1_n64_k128"] = {
        "us_per_call": round(ms0 * 1e3, 2),
        "us_per_call_python_launches": round(ms0_host * 1e3, 2),
        "note": "the smallest call: device time per launch in a replayed HIP graph, and the "
                "rate at which Python enqueues the same call"}

    # The decode time must not depend on the codes: the sweep again with every
    # code 0 (field value 1 in all four positions of a byte).
    zero_codes = [torch.full_like(t, 0x55) for t in packed]
    zplans = [tb.GroupedPlan(1, xs_, zero_codes, w_scales, ys_, [p.N for p in problems],
                             [p.K for p in problems])
              for xs_, ys_ in [([torch.from_numpy(synth.problem_activations(p, 1)).to(dev)
                                 for p in problems],
                                [torch.empty((1, p.N), device=dev) for p in problems])]]
    msz = timer.time(lambda i=0: zplans[0].run(), 200)
    rplans, _, _ = decode_plans(1)
    msr = timer.time(lambda i=0: rplans[0].run(), 200)
    out["decode_sweep_m1_code_independence"] = {
        "us_per_step_random_codes": round(msr * 1e3, 2),
        "us_per_step_all_zero_codes": round(msz * 1e3, 2),
        "note": "both from one copy of the weights (not rotated, so partly served by the "
                "last-level cache); only the codes differ"}
    del zero_codes, zplans, rplans


    pbytes = sum(p.N * p.K // 4 for p in problems)
    out.update(i8_configs(torch, tb, synth, timer, dev))
    out["i8_dwconv_encoder"] = dwconv_config(torch, tb, synth, timer, dev)
    out.update(lmhead_configs(torch, tb, synth, timer, dev))
    out["decode_sweep_m1_lut"] = lut_config(torch, tb, synth, timer, problems, packed, copy_b,
                                            w_scales, alg_bytes, decode_plans, dev)
    # The first launches on freshly allocated buffers run slower (M=4: about 72
    # us per step over 100 steps after 3 warm-up, 67.5 over 1000 after 200), so
    # these sweeps take the headline's warm-up.
    for M in (4, 16):
        plans, _, _ = decode_plans(M)
        ms = timer.time(lambda i=0: plans[i % 2].run(), 1000, warmup=200)
        out[f"decode_sweep_m{M}"] = {
            "us_per_step": round(ms * 1e3, 2), "weight_GBps": round(pbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(alg_bytes(M, problems) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        del plans

    # The same sweeps with the inputs a decoder shares: a layer's q, k and v
    # read one buffer and its gate and up another, so the grouped call
    # quantizes each such input once (112 inputs instead of 196).
    for M in (4, 16):
        shared = {}
        xs_sh = []
        for p in problems:
            key = (p.layer, (0, 0, 0, 1, 2, 2, 3)[p.proj])
            if key not in shared:
                shared[key] = torch.from_numpy(synth.problem_activations(p, M)).to(dev)
            xs_sh.append(shared[key])
        ys = [torch.empty((M, p.N), dtype=torch.float32, device=dev) for p in problems]
        plans = [tb.GroupedPlan(M, xs_sh, c, w_scales, ys, [p.N for p in problems],
                                [p.K for p in problems]) for c in (packed, copy_b)]
        ms = timer.time(lambda i=0: plans[i % 2].run(), 1000, warmup=200)
        sb = (pbytes + sum(x.numel() * 4 for x in shared.values()) +
              sum(M * p.N * 4 for p in problems) + 4 * len(problems))
        out[f"decode_sweep_m{M}_shared_inputs"] = {
            "us_per_step": round(ms * 1e3, 2), "weight_GBps": round(pbytes / (ms * 1e-3) / 1e9, 1),
            "distinct_inputs": len(shared),
            "frac_of_hbm_peak": round(sb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        del plans, ys, xs_sh, shared

    # Prefill at M=256 (30 s of audio + prompt) over the sweep's 196 matrices,
    # activations seed 30000+7l+p.
    layers = len(problems) // 7
    M = synth.PREFILL_M_30S
    out[f"prefill_m{M}"] = prefill_config(torch, tb, synth, timer, synth.prefill_problems(layers),
                                          packed, w_scales, M, dev, SWEEP_WEIGHTS)
    out[f"prefill_one_layer_m{M}"] = prefill_layer_config(
        torch, tb, synth, timer, synth.prefill_problems(layers), packed, w_scales, M, dev)

    # Long-form prefill (M=1800, 4 min of audio) and batched decode (M=32, 64)
    # on their own weights: 196 Student-t(3) masters scaled to std 0.01,
    # weights seed 50000+7l+p, activations seed 60000+7l+p.
    lf = synth.longform_problems(layers)
    t0 = time.perf_counter()
    lf_packed, lf_scales = pack_set(torch, tb, synth, lf, True, dev)
    lf_zero = zero_code_fraction(torch, lf_packed)
    out["longform_weights"] = {"matrices": len(lf), "zero_code_fraction": round(lf_zero, 4),
                               "host_draw_and_pack_s": round(time.perf_counter() - t0, 1),
                               "generator": LONGFORM_WEIGHTS}
    M = synth.PREFILL_M_LONG
    out[f"prefill_m{M}"] = prefill_config(torch, tb, synth, timer, lf, lf_packed, lf_scales, M,
                                          dev, LONGFORM_WEIGHTS, zero_codes_check=True)
    out[f"prefill_m{M}"]["zero_code_fraction"] = round(lf_zero, 4)
    for M in (synth.PREFILL_M_30S, synth.PREFILL_M_LONG):
        out[f"prefill_per_shape_m{M}"] = prefill_shapes_config(
            torch, tb, timer, problems, packed, w_scales, M, dev)

    # Batched decode: M=32 and 64 on the 28 gate and 28 down long-form matrices,
    # two packed copies alternating.
    sub_i = [i for i, p in enumerate(lf) if p.proj in (4, 6)]
    sub = [lf[i] for i in sub_i]
    lf_copy = {i: lf_packed[i].clone() for i in sub_i}
    for M in (32, 64):
        xs = host_activations(torch, synth, sub, M, dev)
        ys = [torch.empty((M, p.N), device=dev) for p in sub]
        plans = [tb.GroupedPlan(M, xs, [c[i] for i in sub_i], [lf_scales[i] for i in sub_i], ys,
                                [p.N for p in sub], [p.K for p in sub])
                 for c in (lf_packed, lf_copy)]
        ms = timer.time(lambda i=0: plans[i % 2].run(), 500, warmup=100)
        sb = sum(p.N * p.K // 4 for p in sub)
        ops = 2.0 * M * sum(p.N * p.K for p in sub)
        out[f"batched_decode_m{M}"] = {
            "us_per_step": round(ms * 1e3, 2), "weight_GBps": round(sb / (ms * 1e-3) / 1e9, 1),
            "int8_TOPS": round(ops / (ms * 1e-3) / 1e12, 1),
            "frac_of_hbm_peak": round(alg_bytes(M, sub) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "weights": LONGFORM_WEIGHTS, "zero_code_fraction": round(lf_zero, 4)}
        del xs, ys, plans
    del lf_packed, lf_scales, lf_copy
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
