#!/usr/bin/env python3
"""Benchmark of the ternary projection path on one MI355X.

Workload (the JSON line's `value`): one decode token through every ternary
projection of the 28-layer, 1536-hidden decoder -- 196 matrices (q, k, v, o,
gate, up, down per layer), M = 1 -- as one grouped launch per step: per-row
int8 quantization of each projection's activations, the ternary x int8
contraction and the fp32 dequantization, all inside the decode kernel.  The
weights (seeded synthetic fp32 masters, ~N(0, 0.02)) are ternarized and packed
on the GPU once before timing, as the format ships pre-ternarized weights.
Two copies of the 327.5 MB packed set alternate between steps so the reads come
from HBM rather than the 256 MB last-level cache.

Also reported in the same line: the prefill half of the metric (M = 256 tokens
through the same 196 matrices, int8 TOPS), the offline ternarize+pack rate, and
the CPU oracle timed on a bounded sample of the decode workload on this host.
"""
from __future__ import annotations

import argparse
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


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=28)
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--prefill-m", type=int, default=256)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the timed CPU-oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path would shard by replicating weights per GPU, see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from ternary_weight_decoder_amd import binding as tb, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    tb.lib()
    stream = torch.cuda.current_stream()

    problems = synth.sweep_problems(args.layers)
    n_mat = len(problems)
    log(f"[bench] generating and ternarizing {n_mat} matrices on the GPU")

    # ---- offline: ternarize + pack every matrix on the GPU -------------------
    packed, w_scales = [], []
    ws_t = torch.empty(tb.bitnet_ternarize_workspace_bytes(synth.INTERMEDIATE), dtype=torch.uint8,
                       device=dev)
    tern_ms = 0.0
    w_bytes = 0
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

    # ---- decode sweep, M = 1 --------------------------------------------------
    M = 1
    xs_host = [synth.problem_activations(p, M) for p in problems]
    xs = [torch.from_numpy(x).to(dev) for x in xs_host]
    ys = [torch.empty((M, p.N), dtype=torch.float32, device=dev) for p in problems]
    Ns = [p.N for p in problems]
    Ks = [p.K for p in problems]
    copy_b = [t.clone() for t in packed]
    plans = [tb.GroupedPlan(M, xs, packed, w_scales, ys, Ns, Ks),
             tb.GroupedPlan(M, xs, copy_b, w_scales, ys, Ns, Ks)]
    alg_bytes = (packed_bytes + sum(M * p.K * 4 for p in problems) +
                 sum(M * p.N * 4 for p in problems) + 4 * n_mat)

    log(f"[bench] decode: warmup {args.warmup}, timed {args.steps} steps")
    for i in range(args.warmup):
        plans[i % 2].run()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        plans[i % 2].run()
    end.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    weight_gbps = packed_bytes / (ms_step * 1e-3) / 1e9
    achieved = alg_bytes / (ms_step * 1e-3) / 1e9
    log(f"[bench] decode {ms_step * 1e3:.1f} us/step, weight {weight_gbps:.0f} GB/s")

    # ---- prefill, M = 256 tokens through the same 196 matrices ---------------
    prefill = None
    if not args.no_prefill:
        Mp = args.prefill_m
        pproblems = synth.prefill_problems(args.layers)
        pxs = [torch.from_numpy(synth.problem_activations(p, Mp)).to(dev) for p in pproblems]
        pys = [torch.empty((Mp, p.N), dtype=torch.float32, device=dev) for p in pproblems]
        pplan = tb.GroupedPlan(Mp, pxs, packed, w_scales, pys, Ns, Ks)
        for _ in range(3):
            pplan.run()
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(args.prefill_steps):
            pplan.run()
        s1.record(stream)
        torch.cuda.synchronize()
        pms = s0.elapsed_time(s1) / args.prefill_steps
        ops = 2.0 * Mp * sum(p.N * p.K for p in pproblems)
        tops = ops / (pms * 1e-3) / 1e12
        prefill = {"workload": f"prefill M={Mp} over {len(pproblems)} matrices, one grouped call "
                               "(quantization launch + int8 MFMA GEMM launch)",
                   "ms_per_step": round(pms, 4), "int8_TOPS": round(tops, 2),
                   "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
                   "ops_per_step": ops}
        log(f"[bench] prefill {pms:.3f} ms/step, {tops:.0f} TOPS")
        del pxs, pys, pplan

    # ---- CPU oracle on a bounded sample of the decode workload ----------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cores = oracle.num_threads()
        t_spent, bytes_done, mats = 0.0, 0, 0
        max_rel = 0.0
        for i, p in enumerate(problems):
            W = synth.problem_weights(p)
            pk_ref, s_ref = oracle.ternarize_pack(W)      # offline step, not timed
            t0 = time.perf_counter()
            ref = oracle.ternary_matmul(xs_host[i], pk_ref, s_ref, p.N)
            t_spent += time.perf_counter() - t0
            bytes_done += p.N * p.K // 4
            mats += 1
            y_gpu = ys[i].cpu().numpy()
            rel = np.abs(y_gpu - ref["y"]) / np.maximum(np.abs(ref["y"]), 1e-30)
            max_rel = max(max_rel, float(rel.max()))
            if t_spent >= args.cpu_seconds:
                break
        cpu = {"value": round(bytes_done / t_spent / 1e9, 4), "unit": "GB/s", "cores": cores,
               "kind": "oracle",
               "sample": f"first {mats} of {n_mat} decode projections (layers in order, M=1): "
                         f"quantize + unpack + int32 matmul + dequant, {t_spent:.1f} s; "
                         f"GPU outputs agree with it to max rel err {max_rel:.2e}"}
        log(f"[bench] cpu oracle {cpu['value']} GB/s on {cores} threads ({mats} matrices)")

    line = {
        "metric": METRIC,
        "value": round(weight_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"decode sweep: {n_mat} ternary projections ({args.layers} layers "
                               "x q,k,v,o,gate,up,down; hidden 1536, intermediate 8960), M=1, "
                               "one grouped launch per step",
                   "M": M, "matrices": n_mat, "packed_weight_bytes": packed_bytes,
                   "weight_copies_rotated": 2},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None, "bytes_per_launch": alg_bytes},
        "cpu_baseline": cpu,
        "prefill": prefill,
        "ternarize_pack": {"ms_total": round(tern_ms, 3),
                           "fp32_read_GBps": round(w_bytes / (tern_ms * 1e-3) / 1e9, 1)},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
