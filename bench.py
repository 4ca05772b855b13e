"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--causal 0|1]
                    [--dtype bf16|fp16|fp8] [--no-cpu-baseline]

A step is one attention forward over the workload's synthetic Q, K, V (already
resident in HBM).  The default workload is one layer of a 70B-class model
with grouped KV heads (B=1, 64 query heads over 8 KV heads, N=8192, d=128),
run non-causal in bf16.  Prints ONE JSON line with the throughput in TFLOPS
(4·N²·d·Hq·B per step, halved when causal), the roofline of the attention
kernel against the dense bf16 matrix-core peak, and the CPU oracle timed on a
bounded row sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp8": 5033.2}   # dense matrix-core peaks


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa_bf16_h64kv8_n8192")
    ap.add_argument("--causal", type=int, default=0)
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048, help="query rows per head in the oracle sample")
    return ap.parse_args()


def cpu_baseline(q, k, v, causal, rows_per_head, seed):
    """Time the oracle on a bounded sample: ``rows_per_head`` random query rows of every head."""
    import numpy as np
    from oracle import attention as A

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    B, N, Hq, d = q.shape
    rows = np.sort(np.random.default_rng(seed).choice(N, size=min(N, rows_per_head), replace=False))
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    t0 = time.perf_counter()
    A.attention_rows(qn, kn, vn, rows, None, causal)
    dt = time.perf_counter() - t0
    if causal:
        flops = sum(4.0 * (int(r) + 1) * d for r in rows) * Hq * B
    else:
        flops = 4.0 * len(rows) * N * d * Hq * B
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(rows)} random query rows x {Hq} heads x B={B} (exact fp64 rows), "
                      f"{flops:.3e} flop in {dt:.2f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the attention forward is benchmarked on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch
    import tiled_attention_10_amd as T
    from tiled_attention_10_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    causal = bool(args.causal)
    dev = torch.device("cuda:0")
    q, k, v = (W.to_torch(x, args.dtype) for x in W.qkv_f32(w))
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(qd)
    print(f"[bench] {w.name} dtype={args.dtype} causal={causal} steps={args.steps} warmup={args.warmup}",
          file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        T.attn_fwd(qd, kd, vd, causal=causal, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        T.attn_fwd(qd, kd, vd, causal=causal, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    flops = w.flops(causal)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[args.dtype]

    res = {
        "metric": "attention fwd TFLOPS (4·N²·d·H, causal/2)",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": w.name + ("_causal" if causal else "_noncausal"), "B": w.B, "N": w.N,
                   "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "causal": causal},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None,
                     "kernel": "attn_fwd16_kernel", "flop_per_launch": flops},
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(q, k, v, causal, args.cpu_rows, w.wid)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
