"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--causal 0|1]
                    [--dtype bf16|fp16|fp8] [--no-cpu-baseline] [--no-fp8] [--no-decode]
                    [--no-configs] [--variant NAME] [--ablation] [--copy-calibration]

A step is one attention forward over the workload's synthetic Q, K, V, already
resident in HBM.  The default workload is one layer of a 70B-class model with
grouped KV heads (B=1, 64 query heads over 8 KV heads, N=8192, d=128), run
non-causal in bf16 (the "bf16, non-causal, d=128, N >= 8k" operating point).
With --dtype fp8 a step is attn_fwd_fp8 on E4M3 codes prepared once by
hadamard_rotate (rotation + quantisation, timed separately as the prologue).

Prints ONE JSON line: throughput in TFLOPS (4·N²·d·Hq·B per step, halved when
causal; mean over the timed steps, plus per-launch median and min; the other GPU
legs below run before the timed steps, so that the GPU's clocks have settled), the
attention kernel's roofline against the dense matrix-core peak (and against that peak
scaled to the shader clock a one-wave probe on a second stream measures under the same load),
its HBM traffic when a counter measurement of the current kernel source is on
record under profiles/, the fp8 leg on the same shape (unless --no-fp8 or
--dtype fp8) with its HBM-bound prologue timed with and without the fused
rotary embedding, and the CPU oracle timed on a bounded row sample of the
workload.

The default run also reports the fp8 path's output RMSE against exact attention of the 16-bit
inputs, with and without the Hadamard rotation, on the outlier workload ("fp8_rmse"), and times
one decode step over an FP8 KV cache (B=4 sequences of up to
131072 cached tokens, 64 query heads over 8 KV heads; "decode" in the JSON line, HBM roofline
on algorithmic bytes); --workload decode_fp8kv_b4_h64kv8_n131072 makes the decode step the
benchmarked step (GB/s, with the decode oracle timed on one sequence's KV head).

The default run also times every other workload of the method's configurations
once each ("configs": MHA fp16 2k non-causal and causal, the 8k GQA layer causal,
the 128k causal prefill, and the fp8 outlier workload with and without rotation
next to bf16 on the same inputs), with ms, TFLOPS and fraction of peak.

--variant NAME routes every call through a scheduling variant of the library
(libtattn_NAME.so, built by build.py).  --ablation times the workload with the
shipped library and every variant, interleaved over rounds, and prints one JSON
line with each variant's median time and its change against the shipped build.

--sweep times the bf16 kernel (both masks) and the fp8 kernel over a list of
shapes (sequence lengths 2k to 128k, GQA and MHA, d = 64 and 128) and prints one
JSON line.

--copy-calibration runs only a plain device copy of known size (for scaling
the FETCH_SIZE / WRITE_SIZE counters of a profiler run) and exits.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Dense matrix-core peaks of MI355X (TFLOP/s)
PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp8": 5033.2}
HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCES = {"attn_fwd16_kernel": ["attn_fwd16.hip", "tattn_pipeline.hpp", "tattn_device.hpp"],
                  "attn_fwd_fp8_kernel": ["attn_fwd_fp8.hip", "tattn_pipeline.hpp", "tattn_device.hpp"],
                  "attn_decode_split_kernel": ["attn_decode.hip", "tattn_pipeline.hpp", "tattn_device.hpp"]}
COPY_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed launches first (the clocks take ~0.1 s of load to settle)")
    ap.add_argument("--workload", default="gqa_bf16_h64kv8_n8192",
                    help="a prefill workload, or a decode workload (decode_fp8kv_...) to time the decode step alone")
    ap.add_argument("--causal", type=int, default=0)
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp16", "fp8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="query rows per head in the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode leg of the default run")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads' legs")
    ap.add_argument("--variant", default=None, help="time a scheduling variant of the library instead")
    ap.add_argument("--ablation", action="store_true", help="time the shipped library against every variant")
    ap.add_argument("--rounds", type=int, default=4, help="interleaved rounds of --ablation")
    ap.add_argument("--sweep", action="store_true",
                    help="time the 16-bit and fp8 kernels over a list of shapes (one JSON line) and exit")
    return ap.parse_args()


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "tiled_attention_10_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from a counter run of this exact kernel source, else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{kernel}:{workload}")
    if not rec or rec.get("source_sha") != source_hash(kernel):
        return None
    return rec.get("traffic_bytes")


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
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOPS", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(rows)} random query rows x {Hq} heads x B={B} (exact fp64 rows), "
                      f"{flops:.3e} flop in {dt:.2f} s"}


def time_launches(torch, fn, steps, warmup, stream, min_warm_s=0.0):
    """Mean ms per launch over ``steps`` launches after ``warmup`` untimed ones (and, with
    ``min_warm_s``, more untimed launches until that much wall time has passed, so that a
    short kernel is timed at the clocks a sustained run settles to)."""
    t0 = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_warm_s:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, time.perf_counter() - t0


def launch_stats(torch, fn, n, stream):
    """Median and min of n launches, each between its own pair of events (run after
    the bracketed timing, so it does not change ``value``)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in ev:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    return round(t[len(t) // 2], 4), round(t[0], 4)


def fp8_inputs(T, torch, W, w, q, k, v, dev):
    """E4M3 inputs of the fp8 leg, made by the one-launch prologue, and the prologue variants
    to time: (inputs, prologue, (with the rotary embedding, embedding as a pass of its own,
    the plain prologue as three calls))."""
    signs = torch.from_numpy(W.rotation_signs(w.wid, w.d)).to(dev)
    ins = T.fp8_prologue(q, k, v, signs)
    q8, k8, v8, sq, sk, sv = ins

    def prologue():
        T.fp8_prologue(q, k, v, signs, out=ins)

    cos, sin = (torch.from_numpy(t).to(dev) for t in W.rotary_tables(w.wid, q.shape[1], q.shape[3]))

    def prologue_rope():
        # the same prologue with the rotary embedding of Q and K fused in
        T.fp8_prologue(q, k, v, signs, (cos, sin), out=ins)

    def prologue_three_calls():
        T.hadamard_rotate(q, signs, quantize=True, out=q8, scales=sq)
        T.hadamard_rotate(k, signs, quantize=True, out=k8, scales=sk)
        T.hadamard_rotate(v, None, quantize=True, out=v8, scales=sv)

    qr, kr = torch.empty_like(q), torch.empty_like(k)

    def prologue_rope_unfused():
        # rotary embedding as a pass of its own (16-bit out), then the plain prologue
        T.rope_hadamard_rotate(q, cos, sin, None, out=qr)
        T.rope_hadamard_rotate(k, cos, sin, None, out=kr)
        T.hadamard_rotate(qr, signs, quantize=True, out=q8, scales=sq)
        T.hadamard_rotate(kr, signs, quantize=True, out=k8, scales=sk)
        T.hadamard_rotate(v, None, quantize=True, out=v8, scales=sv)

    return ins, prologue, (prologue_rope, prologue_rope_unfused, prologue_three_calls)


def prologue_bytes(q, k, v):
    """HBM bytes of the fp8 prologue: 16-bit inputs read once, E4M3 codes and block
    scales written once (the small rotary tables and signs not counted)."""
    n = q.numel() + k.numel() + v.numel()
    blocks = sum(t.shape[0] * t.shape[2] * ((t.shape[1] + 63) // 64) for t in (q, k, v))
    return 2 * n + n + 4 * blocks


def measured_clock_ghz(torch, fn, dev, launches=20):
    """Shader clock (GHz) while the benchmarked kernel runs: a one-wave probe on a second
    stream (default priority) reads the shader cycle counter against the 100 MHz
    reference counter for ~20 ms while ``launches`` kernels run on the current stream.
    None if the probe library is missing."""
    import ctypes

    path = os.path.join(ROOT, "tiled_attention_10_amd", "libtattn_clock.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    u64 = ctypes.c_ulonglong
    L.tattn_clock_probe.argtypes = [u64, u64, ctypes.c_void_p, ctypes.c_void_p]
    L.tattn_clock_probe.restype = ctypes.c_int
    out = torch.zeros(2, dtype=torch.int64, device=dev)
    side = torch.cuda.Stream(dev)
    torch.cuda.synchronize()
    if L.tattn_clock_probe(2_000_000, 10_000_000, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(side.cuda_stream)):
        return None
    for _ in range(launches):
        fn()
    torch.cuda.synchronize()
    ticks, cycles = (int(x) for x in out.tolist())
    return round(cycles / ticks * 0.1, 3) if ticks > 0 else None


def fp8_rmse_leg(T, torch, W, dev, nrows=None):
    """Output RMSE of the fp8 path against exact attention of the unquantised 16-bit inputs,
    with and without the random-sign Hadamard rotation of Q and K, on the outlier workload
    (one x20 channel per head).  Q, K, V are quantised by the GPU prologue and attended by the
    fp8 kernel; the reference is the fp64 CPU oracle on every query row (or ``nrows`` seeded
    rows) of every (batch, head), computed on the host after every timed region."""
    import numpy as np
    from oracle import attention as A

    w = W.WORKLOADS["fp8_outlier_b2_h16_n4096"]
    qh, kh, vh = (W.to_torch(x, "bf16") for x in W.qkv_f32(w))
    q, k, v = qh.to(dev), kh.to(dev), vh.to(dev)
    rows = (np.arange(w.N) if nrows is None
            else np.sort(np.random.default_rng(w.wid).choice(w.N, nrows, replace=False)))
    signs = torch.from_numpy(W.rotation_signs(w.wid, w.d)).to(dev)
    outs = {}
    for rot in (False, True):
        sg = signs if rot else None
        q8, sq = T.hadamard_rotate(q, sg, quantize=True)
        k8, sk = T.hadamard_rotate(k, sg, quantize=True)
        v8, sv = T.hadamard_rotate(v, None, quantize=True)
        outs[rot] = T.attn_fwd_fp8(q8, k8, v8, sq, sk, sv).float().cpu().numpy()[:, rows]
    t0 = time.perf_counter()
    ref, _ = A.attention_rows(qh.float().numpy(), kh.float().numpy(), vh.float().numpy(), rows)
    dt = time.perf_counter() - t0
    res = {}
    for rot in (False, True):
        res["with_hadamard" if rot else "without_hadamard"] = round(float(np.sqrt(np.mean((outs[rot] - ref) ** 2))), 6)
    res["ratio_without_over_with"] = round(res["without_hadamard"] / res["with_hadamard"], 3)
    which = f"all {w.N}" if nrows is None else f"{nrows} seeded"
    res["sample"] = (f"{w.name}: {which} query rows x {w.Hq} heads x B={w.B}; reference: the fp64 "
                     f"CPU oracle (oracle.attention.attention_rows) on the bf16 inputs, {dt:.1f} s on the host")
    return res


def decode_inputs(T, torch, W, w, dev):
    """Query, E4M3 cache and device seqlens of a decode workload: seeded normal rows rounded to
    the query's type, block-quantised on the GPU (timing input only)."""
    q = W.to_torch(W.decode_query_f32(w), w.dtype).to(dev)
    kc = torch.empty((w.B, w.Nmax, w.Hkv, w.d), dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    nb = (w.Nmax + 63) // 64
    ks = torch.empty((w.B, w.Hkv, nb), dtype=torch.float32, device=dev)
    vs = torch.empty_like(ks)
    for b in range(w.B):
        kf, vf = W.decode_cache_f32(w, b)
        T.hadamard_rotate(W.to_torch(kf[None], w.dtype).to(dev), None, quantize=True, out=kc[b:b + 1],
                          scales=ks[b:b + 1])
        T.hadamard_rotate(W.to_torch(vf[None], w.dtype).to(dev), None, quantize=True, out=vc[b:b + 1],
                          scales=vs[b:b + 1])
    seqlens = w.seqlens()
    return q, kc, vc, ks, vs, torch.from_numpy(seqlens).to(dev), seqlens


def decode_cpu_baseline(q, kc, ks, vc, vs, seqlens, w):
    """The decode oracle on one (sequence, KV head) slice: the last (full-length) sequence, KV head 0."""
    import numpy as np
    from oracle import decode as D

    b, g = w.B - 1, w.Hq // w.Hkv
    qs = q[b:b + 1, :g].float().cpu().numpy()
    kcs, vcs = kc[b:b + 1, :, :1].cpu().numpy(), vc[b:b + 1, :, :1].cpu().numpy()
    kss, vss = ks[b:b + 1, :1].cpu().numpy(), vs[b:b + 1, :1].cpu().numpy()
    L = int(seqlens[b])
    t0 = time.perf_counter()
    D.decode_attention(qs, kcs, kss, vcs, vss, [L])
    dt = time.perf_counter() - t0
    nbytes = L * w.d * 2 + 2 * 4 * ((L + 63) // 64) + 2 * g * w.d * 2
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": _cores(), "kind": "oracle",
            "sample": f"sequence {b} (L={L}), KV head 0 with its {g} query heads: {nbytes} algorithmic bytes "
                      f"in {dt:.2f} s"}


def _cores():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] + [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count()


def decode_bench(T, torch, W, name, steps, warmup, stream, dev, cpu=True, min_warm_s=0.0):
    """Time one decode step (split + merge kernels) on a decode workload; HBM roofline."""
    w = W.DECODE_WORKLOADS[name]
    q, kc, vc, ks, vs, sl, seqlens = decode_inputs(T, torch, W, w, dev)
    out = torch.empty_like(q)
    ws = torch.empty(T.decode_workspace_size(w.B, w.Nmax, w.Hq, w.Hkv, w.d), dtype=torch.uint8, device=dev)
    fn = lambda: T.attn_decode_fp8kv(q, kc, vc, ks, vs, sl, out=out, workspace=ws)
    ms, wall = time_launches(torch, fn, steps, warmup, stream, min_warm_s)
    med, mn = launch_stats(torch, fn, steps, stream)
    nbytes = w.hbm_bytes(seqlens)
    gbps = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": name, "B": w.B, "Nmax": w.Nmax, "seqlens": [int(x) for x in seqlens], "Hq": w.Hq,
           "Hkv": w.Hkv, "d": w.d, "ms_per_step": round(ms, 4), "ms_median": med, "ms_min": mn,
           "GB_per_s": round(gbps, 1), "tokens_per_s": round(w.B / (ms * 1e-3), 1),
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(gbps / HBM_PEAK_GBPS, 4),
                        "traffic": recorded_traffic("attn_decode_split_kernel", name),
                        "kernel": "attn_decode_split_kernel + attn_decode_merge_kernel (one step)",
                        "bytes_per_launch": nbytes, "source_sha": source_hash("attn_decode_split_kernel")},
           "wall_s_timed": round(wall, 3)}
    if cpu:
        res["cpu_baseline"] = decode_cpu_baseline(q, kc, ks, vc, vs, seqlens, w)
    return res


def _tf(flops, ms):
    return round(flops / (ms * 1e-3) / 1e12, 2)


def config_legs(T, torch, W, stream, dev, steps=20, warmup=10, min_warm_s=0.25):
    """Each remaining workload of the method's configurations timed once (inputs resident
    in HBM): ms per launch (mean over ``steps`` after at least ``warmup`` launches and
    ``min_warm_s`` seconds of them), TFLOPS, fraction of peak."""
    out = {}

    def leg(name, fn, flops, peak_key, **kw):
        ms, _ = time_launches(torch, fn, steps, warmup, stream, min_warm_s)
        out[name] = {"ms": round(ms, 4), "tflops": _tf(flops, ms),
                     "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS[peak_key], 4), **kw}
        print(f"[bench] config {name}: {ms:.4f} ms", file=sys.stderr, flush=True)
        return ms

    w = W.WORKLOADS["mha_fp16_b4_h16_n2048"]
    q, k, v = (W.to_torch(x, "fp16").to(dev) for x in W.qkv_f32(w))
    o = torch.empty_like(q)
    for c in (False, True):
        leg(f"{w.name}_{'causal' if c else 'noncausal'}", lambda: T.attn_fwd(q, k, v, causal=c, out=o),
            w.flops(c), "fp16", dtype="fp16")
    w = W.WORKLOADS["gqa_bf16_h64kv8_n8192"]
    q, k, v = (W.to_torch(x, "bf16").to(dev) for x in W.qkv_f32(w))
    o = torch.empty_like(q)
    leg(f"{w.name}_causal", lambda: T.attn_fwd(q, k, v, causal=True, out=o), w.flops(True), "bf16", dtype="bf16")
    w = W.WORKLOADS["long_bf16_h8kv1_n131072"]
    q, k, v = (W.to_torch(x, "bf16").to(dev) for x in W.qkv_f32(w))
    o = torch.empty_like(q)
    leg(f"{w.name}_causal", lambda: T.attn_fwd(q, k, v, causal=True, out=o), w.flops(True), "bf16",
        dtype="bf16")
    del q, k, v, o
    w = W.WORKLOADS["fp8_outlier_b2_h16_n4096"]
    q, k, v = (W.to_torch(x, "bf16").to(dev) for x in W.qkv_f32(w))
    o = torch.empty_like(q)
    f = w.flops(False)
    ms16 = leg(f"{w.name}_bf16", lambda: T.attn_fwd(q, k, v, out=o), f, "bf16", dtype="bf16")
    signs = torch.from_numpy(W.rotation_signs(w.wid, w.d)).to(dev)
    for rot in (False, True):
        sg = signs if rot else None
        q8, sq = T.hadamard_rotate(q, sg, quantize=True)
        k8, sk = T.hadamard_rotate(k, sg, quantize=True)
        v8, sv = T.hadamard_rotate(v, None, quantize=True)
        name = f"{w.name}_fp8_{'with' if rot else 'without'}_hadamard"
        ms8 = leg(name, lambda: T.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, out=o), f, "fp8", dtype="fp8")
        out[name]["speedup_vs_bf16"] = round(ms16 / ms8, 3)
    return out


SWEEP_SHAPES = [  # B, N, Hq, Hkv, d
    (16, 2048, 64, 8, 128), (8, 4096, 64, 8, 128), (1, 8192, 64, 8, 128), (1, 16384, 64, 8, 128),
    (1, 32768, 32, 4, 128), (1, 131072, 8, 1, 128), (4, 8192, 32, 32, 128), (1, 8192, 64, 8, 64),
]


def sweep(args, T, torch, W, stream, dev):
    """TFLOPS of the bf16 kernel (non-causal and causal) and of the fp8 kernel on E4M3 codes from
    the one-launch prologue with seeded signs, over SWEEP_SHAPES; each timing is the mean of
    ``steps`` launches after at least ``warmup`` launches and 0.25 s of them."""
    out = []
    for (B, N, Hq, Hkv, d) in SWEEP_SHAPES:
        q, k, v = (W.to_torch(x, "bf16").to(dev) for x in W.random_qkv(1000 + N + d, B, N, Hq, Hkv, d))
        o = torch.empty_like(q)
        row = {"B": B, "N": N, "Hq": Hq, "Hkv": Hkv, "d": d}
        for causal in (False, True):
            fl = 4.0 * N * N * d * Hq * B / (2 if causal else 1)
            ms, _ = time_launches(torch, lambda: T.attn_fwd(q, k, v, causal=causal, out=o), args.steps,
                                  args.warmup, stream, min_warm_s=0.25)
            row["bf16_causal" if causal else "bf16"] = _tf(fl, ms)
            if d == 128:
                ins = T.fp8_prologue(q, k, v, torch.from_numpy(W.rotation_signs(N, d)).to(dev))
                ms8, _ = time_launches(torch, lambda: T.attn_fwd_fp8(*ins, causal=causal, out=o), args.steps,
                                       args.warmup, stream, min_warm_s=0.25)
                row["fp8_causal" if causal else "fp8"] = _tf(fl, ms8)
        print(f"[sweep] {row}", file=sys.stderr, flush=True)
        out.append(row)
        del q, k, v, o
    return {"metric": "attention fwd TFLOPS over shapes (4·N²·d·H, causal/2)", "unit": "TFLOPS", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "shapes": out}


def ablation(args, T, torch, W, stream, dev):
    """The workload timed with the shipped library and each scheduling variant, in
    interleaved rounds (shipped, v1, v2, ..., shipped, v1, ...), median over rounds."""
    import statistics
    from tiled_attention_10_amd.build import FP8_VARIANTS, VARIANTS

    w = W.WORKLOADS[args.workload]
    causal = bool(args.causal)
    dt = "bf16" if args.dtype == "fp8" else args.dtype
    q, k, v = (W.to_torch(x, dt).to(dev) for x in W.qkv_f32(w))
    o = torch.empty_like(q)
    if args.dtype == "fp8":
        ins, _, _ = fp8_inputs(T, torch, W, w, q, k, v, dev)
        names = ["shipped"] + sorted(FP8_VARIANTS)
        step = lambda: T.attn_fwd_fp8(*ins, causal=causal, out=o)
    else:
        names = ["shipped"] + sorted(VARIANTS)
        step = lambda: T.attn_fwd(q, k, v, causal=causal, out=o)
    times = {n: [] for n in names}
    for r in range(args.rounds):
        for n in names:
            path = T.LIB_PATH if n == "shipped" else T.variant_path(n)
            with T.use_library(path):
                ms, _ = time_launches(torch, step, args.steps, args.warmup, stream)
            times[n].append(ms)
            print(f"[ablation] round {r} {n}: {ms:.4f} ms", file=sys.stderr, flush=True)
    flops = w.flops(causal)
    base = statistics.median(times["shipped"])
    res = {"metric": "attention fwd TFLOPS per scheduling variant (4·N²·d·H, causal/2)", "unit": "TFLOPS",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "rounds": args.rounds, "dtype": args.dtype,
           "config": {"workload": w.name + ("_causal" if causal else "_noncausal"), "B": w.B, "N": w.N,
                      "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "causal": causal},
           "variants": {}}
    for n in names:
        m = statistics.median(times[n])
        res["variants"][n] = {"ms_median": round(m, 4), "ms_rounds": [round(t, 4) for t in times[n]],
                              "tflops": _tf(flops, m), "delta_vs_shipped": round(base / m - 1, 4)}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the attention forward is benchmarked on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch
    import tiled_attention_10_amd as T
    from tiled_attention_10_amd import workloads as W

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.ablation:
        print(json.dumps(ablation(args, T, torch, W, stream, dev)), flush=True)
        return
    if args.sweep:
        print(json.dumps(sweep(args, T, torch, W, stream, dev)), flush=True)
        return
    if args.variant is not None:
        # every call below goes through the variant build of the library
        T.use_library(T.variant_path(args.variant)).__enter__()
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}), flush=True)
        return

    if args.workload in W.DECODE_WORKLOADS:
        print(f"[bench] decode {args.workload} steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)
        d = decode_bench(T, torch, W, args.workload, args.steps, args.warmup, stream, dev,
                         cpu=not args.no_cpu_baseline)
        res = {"metric": "decode step HBM GB/s (algorithmic bytes: valid FP8 cache rows + scales + q + o)",
               "value": d["GB_per_s"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
               "ms_per_step": d["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
               "dtype": "e4m3 cache / bf16", "data": "synthetic",
               "config": {"workload": args.workload, "B": d["B"], "Nmax": d["Nmax"], "Hq": d["Hq"],
                          "Hkv": d["Hkv"], "d": d["d"]},
               "roofline": d["roofline"], "ms_median": d["ms_median"], "ms_min": d["ms_min"],
               "tokens_per_s": d["tokens_per_s"], "wall_s_timed": d["wall_s_timed"]}
        if "cpu_baseline" in d:
            res["cpu_baseline"] = d["cpu_baseline"]
        print(json.dumps(res), flush=True)
        return

    w = W.WORKLOADS[args.workload]
    causal = bool(args.causal)
    src_dtype = "bf16" if args.dtype == "fp8" else args.dtype
    q, k, v = (W.to_torch(x, src_dtype) for x in W.qkv_f32(w))
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty(qd.shape, dtype=torch.bfloat16 if args.dtype == "fp8" else qd.dtype, device=dev)
    print(f"[bench] {w.name} dtype={args.dtype} causal={causal} steps={args.steps} warmup={args.warmup}",
          file=sys.stderr, flush=True)
    flops = w.flops(causal)
    wl_name = w.name + ("_causal" if causal else "_noncausal")

    # The other GPU legs run first, back to back, so that the step below is timed on a
    # GPU whose clocks have settled (after an idle period they ramp up over the first
    # ~20 launches); the legs that only use the host run last.
    pre = {}
    fp8_leg = args.dtype != "fp8" and not args.no_fp8 and w.d == 128
    if fp8_leg:
        ins8, prologue8, prologue_more = fp8_inputs(T, torch, W, w, qd, kd, vd, dev)
        out8 = torch.empty(out.shape, dtype=torch.bfloat16, device=dev)
        fms, _ = time_launches(torch, lambda: T.attn_fwd_fp8(*ins8, causal=causal, out=out8),
                               args.steps, args.warmup, stream, min_warm_s=0.25)
        pms, _ = time_launches(torch, prologue8, 20, 10, stream, min_warm_s=0.1)
        prms, _ = time_launches(torch, prologue_more[0], 20, 10, stream, min_warm_s=0.1)
        purms, _ = time_launches(torch, prologue_more[1], 20, 10, stream, min_warm_s=0.1)
        p3ms, _ = time_launches(torch, prologue_more[2], 20, 10, stream, min_warm_s=0.1)
        pbytes = prologue_bytes(qd, kd, vd)
        pre["fp8_prologue"] = {"ms": round(pms, 4), "with_rope_ms": round(prms, 4),
                               "with_rope_separate_pass_ms": round(purms, 4), "three_calls_ms": round(p3ms, 4),
                               "hbm_bytes": pbytes, "GB_per_s": round(pbytes / (pms * 1e-3) / 1e9, 1),
                               "with_rope_GB_per_s": round(pbytes / (prms * 1e-3) / 1e9, 1),
                               "frac_of_hbm_8TBps": round(pbytes / (pms * 1e-3) / 8e12, 4)}
        del out8
    if not args.no_configs:
        pre["configs"] = config_legs(T, torch, W, stream, dev)
    if not args.no_decode:
        pre["decode"] = decode_bench(T, torch, W, "decode_fp8kv_b4_h64kv8_n131072", args.steps, args.warmup,
                                     stream, dev, cpu=False, min_warm_s=0.25)

    extra = {}
    if args.dtype == "fp8":
        ins, prologue, _ = fp8_inputs(T, torch, W, w, qd, kd, vd, dev)
        kernel = "attn_fwd_fp8_kernel"
        step_fn = lambda: T.attn_fwd_fp8(*ins, causal=causal, out=out)
        ms, wall = time_launches(torch, step_fn, args.steps, args.warmup, stream)
        extra["ms_median"], extra["ms_min"] = launch_stats(torch, step_fn, args.steps, stream)
        pms, _ = time_launches(torch, prologue, max(3, args.steps // 4), 5, stream)
        extra["prologue_ms"] = round(pms, 4)
        extra["with_prologue_tflops"] = round(flops / ((ms + pms) * 1e-3) / 1e12, 2)
    else:
        kernel = "attn_fwd16_kernel"
        step_fn = lambda: T.attn_fwd(qd, kd, vd, causal=causal, out=out)
        ms, wall = time_launches(torch, step_fn, args.steps, args.warmup, stream)
        extra["ms_median"], extra["ms_min"] = launch_stats(torch, step_fn, args.steps, stream)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[args.dtype]
    clock = measured_clock_ghz(torch, step_fn, dev)

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
        "config": {"workload": wl_name, "B": w.B, "N": w.N, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
                   "causal": causal, **({"variant": args.variant} if args.variant else {})},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": recorded_traffic(kernel, wl_name),
                     "kernel": kernel, "flop_per_launch": flops, "source_sha": source_hash(kernel),
                     "clock_ghz_measured": clock,
                     "frac_at_measured_clock": round(tflops / (peak * clock / 2.4), 4) if clock else None},
        "wall_s_timed": round(wall, 3),
    }
    res.update(extra)
    if fp8_leg:
        res["fp8_prologue"] = pre["fp8_prologue"]
        pms = pre["fp8_prologue"]["ms"]
        res["fp8"] = {"ms_per_step": round(fms, 4), "tflops": round(flops / (fms * 1e-3) / 1e12, 2),
                      "frac_of_fp8_peak": round(flops / (fms * 1e-3) / 1e12 / PEAK_TFLOPS["fp8"], 4),
                      "prologue_ms": round(pms, 4), "speedup_vs_" + args.dtype: round(ms / fms, 3),
                      "speedup_incl_prologue": round(ms / (fms + pms), 3)}
    for key in ("configs", "decode"):
        if key in pre:
            res[key] = pre[key]
    if args.dtype != "fp8" and not args.no_fp8:
        res["fp8_rmse"] = fp8_rmse_leg(T, torch, W, dev)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(q, k, v, causal, args.cpu_rows, w.wid)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
