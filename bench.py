#!/usr/bin/env python3
"""Benchmark: causal GQA attention forward + backward on one MI355X, through the C ABI.

A step is one pass of the whole hot path over one batch of synthetic input, through the library's
training pair: the RoPE-fused forward (O and L; it also leaves the rotated queries and keys in the
shared workspace) then the backward (the delta preprocess and the main kernel: dQ, dK, dV), for
every layer of the workload.  Inputs are resident in HBM before the timed region; outputs and workspace are
preallocated; nothing is allocated or copied inside it.

Prints ONE JSON line.  value = whole-job algorithmic TFLOP/s with the causal pairs counted exactly:
14 * D * B * Hq * T(T+1)/2 per layer (forward 4*D, backward 10*D per pair).  After the timed steps,
the same K steps run again with an event pair around every call (kernel_avg_us, which includes
each pair's own overhead), then each call runs alone K times back to back between one event pair
(kernel_alone_us); the roofline is that of the call with the longest alone time, at that time.
Beside it: the FlashAttention-2-convention figure (7 B H T^2 D per layer), the step's algorithmic
bytes per second against the HBM peak, and, with the CPU baseline, `parity`: the timed step's own
layer-0 outputs against the oracle's on the sampled (batch, kv group) units, per output tensor.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--no-cpu-baseline]

With --qkv 1, the step is one call of the query/key/value projection (ne_qkv_proj: x W^T with
RoPE on queries and keys, written into the attention layout) on the 116M model's shapes, and
value = its TFLOP/s (2 * B*T * C * (Hq + 2 Hkv) D per call).

With --block 1, the step is one forward + backward of a pre-norm attention block of the 116M
model (block.py: RMSNorm, the projection, attention, output projection, residual; the library's
kernels for the projection, attention and RoPE, torch float32 for the rest), and value = its
algorithmic TFLOP/s.

With --decode D, the step is instead one decode call (ne_attn_decode: n new tokens per sequence
against a rotated bf16 KV cache, split over the key range and merged) on decode workload D, and
value = algorithmic HBM GB/s of that call (cache rows read once, queries read, outputs written).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}   # MI355X dense matrix peaks
PEAK_HBM_GBS = 8000.0
METRIC = "causal GQA attention fwd+bwd TFLOP/s (T=512,d=64); % of MI355X MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first (the default lets the clocks settle: ~40 ms of work)")
    ap.add_argument("--workload", type=int, default=3, help="workload id 1..5 (default: the 116M-model layer)")
    ap.add_argument("--decode", type=int, default=0, help="decode workload id 1..2 instead of the training step")
    ap.add_argument("--qkv", type=int, default=0, help="projection workload id (1) instead of the training step")
    ap.add_argument("--block", type=int, default=0, help="1: attention block forward + backward instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads (default: the host cores this process may use, see host_threads)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the bench, run a plain 256 MiB elementwise copy 5 times (reference kernel of "
                         "known traffic for HBM byte counters)")
    return ap.parse_args()


def host_threads():
    """Host cores the oracle may use: OMP_NUM_THREADS when the environment sets it (a GPU machine gives
    each GPU a fixed share of its cores this way), else every core of this process's affinity."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def host_info():
    """Total logical cores of the host and its CPU model (from /proc/cpuinfo)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_cores": os.cpu_count(), "cpu_model": model}


def device_info(torch, dev):
    """The GPU's name, architecture and compute-unit count as the runtime reports them (the peaks
    above are the published figures for 256 compute units)."""
    pr = torch.cuda.get_device_properties(dev)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", None), "compute_units": pr.multi_processor_count}


def kernel_bytes(w, elem):
    """Algorithmic HBM bytes per layer (every tensor read or written once)."""
    q = w.B * w.Hq * w.T * w.D * elem
    kv = w.B * w.Hkv * w.T * w.D * elem
    rows = w.B * w.Hq * w.T * 4
    return {
        "fwd": q + 2 * kv + q + rows,                     # Q, K, V in; O, L out
        "bwd_pre": 2 * q + rows,                          # O, dO in; delta out
        "bwd_main": q + 2 * kv + q + 2 * rows + q + 2 * kv,  # Q, K, V, dO, L, delta in; dQ, dK, dV out
    }


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter profile of this workload, or None
    when there is none or the kernel sources changed since it was taken."""
    from causal_gqa_flashattention_ne_amd import profsum
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    k = t.get("kernels", {}).get(kernel)
    if k is None or k.get("source_sha256") != profsum.source_hash(kernel):
        return None
    return k["read_bytes"] + k["write_bytes"]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the attention path is sharded by (batch, kv group) with no "
              "communication, so each GPU would run this same step on its share; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import causal_gqa_flashattention_ne_amd as ne
    import gen

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.decode:
        return bench_decode(args, dev)
    if args.qkv:
        return bench_qkv(args, dev)
    if args.block:
        return bench_block(args, dev)
    w = gen.WORKLOADS[args.workload]
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    elem = 2 if w.dtype == "bf16" else 4

    # ---- inputs resident in HBM, outputs and workspace preallocated ----
    layers = []
    host_inputs = []
    for layer in range(w.layers):
        q, k, v, do = gen.layer_inputs(w, layer)
        if layer == 0:
            host_inputs = (q, k, v, do)
        t = [torch.from_numpy(x).to(dev).to(tdt).contiguous() for x in (q, k, v, do)]
        layers.append(t)
    cs = ne.rope_table(w.T, w.D, w.theta, dev)
    p = ne.make_params(w.B, w.Hq, w.Hkv, w.T, w.D, ne._dtype_code(layers[0][0]), None, cs)
    ws = torch.empty(ne.bwd_workspace_bytes(p), dtype=torch.uint8, device=dev)   # shared by the pair
    outs = []
    for (q, k, v, do) in layers:
        outs.append((torch.empty_like(q), torch.empty(w.B, w.Hq, w.T, dtype=torch.float32, device=dev),
                     torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)))
    stream = torch.cuda.current_stream(dev)
    st = ne.ctypes.c_void_p(stream.cuda_stream)

    def step(ev=None):
        for li, ((q, k, v, do), (o, lse, dq, dk, dv)) in enumerate(zip(layers, outs)):
            if ev is not None:
                ev[0][li].record(stream)
            ne.attn_fwd_train_into(p, q, k, v, o, lse, ws, st)
            if ev is not None:
                ev[1][li].record(stream)
            ne.attn_bwd_train_preprocess_into(p, q, k, o, lse, do, ws, st)
            if ev is not None:
                ev[2][li].record(stream)
            ne.attn_bwd_main_into(p, q, k, v, lse, do, dq, dk, dv, ws, st)
            if ev is not None:
                ev[3][li].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps between two events on the launch stream ----
    K = args.steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(K):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / K

    # ---- the same K steps again with an event pair around every kernel call (same stream) ----
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(w.layers)] for _ in range(4)] for _ in range(K)]
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    dur = {"fwd": [], "bwd_pre": [], "bwd_main": []}
    for i in range(K):
        for li in range(w.layers):
            e = evs[i]
            dur["fwd"].append(e[0][li].elapsed_time(e[1][li]))
            dur["bwd_pre"].append(e[1][li].elapsed_time(e[2][li]))
            dur["bwd_main"].append(e[2][li].elapsed_time(e[3][li]))
    avg_us = {kname: 1000.0 * float(np.mean(v)) for kname, v in dur.items()}

    # ---- each call alone: K launches back to back (every layer's inputs in turn) between one event
    # pair on the launch stream, so no per-call event overhead enters its average duration ----
    def call(kname, li):
        (q, k, v, do), (o, lse, dq, dk, dv) = layers[li], outs[li]
        if kname == "fwd":
            ne.attn_fwd_train_into(p, q, k, v, o, lse, ws, st)
        elif kname == "bwd_pre":
            ne.attn_bwd_train_preprocess_into(p, q, k, o, lse, do, ws, st)
        else:
            ne.attn_bwd_main_into(p, q, k, v, lse, do, dq, dk, dv, ws, st)

    alone_us = {}
    for kname in ("fwd", "bwd_pre", "bwd_main"):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            for li in range(w.layers):
                call(kname, li)
        e1.record(stream)
        torch.cuda.synchronize()
        alone_us[kname] = 1000.0 * e0.elapsed_time(e1) / (K * w.layers)
    step()                                   # leave the outputs of one whole step in place
    torch.cuda.synchronize()

    pairs = w.causal_pairs
    flop_layer = 14.0 * w.D * pairs
    value = flop_layer * w.layers / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]

    # ---- roofline of the dominant kernel ----
    kflops = {"fwd": 4.0 * w.D * pairs, "bwd_pre": 0.0, "bwd_main": 10.0 * w.D * pairs}
    kbytes = kernel_bytes(w, elem)
    step_bytes = float(sum(kbytes.values())) * w.layers
    dom = max(alone_us, key=lambda kname: alone_us[kname])
    t_s = alone_us[dom] * 1e-6
    t_mfma = kflops[dom] / (peak * 1e12)
    t_hbm = kbytes[dom] / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": kflops[dom] / t_s / 1e12, "peak": peak, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": kbytes[dom] / t_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(w.name, dom)
    roof["kernel"] = dom
    roof["avg_us"] = alone_us[dom]
    roof["timing"] = "%d launches back to back between one HIP event pair on the launch stream" % (K * w.layers)
    roof["algorithmic_flop"] = kflops[dom]
    roof["algorithmic_bytes"] = kbytes[dom]
    roof["mfma_tflops"] = kflops[dom] / t_s / 1e12
    roof["hbm_gbs"] = kbytes[dom] / t_s / 1e9

    # ---- CPU baseline: the oracle on the host cores (rank 0, N = 1 only) ----
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        threads = args.cpu_threads or host_threads()
        q, k, v, do = host_inputs
        groups = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
        # bounded sample: whole kv groups of layer 0, up to ~10-30 s of CPU work
        est_core_s_per_group = 1.0e-9 * 14 * w.D * w.G * w.T * (w.T + 1) / 2 / 1.2   # ~1.2 GFLOP/s/core
        budget = 20.0 * threads
        n = max(1, min(len(groups), int(budget / max(est_core_s_per_group, 1e-9))))
        sample = groups[:n]
        used = min(threads, n)
        t0 = time.perf_counter()
        ref = oracle.attention(q, k, v, do, theta=w.theta, groups=sample, nthreads=used)
        dt = time.perf_counter() - t0
        # the timed path's own layer-0 outputs (left in place by the last step) against the oracle
        # on the sampled units: e(X) = max |X - X_ref| / max |X_ref| per output tensor
        o0, lse0, dq0, dk0, dv0 = (t.float().cpu().numpy().astype(np.float64) for t in outs[0])
        got = {"O": o0, "L": lse0, "dQ": dq0, "dK": dk0, "dV": dv0}
        want = dict(zip(("O", "L", "dQ", "dK", "dV"), ref))
        tol = 2e-2 if w.dtype == "bf16" else 1e-5
        errs = {}
        for name in got:
            kv_side = name in ("dK", "dV")
            sl = [(b, g) if kv_side else (b, slice(g * w.G, (g + 1) * w.G)) for b, g in sample]
            diff = max(float(np.max(np.abs(got[name][i] - want[name][i]))) for i in sl)
            scale = max(float(np.max(np.abs(want[name][i]))) for i in sl)
            errs[name] = diff / scale if scale > 0 else diff
        parity = {"max_rel_err": errs, "tol": tol, "pass": all(e <= tol for e in errs.values()),
                  "sample": "the timed step's layer-0 outputs on the units of the CPU sample"}
        sample_flop = 14.0 * w.D * len(sample) * w.G * w.T * (w.T + 1) / 2
        cpu = {"value": sample_flop / dt / 1e12, "unit": "TFLOP/s", "cores": used, "kind": "oracle",
               "sample": "%d of %d (batch, kv group) units of layer 0 (all %d query heads each, all T=%d "
                         "positions), forward+backward in double, %.2f s wall" %
                         (len(sample), len(groups), w.G, w.T, dt)}
        cpu.update(host_info())
        if w.dtype == "f32":
            # the small float32 workloads: the same sample on one core as well
            t0 = time.perf_counter()
            oracle.attention(q, k, v, do, theta=w.theta, groups=sample, nthreads=1)
            dt1 = time.perf_counter() - t0
            cpu["single_thread"] = {"value": sample_flop / dt1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                                    "seconds": dt1}

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded SplitMix64 normals; shapes of the workload)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "T": w.T, "D": w.D,
                   "layers": w.layers, "causal": True, "rope_theta": w.theta, "parallelism": "none (1 GPU)"},
        "pct_of_peak": 100.0 * value / peak,
        "peak_tflops": peak,
        # FlashAttention-2's causal count, 7 B H T^2 D per layer (the value above counts the
        # T(T+1)/2 pairs exactly)
        "fa2_convention_tflops": 7.0 * w.B * w.Hq * w.T * w.T * w.D * w.layers / (ms_per_step * 1e-3) / 1e12,
        # every tensor of the step read or written once, against the HBM peak
        "step_hbm_gbs": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_pct_of_hbm_peak": 100.0 * step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "device": device_info(torch, dev),
        "kernel_avg_us": avg_us,
        "kernel_alone_us": alone_us,
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    if args.copy_calibration:
        out["copy_calibration"] = copy_calibration(dev)
    print(json.dumps(out))


def copy_calibration(dev):
    """A kernel of known traffic for the HBM byte counters: reads 256 MiB and writes 256 MiB per
    launch, 5 launches."""
    import torch
    src = torch.ones(128 << 20, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    return {"kernel": "torch.neg (elementwise)", "read_bytes": src.numel() * 2, "write_bytes": dst.numel() * 2,
            "launches": 5}


def bench_qkv(args, dev):
    import torch

    import causal_gqa_flashattention_ne_amd as ne
    import gen

    w = gen.QKV_WORKLOADS[args.qkv]
    x, wt = gen.qkv_case(w.seed, w.B, w.T, w.C, w.Hq, w.Hkv, w.D)
    xd = torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous()
    wd = torch.from_numpy(wt).to(dev).to(torch.bfloat16).contiguous()
    cs = ne.rope_table(w.T, w.D, w.theta, dev)
    p = ne.make_qkv_params(w.B, w.T, w.C, w.Hq, w.Hkv, w.D, cs)
    q = torch.empty(w.B, w.Hq, w.T, w.D, dtype=torch.bfloat16, device=dev)
    k = torch.empty(w.B, w.Hkv, w.T, w.D, dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    stream = torch.cuda.current_stream(dev)
    st = ne.ctypes.c_void_p(stream.cuda_stream)

    def step():
        ne.qkv_proj_into(p, xd, wd, q, k, v, st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(K):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    avg_us = 1000.0 * float(np.mean([a.elapsed_time(b) for a, b in evs]))
    flop = float(w.flops)
    M, N = w.B * w.T, (w.Hq + 2 * w.Hkv) * w.D
    nbytes = 2 * (M * w.C + N * w.C + M * N)         # x, w read once; q, k, v written once
    peak = PEAK_TFLOPS["bf16"]
    roof = {"bound": "mfma", "achieved": flop / (avg_us * 1e-6) / 1e12, "peak": peak, "unit": "TFLOP/s"}
    if nbytes / (PEAK_HBM_GBS * 1e9) > flop / (peak * 1e12):
        roof = {"bound": "hbm", "achieved": nbytes / (avg_us * 1e-6) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(w.name, "qkv_proj")
    roof.update({"kernel": "qkv_proj", "avg_us": avg_us, "algorithmic_flop": flop, "algorithmic_bytes": nbytes})

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_limits
        threads = args.cpu_threads or host_threads()
        with threadpool_limits(limits=threads):
            t_s = time.perf_counter()
            passes = 0
            while True:               # the whole projection in double, repeated for >= 2 s
                oracle.qkv_proj(x, wt, w.Hq, w.Hkv, theta=w.theta)
                passes += 1
                if time.perf_counter() - t_s >= 2.0:
                    break
            dt = time.perf_counter() - t_s
        cpu = {"value": flop * passes / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "sample": "the whole projection in double (numpy matmul + RoPE) x %d passes, %.2f s wall"
                         % (passes, dt)}
        cpu.update(host_info())

    out = {
        "metric": "query/key/value projection with RoPE epilogue, TFLOP/s",
        "value": flop / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64 normals: x ~ N(0,1), w ~ N(0,1/C))",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "C": w.C, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "rope_theta": w.theta, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if args.copy_calibration:
        out["copy_calibration"] = copy_calibration(dev)
    print(json.dumps(out))


def bench_block(args, dev):
    import torch

    import causal_gqa_flashattention_ne_amd as ne
    import gen
    from causal_gqa_flashattention_ne_amd.block import block_forward_backward

    w = gen.QKV_WORKLOADS[1]                       # the 116M model's block: B 16, T 512, C 768
    B, T, C, Hq, Hkv, D = w.B, w.T, w.C, w.Hq, w.Hkv, w.D
    x, wqkv = gen.qkv_case(w.seed, B, T, C, Hq, Hkv, D)
    rng = np.random.default_rng(w.seed)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(torch.bfloat16).contiguous()
    xd, wd = t(x), t(wqkv)
    g = t(1.0 + 0.1 * rng.standard_normal(C))
    wo = t(rng.standard_normal((C, Hq * D)) / np.sqrt(Hq * D))
    dy = t(rng.standard_normal((B, T, C)))

    def step():
        return block_forward_backward(xd, g, wd, wo, dy, Hq, Hkv, rope_theta=w.theta)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    stream = torch.cuda.current_stream(dev)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(K):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K
    M, N = B * T, (Hq + 2 * Hkv) * D
    pairs = B * Hq * T * (T + 1) // 2
    proj = 2 * M * C * N + 2 * M * Hq * D * C            # projection and output projection, forward
    flop = 3 * proj + 14 * D * pairs                     # backward products twice the forward's
    out = {
        "metric": "pre-norm attention block forward+backward, algorithmic TFLOP/s",
        "value": flop / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64 normals)",
        "config": {"workload": "gpt116m-block-bf16", "B": B, "T": T, "C": C, "Hq": Hq, "Hkv": Hkv, "D": D,
                   "rope_theta": w.theta, "parallelism": "none (1 GPU)"},
        "algorithmic_flop": flop,
        "roofline": None,            # a composition: each library kernel has its own bench mode
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_limits
        threads = args.cpu_threads or host_threads()
        xs, ws, gs, wos, dys = x[:1], wqkv, g.float().cpu().numpy(), wo.float().cpu().numpy(), dy[:1].float().cpu().numpy()
        flop1 = flop / B                                 # one sequence
        with threadpool_limits(limits=threads):
            t_s = time.perf_counter()
            passes = 0
            while True:                                  # one sequence's block, for >= 2 s
                oracle.block(xs, gs, ws, wos, dys, Hq, Hkv, theta=w.theta)
                passes += 1
                if time.perf_counter() - t_s >= 2.0:
                    break
            dt = time.perf_counter() - t_s
        out["cpu_baseline"] = {"value": flop1 * passes / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
                               "kind": "oracle", "sample": "1 of %d sequences x %d passes, block forward + "
                               "backward in double, %.2f s wall" % (B, passes, dt)}
        out["cpu_baseline"].update(host_info())
    print(json.dumps(out))


def decode_bytes(w, lens):
    """Algorithmic HBM bytes of one decode call: the valid K and V cache rows, the queries, the
    table rows of the new tokens' positions, O and L."""
    cache = int(np.sum(lens, dtype=np.int64)) * w.Hkv * w.D * 2 * 2
    qo = 2 * w.B * w.Hq * w.n * w.D * 2
    return cache + qo + w.B * w.n * w.D * 4 + w.B * w.Hq * w.n * 4


def bench_decode(args, dev):
    import torch

    import causal_gqa_flashattention_ne_amd as ne
    import gen

    w = gen.DECODE_WORKLOADS[args.decode]
    q, k, v, lens = gen.decode_inputs(w)
    qd = torch.from_numpy(q).to(dev).to(torch.bfloat16).contiguous()
    kc = ne.rope_apply(torch.from_numpy(k).to(dev).to(torch.bfloat16).contiguous(), w.theta)
    vc = torch.from_numpy(v).to(dev).to(torch.bfloat16).contiguous()
    kl = torch.from_numpy(lens).to(dev)
    cs = ne.rope_table(w.cache_rows, w.D, w.theta, dev)
    p = ne.make_decode_params(w.B, w.Hq, w.Hkv, w.n, w.D, w.cache_rows, None, cs)
    o = torch.empty_like(qd)
    lse = torch.empty(w.B, w.Hq, w.n, dtype=torch.float32, device=dev)
    ws = torch.zeros(ne.decode_workspace_bytes(p), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    st = ne.ctypes.c_void_p(stream.cuda_stream)

    def step():
        ne.attn_decode_into(p, qd, kc, vc, kl, o, lse, ws, st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(K):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K
    # per-call durations from event pairs around every call, on the launch stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    avg_us = 1000.0 * float(np.mean([a.elapsed_time(b) for a, b in evs]))
    nbytes = decode_bytes(w, lens)
    roof = {"bound": "hbm", "achieved": nbytes / (avg_us * 1e-6) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # at most 16 query columns per kv group: one balanced kernel; otherwise split chunks + merge
    narrow = (w.Hq // w.Hkv) * w.n <= 16
    roof["traffic"] = measured_traffic(w.name, "decode16" if narrow else "decode_split")
    roof.update({"kernel": "decode16" if narrow else "decode_split + decode_merge", "avg_us": avg_us,
                 "algorithmic_bytes": nbytes})

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # the whole batch, one oracle call per sequence; the cache is rotated beforehand, untimed, as
        # the GPU call also receives a rotated cache
        kco = [oracle.rope(k[b:b + 1], w.theta) for b in range(w.B)]
        t_s = time.perf_counter()
        passes = 0
        while True:                   # whole batch, repeated for at least 2 s of wall time
            for b in range(w.B):
                oracle.decode(q[b:b + 1], kco[b], v[b:b + 1], lens[b:b + 1], theta=w.theta)
            passes += 1
            if time.perf_counter() - t_s >= 2.0:
                break
        dt = time.perf_counter() - t_s
        done, nb = w.B, nbytes * passes
        cpu = {"value": nb / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": "%d of %d sequences x %d passes, decode in double over the oracle-rotated cache, "
                         "%.2f s wall" % (done, w.B, passes, dt)}
        cpu.update(host_info())

    out = {
        "metric": "decode attention, algorithmic HBM GB/s of one call (KV cache read once)",
        "value": nbytes / (ms * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64 normals; ragged kv lengths uniform in [n, cache_rows])",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "n": w.n, "cache_rows": w.cache_rows,
                   "D": w.D, "kv_len_total": int(np.sum(lens)), "rope_theta": w.theta, "parallelism": "none (1 GPU)"},
        "tokens_per_s": w.B * w.n / (ms * 1e-3),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if args.copy_calibration:
        out["copy_calibration"] = copy_calibration(dev)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
