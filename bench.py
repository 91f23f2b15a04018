#!/usr/bin/env python3
"""Benchmark of the routed MoE FFN layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--lines A,B|none]
                    [--gpus 1] [--pass backward|train]

One step = one full pass of the layer (routing, [MX quantization of x,]
gate/up + SwiGLU, down + weighted combine) over one batch of synthetic tokens,
with every input resident in HBM before the timed region starts.

Default headline: the Kimi-K2.7-Code-shaped batched layer at the pages'
2,048 tokens per GPU (H 7168, E 384 all resident, k 8, I 2048, BF16; the
largest shape, HBM-bound at ~43 routed rows per expert).  The same JSON line
carries, under "lines", the pages' other shapes measured in the same run: the
DeepSeek-V4-Pro-shaped MXFP8 layer, both one-GPU expert-parallel shares
(MFMA-bound), the Qwen3-style decode layer at T = 1, 8 and 32, and the
Qwen3.5-shaped Zipf-skewed decode at T = 64.  Decode steps cycle through
independent weight sets (like the layers of a model), so each step streams
weights the 256 MB last-level cache does not hold, and every step routes a
fresh batch of tokens; their throughput is that of the same steps replayed from a
HIP graph (8 captured steps per replay, as a serving loop would issue them; the
eager per-call figures are kept under "issue").  Lines named "<workload>:backward" time the
layer's backward pass on that shape (BF16 reading the pre-activations the
training forward kept; MXFP8 recomputing them), segment by segment.

With --pass backward (batched workloads, BF16 or MXFP8) a step is routing plus
the layer's backward pass instead (dx, both weight gradients, the routing-weight
and logit gradients for a seeded output gradient); --pass train adds the
forward before it.

Prints ONE JSON line.  Besides the throughput it carries
  roofline:     the dominant kernel's algorithmic HBM bytes (or MFMA flops)
                per launch divided by its average launch time, taken with HIP
                events recorded around that kernel on the library's stream
                during the timed steps, against the 8 TB/s HBM peak (or the
                dense MFMA peak of the dtype);
  cpu_baseline: the FP64 CPU oracle, timed on this host on a bounded sample
                of the same workload, with the cores, CPU model and thread
                settings it ran with.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

# the CPU oracle's BLAS threads: every core this process may use, unless set
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS"):
    os.environ.setdefault(_v, str(len(os.sched_getaffinity(0))))

import hashlib

METRIC = "MoE layer tokens/s; decode HBM TB/s % of peak; batched MFMA util %"
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "mixture_experts_ffn_07_amd", "csrc")

# HBM bytes per launch of the dominant kernel (read + written), from two rocprofv3
# counter passes (FETCH_SIZE, WRITE_SIZE) scaled by a 1 GiB copy
# (profiles/copy_calibration_1GiB.md).
# Each record holds a fingerprint of the kernel sources it was measured on; when
# the sources change the figure no longer describes the kernel and is reported
# as null until the counters are taken again.
TRAFFIC = {
    ("gemm_gate_up", "kimi-bf16-T2048"): (
        23012.2e6, ('batched.hip', 'common.h', 'tiles.h', 'internal.h'), "12e9ae18e929026f",
        "profiles/gemm_gate_up_kimi-bf16-T2048.md"),
    ("gemm_gate_up", "dsv4-mxfp8-T2048"): (
        18188.0e6, ('batched.hip', 'common.h', 'tiles.h', 'internal.h'), "12e9ae18e929026f",
        "profiles/gemm_gate_up_dsv4-mxfp8-T2048.md"),
    ("gemm_gate_up", "glm-bf16-T2048"): (
        13239.0e6, ('batched.hip', 'common.h', 'tiles.h', 'internal.h'), "12e9ae18e929026f",
        "profiles/gemm_gate_up_glm-bf16-T2048.md"),
    ("gemm_gate_up", "kimi-bf16-ep64share"): (
        2055.4e6, ('gemm_large.hip', 'common.h', 'tiles.h', 'internal.h'), "d632fb8a73731959",
        "profiles/gemm_gate_up_kimi-bf16-ep64share.md"),
    ("gemm_gate_up", "dsv4-mxfp8-ep64share"): (
        1671.8e6, ('gemm_large.hip', 'common.h', 'tiles.h', 'internal.h'), "d632fb8a73731959",
        "profiles/gemm_gate_up_dsv4-mxfp8-ep64share.md"),
    ("decode_gate_up", "qwen3-decode-T32"): (
        700.8e6, ('decode.hip', 'common.h', 'internal.h', 'route.h', 'tiles.h'), "fd2144a70db086dc",
        "profiles/decode_gate_up_qwen3-decode-T32.md"),
    ("decode_gate_up", "qwen3-decode-T1"): (
        50.9e6, ('decode.hip', 'common.h', 'internal.h', 'route.h', 'tiles.h'), "fd2144a70db086dc",
        "profiles/decode_gate_up_qwen3-decode-T1.md"),
    ("decode_gate_up", "qwen3-decode-T8"): (
        317.1e6, ('decode.hip', 'common.h', 'internal.h', 'route.h', 'tiles.h'), "fd2144a70db086dc",
        "profiles/decode_gate_up_qwen3-decode-T8.md"),
    ("decode_gate_up", "q35-zipf-T64"): (
        1114.8e6, ('decode.hip', 'common.h', 'internal.h', 'route.h', 'tiles.h'), "fd2144a70db086dc",
        "profiles/decode_gate_up_q35-zipf-T64.md"),
    ("gemm_gate_up", "qwen3-mxfp8-decode-T32"): (
        378.8e6, ('batched.hip', 'common.h', 'tiles.h', 'internal.h'), "12e9ae18e929026f",
        "profiles/gemm_gate_up_qwen3-mxfp8-decode-T32.md"),
    ("bwd_input", "kimi-bf16-T2048"): (
        24773.4e6, ('backward.hip', 'batched.hip', 'gemm_large.hip', 'common.h', 'tiles.h', 'internal.h'), "2bf00baff9e035ff",
        "profiles/bwd_kimi-bf16-T2048.md"),
    ("bwd_wgate_up", "kimi-bf16-T2048"): (
        22916.5e6, ('backward.hip', 'batched.hip', 'gemm_large.hip', 'common.h', 'tiles.h', 'internal.h'), "2bf00baff9e035ff",
        "profiles/bwd_kimi-bf16-T2048.md"),
    ("bwd_input", "kimi-bf16-ep64share"): (
        2189.0e6, ('backward.hip', 'batched.hip', 'gemm_large.hip', 'common.h', 'tiles.h', 'internal.h'), "2bf00baff9e035ff",
        "profiles/bwd_kimi-bf16-ep64share.md"),
    ("bwd_wgate_up", "kimi-bf16-ep64share"): (
        2558.1e6, ('backward.hip', 'batched.hip', 'gemm_large.hip', 'common.h', 'tiles.h', 'internal.h'), "2bf00baff9e035ff",
        "profiles/bwd_kimi-bf16-ep64share.md"),
    ("bwd_requant", "dsv4-mxfp8-T2048"): (
        59007.7e6, ('backward.hip', 'batched.hip', 'gemm_large.hip', 'common.h', 'tiles.h', 'internal.h'), "2bf00baff9e035ff",
        "profiles/bwd_mxfp8_dsv4-mxfp8-T2048.md"),
    ("bwd_wgate_up", "dsv4-mxfp8-T2048"): (
        56072.7e6, ('backward.hip', 'batched.hip', 'gemm_large.hip', 'common.h', 'tiles.h', 'internal.h'), "2bf00baff9e035ff",
        "profiles/bwd_mxfp8_dsv4-mxfp8-T2048.md"),
    ("bwd_wgate_up", "dsv4-mxfp8-ep64share"): (
        4018.3e6, ('backward.hip', 'batched.hip', 'gemm_large.hip', 'common.h', 'tiles.h', 'internal.h'), "2bf00baff9e035ff",
        "profiles/bwd_mxfp8_dsv4-mxfp8-ep64share.md"),
}


def source_fingerprint(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, workload):
    rec = TRAFFIC.get((kernel, workload))
    if rec is None:
        return None, None
    nbytes, files, fp, prof = rec
    if source_fingerprint(files) != fp:
        return None, None
    return nbytes, prof
HBM_PEAK_GBS = 8000.0
DECODE_FUSED = [False]      # --decode-fused: the single-launch decode at T <= 16
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0}   # dense, MI355X


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=None,
                   help="one workload (default: kimi-bf16-T2048 with the other shapes "
                        "reported under 'lines')")
    p.add_argument("--lines", default=None,
                   help="comma-separated workloads reported beside the headline in the same "
                        "JSON line ('none' for none; default: the pages' other shapes when the "
                        "headline is the default workload)")
    p.add_argument("--layers", type=int, default=8, help="independent weight sets to cycle")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time for the oracle baseline (0 = skip)")
    p.add_argument("--pass", dest="pass_", choices=("forward", "backward", "train"),
                   default="forward",
                   help="backward: the layer's backward pass; train: forward + backward "
                        "(batched BF16 workloads)")
    p.add_argument("--recompute", action="store_true",
                   help="backward recomputes the gate/up pre-activations instead of reading "
                        "those the training forward kept")
    p.add_argument("--decode-fused", action="store_true",
                   help="decode at T <= 16 as one launch (routing, gate_up, device-wide wait, "
                        "down) instead of two")
    p.add_argument("--calibrate-fill-mib", type=int, default=0,
                   help="only time a plain device fill of this many MiB (HBM write rate)")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB three times (the "
                        "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    a = p.parse_args()
    if a.lines is None:
        a.lines = DEFAULT_LINES if (a.workload is None and a.pass_ == "forward") else "none"
    if a.workload is None:
        a.workload = "kimi-bf16-T2048"
    return a


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def decode_algorithmic_bytes(cfg, U):
    """HBM bytes the decode kernels must move at least, given U touched experts."""
    T, H, I, k = cfg.T, cfg.H, cfg.I, cfg.k
    gate_up = U * 2 * I * H * 2 + T * H * 2 + T * k * I * 4          # weights, x, h hand-off
    down = U * H * I * 2 + T * k * I * 4 + T * H * 2                  # weights, h, out
    route = T * cfg.E * 4 + T * k * 8
    return {"gate_up": gate_up, "down": down, "route": route}


def launch_percentiles(durs_ms):
    """p10 / median / p90 of per-launch durations, in microseconds."""
    v = sorted(1e3 * d for d in durs_ms)
    q = lambda f: v[min(len(v) - 1, int(f * (len(v) - 1) + 0.5))]
    return {"p10": round(q(0.1), 2), "median": round(q(0.5), 2), "p90": round(q(0.9), 2)}


def decode_weight_sets(W, cfg, layers, seed, dev="cuda"):
    log(f"generating {layers} weight sets of {cfg.name} ({layers * W.expert_bytes(cfg) * cfg.E / 1e9:.1f} GB)")
    return [W.make_weights(cfg, seed=seed + 1000 * l, device=dev) for l in range(layers)]


def run_decode(M, W, torch, cfg, steps, warmup, layers, seed, hook_kernel="auto",
               weights=None, use_graph=True):
    from mixture_experts_ffn_07_amd.hip_events import HipEvent
    dev = "cuda"
    n_batches = steps + warmup
    if weights is None:
        weights = decode_weight_sets(W, cfg, layers, seed, dev)
    layers = len(weights)
    acts = [W.make_activations(cfg, seed=seed + 7919 * (b + 1), device=dev) for b in range(n_batches)]
    T, k = cfg.T, cfg.k
    out = torch.empty(T, cfg.H, dtype=torch.bfloat16, device=dev)
    idx = torch.empty(n_batches, T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(n_batches, T, k, dtype=torch.float32, device=dev)
    ws = M.workspace(M.moe_decode_workspace_bytes(T, cfg.H, cfg.I, cfg.E, k), dev)
    stream = torch.cuda.current_stream()

    def step(i):
        wl = weights[i % layers]
        a = acts[i]
        M.moe_decode_forward(a["x"], a["logits"], wl["w_gate_up"], wl["w_down"], k, out=out,
                             topk_idx=idx[i], topk_w=wts[i], ws=ws, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(HipEvent(), HipEvent()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if hook_kernel == "auto":
        hook_kernel = "decode_fused" if (T <= 16 and DECODE_FUSED[0]) else "decode_gate_up"
    for s in range(steps):
        M.moe_profile_kernel(hook_kernel, evs[s][0].handle, evs[s][1].handle)
        step(warmup + s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    M.moe_profile_kernel("none", None, None)
    durs = [a.elapsed_ms(b) for a, b in evs]
    U = [int(torch.unique(idx[warmup + s]).numel()) for s in range(steps)]
    bytes_ = [decode_algorithmic_bytes(cfg, u) for u in U]
    graph = graph_decode(M, torch, cfg, weights, acts, steps, ws) if use_graph else None
    if hook_kernel == "decode_fused":                 # one launch: the whole layer
        kern_bytes = sum(sum(b.values()) for b in bytes_)
    else:
        kern_bytes = sum(b["gate_up"] for b in bytes_)
    layer_bytes = sum(sum(b.values()) for b in bytes_)
    elapsed = t1 - t0
    res = {
        "elapsed_s": elapsed,
        "ms_per_step": 1e3 * elapsed / steps,
        "tokens_per_s": T * steps / elapsed,
        "kernel_avg_us": 1e3 * sum(durs) / steps,
        "kernel_pct_us": launch_percentiles(durs),
        "kernel_gbs": kern_bytes / (sum(durs) * 1e-3) / 1e9,
        "kernel_bytes_per_launch": kern_bytes / steps,
        "layer_gbs": layer_bytes / elapsed / 1e9,
        "kernel": hook_kernel,
        "avg_touched_experts": sum(U) / steps,
        "first_batch": acts[warmup], "first_weights": weights[warmup % layers],
    }
    if graph is not None:
        # the line's throughput: the same steps replayed from a HIP graph (one host
        # call per captured cycle), the eager figures kept beside it
        res["eager"] = {"ms_per_step": round(res["ms_per_step"], 5),
                        "tokens_per_s": round(res["tokens_per_s"], 1),
                        "layer_gbs": round(layer_bytes / elapsed / 1e9, 1)}
        res["ms_per_step"] = graph["ms_per_step"]
        res["tokens_per_s"] = graph["tokens_per_s"]
        res["layer_gbs"] = graph["layer_bytes_per_step"] / (graph["ms_per_step"] * 1e-3) / 1e9
        res["graph"] = {k_: graph[k_] for k_ in ("captured_steps", "replays", "steps")}
    return res


def graph_decode(M, torch, cfg, weights, acts, steps, ws):
    """Decode steps replayed from a HIP graph: G consecutive steps (each with its
    own activation batch, weight sets cycling as in the eager loop) are captured
    once on a side stream, then the graph is replayed until at least `steps`
    steps have run.  A serving loop issues decode this way: the host's per-call
    work (argument checks, launches) leaves the critical path."""
    T, k = cfg.T, cfg.k
    G = min(len(acts), max(len(weights), 8))
    out = torch.empty(G, T, cfg.H, dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(G, T, k, dtype=torch.int32, device="cuda")
    wts = torch.empty(G, T, k, dtype=torch.float32, device="cuda")

    def step(j, stream):
        wl = weights[j % len(weights)]
        a = acts[j]
        M.moe_decode_forward(a["x"], a["logits"], wl["w_gate_up"], wl["w_down"], k, out=out[j],
                             topk_idx=idx[j], topk_w=wts[j], ws=ws, stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for j in range(G):
            step(j, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream()
        for j in range(G):
            step(j, cs)
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-steps // G))
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    U = [int(torch.unique(idx[j]).numel()) for j in range(G)]
    lb = sum(sum(decode_algorithmic_bytes(cfg, u).values()) for u in U) / G
    n = reps * G
    return {"captured_steps": G, "replays": reps, "steps": n,
            "ms_per_step": 1e3 * (t1 - t0) / n, "tokens_per_s": T * n / (t1 - t0),
            "layer_bytes_per_step": lb}


def batched_algorithmic(cfg, U):
    """HBM bytes and MFMA flops the batched kernels must at least move / do."""
    T, H, I, k = cfg.T, cfg.H, cfg.I, cfg.k
    P = T * k
    eb = 1 if cfg.dtype == "mxfp8" else 2            # bytes per weight / activation code
    sb = (1.0 / 32) if cfg.dtype == "mxfp8" else 0.0  # scale bytes per element
    gate_up = U * 2 * I * H * (eb + sb) + T * H * (eb + sb) + P * I * (eb + sb)
    down = U * H * I * (eb + sb) + P * I * (eb + sb)
    down += (T * H * 2) if k == 1 else (P * H * 4 * 2 + T * H * 2)   # y round trip + out
    return {"gate_up": gate_up, "down": down,
            "flops_gate_up": 2.0 * P * 2 * I * H, "flops_down": 2.0 * P * H * I}


def run_batched(M, W, torch, cfg, steps, warmup, seed, n_batches=4, layers=1):
    """Steps cycle through `layers` weight sets when they fit in 16 GB (decode-sized
    layers: each step then streams weights the last-level cache does not hold)."""
    from mixture_experts_ffn_07_amd.hip_events import HipEvent
    dev = "cuda"
    gb = W.expert_bytes(cfg) * cfg.E / 1e9
    n_sets = layers if gb * layers <= 16.0 else 1
    log(f"generating {n_sets} weight set(s) of {cfg.name} ({gb:.1f} GB each)")
    sets = [W.make_weights(cfg, seed=seed + 1000003 * l, device=dev) for l in range(n_sets)]
    wts = sets[0]
    acts = [W.make_activations(cfg, seed=seed + 7919 * (b + 1), device=dev) for b in range(n_batches)]
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    dt = M.MOE_MXFP8 if cfg.dtype == "mxfp8" else M.MOE_BF16
    stream = torch.cuda.current_stream()
    ws = M.workspace(M.moe_workspace_bytes(T, H, I, E, k, dt), dev)
    idx = torch.empty(n_batches, T, k, dtype=torch.int32, device=dev)
    tw = torch.empty(n_batches, T, k, dtype=torch.float32, device=dev)
    hdt = torch.uint8 if dt == M.MOE_MXFP8 else torch.bfloat16
    h = torch.empty(T * k, I, dtype=hdt, device=dev)
    hs = torch.empty(T * k, I // 32, dtype=torch.uint8, device=dev) if dt == M.MOE_MXFP8 else None
    xc = torch.empty(T, H, dtype=torch.uint8, device=dev) if dt == M.MOE_MXFP8 else None
    xs = torch.empty(T, H // 32, dtype=torch.uint8, device=dev) if dt == M.MOE_MXFP8 else None
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)

    def step(i):
        b = i % n_batches
        a = acts[b]
        wts = sets[i % n_sets]
        M.moe_route_topk(a["logits"], k, topk_idx=idx[b], topk_w=tw[b], stream=stream)
        if dt == M.MOE_MXFP8:
            M.moe_quantize_mxfp8(a["x"], codes=xc, scales=xs, stream=stream)
            M.moe_gate_up_3d_batched(xc, wts["w_gate_up"], idx[b], k, dt, x_scales=xs,
                                     w_gate_up_scales=wts["w_gate_up_scales"], h=h, h_scales=hs,
                                     ws=ws, stream=stream)
            M.moe_down_3d_batched(h, wts["w_down"], idx[b], tw[b], ws, k, dt, h_scales=hs,
                                  w_down_scales=wts["w_down_scales"], out=out, stream=stream)
        else:
            M.moe_gate_up_3d_batched(a["x"], wts["w_gate_up"], idx[b], k, dt, h=h, ws=ws,
                                     stream=stream)
            M.moe_down_3d_batched(h, wts["w_down"], idx[b], tw[b], ws, k, dt, out=out,
                                  stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(HipEvent(), HipEvent()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        M.moe_profile_kernel("gemm_gate_up", evs[s][0].handle, evs[s][1].handle)
        step(warmup + s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    M.moe_profile_kernel("none", None, None)
    durs = [a.elapsed_ms(b) for a, b in evs]
    U = [int(torch.unique(idx[(warmup + s) % n_batches]).numel()) for s in range(steps)]
    alg = [batched_algorithmic(cfg, u) for u in U]
    elapsed = t1 - t0
    kern_s = sum(durs) * 1e-3
    return {
        "elapsed_s": elapsed, "ms_per_step": 1e3 * elapsed / steps,
        "tokens_per_s": T * steps / elapsed,
        "kernel_avg_us": 1e3 * sum(durs) / steps,
        "kernel_pct_us": launch_percentiles(durs),
        "kernel_gbs": sum(a["gate_up"] for a in alg) / kern_s / 1e9,
        "kernel_tflops": sum(a["flops_gate_up"] for a in alg) / kern_s / 1e12,
        "kernel_bytes_per_launch": sum(a["gate_up"] for a in alg) / steps,
        "kernel_flops_per_launch": sum(a["flops_gate_up"] for a in alg) / steps,
        "layer_gbs": sum(a["gate_up"] + a["down"] for a in alg) / elapsed / 1e9,
        "layer_tflops": sum(a["flops_gate_up"] + a["flops_down"] for a in alg) / elapsed / 1e12,
        "avg_touched_experts": sum(U) / steps, "weight_sets": n_sets,
        "first_batch": acts[warmup % n_batches], "first_weights": wts,
    }


BWD_KERNELS = ("bwd_gate_up", "bwd_down", "bwd_input", "bwd_wdown", "bwd_wgate_up")


def backward_algorithmic(cfg, U):
    """Bytes each backward kernel must at least move, and its MFMA flops."""
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    P = T * k
    wgu, wd = U * 2 * I * H * 2, U * H * I * 2
    slots = (P * H * 4 * 2 + T * H * 2) if k > 1 else T * H * 2
    return {
        "bwd_gate_up": (wgu + T * H * 2 + P * 2 * I * 4, 2.0 * P * 2 * I * H),
        # reads W_down, dout, [g; u]; writes [dg; du] and w * a (both BF16)
        "bwd_down": (wd + T * H * 2 + P * 2 * I * 4 + P * 2 * I * 2 + P * I * 2, 2.0 * P * H * I),
        "bwd_input": (wgu + P * 2 * I * 2 + slots, 2.0 * P * 2 * I * H),
        "bwd_wdown": (T * H * 2 + P * I * 2 + E * H * I * 2, 2.0 * P * H * I),
        "bwd_wgate_up": (P * 2 * I * 2 + T * H * 2 + E * 2 * I * H * 2, 2.0 * P * 2 * I * H),
    }


MX_BWD_KERNELS = ("bwd_requant", "bwd_gate_up", "bwd_down", "bwd_input", "bwd_wgate_up")


def mx_backward_algorithmic(cfg, U):
    """The MXFP8 backward's timed segments: bytes they must at least move and their
    MFMA flops.  bwd_requant encodes x and dout along H and the touched experts'
    weights along their output axes; bwd_down is the dh product with its SwiGLU
    finish; bwd_wgate_up covers the pair-axis encodings and both weight gradients."""
    T, H, I, k = cfg.T, cfg.H, cfg.I, cfg.k
    P = T * k
    q = 1.0 + 1.0 / 32                                   # an MX code and its share of a scale
    w_mx = U * 3 * I * H * q                             # both weights, MX
    return {
        "bwd_requant": (2 * T * H * 2 + 2 * T * H * q + 2 * w_mx, 0.0),
        "bwd_gate_up": (U * 2 * I * H * q + T * H * q + P * 2 * I * 4, 2.0 * P * 2 * I * H),
        "bwd_down": (U * H * I * q + T * H * q + P * 2 * I * 4 + P * I * 4 + P * 2 * I * (4 + q),
                     2.0 * P * H * I),
        "bwd_input": (U * 2 * I * H * q + P * 2 * I * q
                      + ((P * H * 4 * 2 + T * H * 2) if k > 1 else T * H * 2), 2.0 * P * 2 * I * H),
        "bwd_wgate_up": (2 * T * H * 2 + P * 3 * I * 4 + U * 3 * I * H * 2,
                         2.0 * P * H * I + 2.0 * P * 2 * I * H),
    }


def backward_roofline(cfg, r):
    """Roofline of the backward's longest timed segment: MFMA-bound where each
    expert's weights meet >= 256 routed rows, HBM-bound otherwise."""
    name, k = max(r["per_kernel"].items(), key=lambda kv: kv[1]["avg_us"])
    traffic, tprof = traffic_for(name, cfg.name)
    peak = MFMA_PEAK_TFLOPS[cfg.dtype]
    if cfg.T * cfg.k / cfg.E >= 256 and k["flops_per_launch"] > 0:   # MFMA-bound reuse
        roof = {"bound": "mfma", "kernel": name, "achieved": round(k["tflops"], 1),
                "peak": peak, "unit": "TFLOP/s",
                "frac": round(k["tflops"] / peak, 4),
                "traffic": traffic, "traffic_unit": "bytes per launch", "traffic_source": tprof,
                "avg_launch_us": round(k["avg_us"], 2),
                "algorithmic_flops_per_launch": int(k["flops_per_launch"])}
    else:
        roof = {"bound": "hbm", "kernel": name, "achieved": round(k["gbs"], 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(k["gbs"] / HBM_PEAK_GBS, 4),
                "traffic": traffic, "traffic_unit": "bytes per launch", "traffic_source": tprof,
                "avg_launch_us": round(k["avg_us"], 2),
                "algorithmic_bytes_per_launch": int(k["bytes_per_launch"])}
    return roof


def run_backward(M, W, torch, cfg, steps, warmup, seed, n_batches=2, recompute=False,
                 train=False):
    """One step = routing + the backward pass of one batch (train: routing, the
    training forward, then the backward).  Without recompute the backward reads
    the gate/up pre-activations that moe_gate_up_3d_batched_train kept (made
    before the timed region for the backward-only step).  The timed steps
    bracket the step's kernels in turn with HIP events."""
    from mixture_experts_ffn_07_amd.hip_events import HipEvent
    dev = "cuda"
    log(f"generating weights of {cfg.name} ({W.expert_bytes(cfg) * cfg.E / 1e9:.1f} GB)")
    wts = W.make_weights(cfg, seed=seed, device=dev)
    acts = [W.make_activations(cfg, seed=seed + 7919 * (b + 1), device=dev) for b in range(n_batches)]
    douts = [W.make_output_grad(cfg, seed=seed + 104729 * (b + 1), device=dev)
             for b in range(n_batches)]
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    stream = torch.cuda.current_stream()
    mx = cfg.dtype == "mxfp8"
    if mx:
        return run_backward_mx(M, torch, cfg, steps, warmup, wts, acts, douts, train)
    ws = M.workspace(M.moe_backward_workspace_bytes(T, H, I, E, k), dev)
    idx = torch.empty(n_batches, T, k, dtype=torch.int32, device=dev)
    tw = torch.empty(n_batches, T, k, dtype=torch.float32, device=dev)
    dx = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    dwgu = torch.empty(E, 2 * I, H, dtype=torch.bfloat16, device=dev)
    dwd = torch.empty(E, H, I, dtype=torch.bfloat16, device=dev)
    dtw = torch.empty(T, k, dtype=torch.float32, device=dev)
    dl = torch.empty(T, E, dtype=torch.float32, device=dev)
    fws = M.workspace(M.moe_workspace_bytes(T, H, I, E, k, M.MOE_BF16), dev)
    h = torch.empty(T * k, I, dtype=torch.bfloat16, device=dev)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    gus = [None] * n_batches
    if not recompute:
        for b in range(n_batches):
            gus[b] = torch.empty(T * k, 2 * I, dtype=torch.float32, device=dev)
            M.moe_route_topk(acts[b]["logits"], k, topk_idx=idx[b], topk_w=tw[b], stream=stream)
            M.moe_gate_up_3d_batched_train(acts[b]["x"], wts["w_gate_up"], idx[b], k, h=h,
                                           gu=gus[b], ws=fws, stream=stream)

    def step(i):
        b = i % n_batches
        a = acts[b]
        M.moe_route_topk(a["logits"], k, topk_idx=idx[b], topk_w=tw[b], stream=stream)
        if train:
            M.moe_gate_up_3d_batched_train(a["x"], wts["w_gate_up"], idx[b], k, h=h, gu=gus[b],
                                           ws=fws, stream=stream)
            M.moe_down_3d_batched(h, wts["w_down"], idx[b], tw[b], fws, k, out=out, stream=stream)
        M.moe_backward_batched(a["x"], wts["w_gate_up"], wts["w_down"], idx[b], tw[b], douts[b],
                               k, gu_saved=gus[b], dx=dx, dw_gate_up=dwgu, dw_down=dwd,
                               d_topk_w=dtw, dlogits=dl, ws=ws, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(HipEvent(), HipEvent()) for _ in range(steps)]
    torch.cuda.synchronize()
    kernels = [n for n in BWD_KERNELS if recompute or n != "bwd_gate_up"]
    if train:
        kernels = ["gemm_gate_up", "gemm_down"] + kernels
    t0 = time.perf_counter()
    for s in range(steps):
        M.moe_profile_kernel(kernels[s % len(kernels)], evs[s][0].handle, evs[s][1].handle)
        step(warmup + s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    M.moe_profile_kernel("none", None, None)
    U = [int(torch.unique(idx[(warmup + s) % n_batches]).numel()) for s in range(steps)]

    def alg(u):
        d = dict(backward_algorithmic(cfg, u))
        if not recompute:
            del d["bwd_gate_up"]
        if train:
            f = batched_algorithmic(cfg, u)
            d["gemm_gate_up"] = (f["gate_up"] + T * k * 2 * I * 4, f["flops_gate_up"])
            d["gemm_down"] = (f["down"], f["flops_down"])
        return d
    per = {}
    for q, name in enumerate(kernels):
        ss = [s for s in range(steps) if s % len(kernels) == q]
        if not ss:
            continue
        dur = sum(evs[s][0].elapsed_ms(evs[s][1]) for s in ss) * 1e-3
        nbytes = sum(alg(U[s])[name][0] for s in ss)
        flops = sum(alg(U[s])[name][1] for s in ss)
        per[name] = {"avg_us": 1e6 * dur / len(ss), "gbs": nbytes / dur / 1e9,
                     "tflops": flops / dur / 1e12, "bytes_per_launch": nbytes / len(ss),
                     "flops_per_launch": flops / len(ss)}
    elapsed = t1 - t0
    tot_bytes = sum(sum(v[0] for v in alg(u).values()) for u in U)
    return {"elapsed_s": elapsed, "ms_per_step": 1e3 * elapsed / steps,
            "tokens_per_s": T * steps / elapsed, "per_kernel": per,
            "layer_gbs": tot_bytes / elapsed / 1e9, "avg_touched_experts": sum(U) / steps}


def run_backward_mx(M, torch, cfg, steps, warmup, wts, acts, douts, train):
    """The MXFP8 backward (moe_backward_batched_mxfp8, which always recomputes the
    pre-activations from the E4M3 weights); train: routing, the MXFP8 forward
    (x quantized, gate_up, down) and the backward.  Segments are timed in turn."""
    from mixture_experts_ffn_07_amd.hip_events import HipEvent
    dev = "cuda"
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    n_batches = len(acts)
    stream = torch.cuda.current_stream()
    ws = M.workspace(M.moe_backward_mxfp8_workspace_bytes(T, H, I, E, k), dev)
    idx = torch.empty(n_batches, T, k, dtype=torch.int32, device=dev)
    tw = torch.empty(n_batches, T, k, dtype=torch.float32, device=dev)
    dx = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    dwgu = torch.empty(E, 2 * I, H, dtype=torch.bfloat16, device=dev)
    dwd = torch.empty(E, H, I, dtype=torch.bfloat16, device=dev)
    dtw = torch.empty(T, k, dtype=torch.float32, device=dev)
    dl = torch.empty(T, E, dtype=torch.float32, device=dev)
    if train:
        fws = M.workspace(M.moe_workspace_bytes(T, H, I, E, k, M.MOE_MXFP8), dev)
        h = torch.empty(T * k, I, dtype=torch.uint8, device=dev)
        hs = torch.empty(T * k, I // 32, dtype=torch.uint8, device=dev)
        xc = torch.empty(T, H, dtype=torch.uint8, device=dev)
        xs = torch.empty(T, H // 32, dtype=torch.uint8, device=dev)
        out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)

    def step(i):
        b = i % n_batches
        a = acts[b]
        M.moe_route_topk(a["logits"], k, topk_idx=idx[b], topk_w=tw[b], stream=stream)
        if train:
            M.moe_quantize_mxfp8(a["x"], codes=xc, scales=xs, stream=stream)
            M.moe_gate_up_3d_batched(xc, wts["w_gate_up"], idx[b], k, M.MOE_MXFP8, x_scales=xs,
                                     w_gate_up_scales=wts["w_gate_up_scales"], h=h, h_scales=hs,
                                     ws=fws, stream=stream)
            M.moe_down_3d_batched(h, wts["w_down"], idx[b], tw[b], fws, k, M.MOE_MXFP8,
                                  h_scales=hs, w_down_scales=wts["w_down_scales"], out=out,
                                  stream=stream)
        M.moe_backward_batched_mxfp8(a["x"], wts["w_gate_up"], wts["w_gate_up_scales"],
                                     wts["w_down"], wts["w_down_scales"], idx[b], tw[b], douts[b],
                                     k, dx=dx, dw_gate_up=dwgu, dw_down=dwd, d_topk_w=dtw,
                                     dlogits=dl, ws=ws, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(HipEvent(), HipEvent()) for _ in range(steps)]
    torch.cuda.synchronize()
    kernels = list(MX_BWD_KERNELS)
    if train:
        kernels = ["gemm_gate_up", "gemm_down"] + kernels
    t0 = time.perf_counter()
    for s in range(steps):
        M.moe_profile_kernel(kernels[s % len(kernels)], evs[s][0].handle, evs[s][1].handle)
        step(warmup + s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    M.moe_profile_kernel("none", None, None)
    U = [int(torch.unique(idx[(warmup + s) % n_batches]).numel()) for s in range(steps)]

    def alg(u):
        d = dict(mx_backward_algorithmic(cfg, u))
        if train:
            f = batched_algorithmic(cfg, u)
            d["gemm_gate_up"] = (f["gate_up"], f["flops_gate_up"])
            d["gemm_down"] = (f["down"], f["flops_down"])
        return d
    per = {}
    for q, name in enumerate(kernels):
        ss = [s for s in range(steps) if s % len(kernels) == q]
        if not ss:
            continue
        dur = sum(evs[s][0].elapsed_ms(evs[s][1]) for s in ss) * 1e-3
        nbytes = sum(alg(U[s])[name][0] for s in ss)
        flops = sum(alg(U[s])[name][1] for s in ss)
        per[name] = {"avg_us": 1e6 * dur / len(ss), "gbs": nbytes / dur / 1e9,
                     "tflops": flops / dur / 1e12, "bytes_per_launch": nbytes / len(ss),
                     "flops_per_launch": flops / len(ss)}
    elapsed = t1 - t0
    tot_bytes = sum(sum(v[0] for v in alg(u).values()) for u in U)
    return {"elapsed_s": elapsed, "ms_per_step": 1e3 * elapsed / steps,
            "tokens_per_s": T * steps / elapsed, "per_kernel": per,
            "layer_gbs": tot_bytes / elapsed / 1e9, "avg_touched_experts": sum(U) / steps}


def host_info():
    """Cores this process may use, the CPU model and the thread settings the
    oracle's BLAS runs with."""
    cores = len(os.sched_getaffinity(0))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                         "MKL_NUM_THREADS")}
    return cores, model, blas, env


def cpu_baseline(W, cfg, act, weights, seconds, n_tokens=None):
    """Time the FP64 oracle on this host on a bounded sample of the same
    workload: the first n_tokens tokens of one batch (all of it by default),
    with the routed experts' weights copied to host memory first (outside the
    timing).  Passes repeat until `seconds` have gone by."""
    import numpy as np
    from oracle import moe_forward, route
    import torch
    T = cfg.T if n_tokens is None else min(n_tokens, cfg.T)
    x = act["x"][:T].cpu().view(torch.int16).numpy().view(np.uint16)
    logits = act["logits"][:T].cpu().numpy()
    ids = np.unique(route(logits, cfg.k)[0])

    def host(name):
        t = weights[name]
        if t.dtype == torch.bfloat16:
            return {int(e): t[int(e)].cpu().view(torch.int16).numpy().view(np.uint16) for e in ids}
        return {int(e): t[int(e)].cpu().numpy() for e in ids}
    wgu, wd = host("w_gate_up"), host("w_down")
    kw = {}
    if cfg.dtype == "mxfp8":
        sg, sd = host("w_gate_up_scales"), host("w_down_scales")
        kw = dict(w_gate_up_scales=sg.__getitem__, w_down_scales=sd.__getitem__)
    n, t0 = 0, time.perf_counter()
    while True:
        moe_forward(x, logits, wgu.__getitem__, wd.__getitem__, cfg.k, dtype=cfg.dtype, **kw)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    cores, model, blas, env = host_info()
    return {"value": n * T / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "blas_threads": blas, "cpu_model": model, "thread_env": env,
            "sample": f"{n} pass(es) of the FP64 oracle over the first {T} token(s) of one "
                      f"{cfg.T}-token batch of {cfg.name} ({len(ids)} routed experts), weights "
                      f"already in host memory, {el:.1f} s"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported: this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    import mixture_experts_ffn_07_amd as M
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}), flush=True)
        return
    if args.calibrate_fill_mib:
        n = args.calibrate_fill_mib << 20
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst.fill_(1)
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dst.fill_(0)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        print(json.dumps({"fill_bytes": n, "best_gbs": round(n / min(ts) / 1e9, 1),
                          "median_gbs": round(n / sorted(ts)[2] / 1e9, 1)}), flush=True)
        return
    cfg = W.get(args.workload)
    log(f"device {torch.cuda.get_device_name(0)}; workload {cfg.name}")
    if args.decode_fused:
        M.moe_set_debug_options(M.MOE_DEBUG_DECODE_FUSED, 0)
        DECODE_FUSED[0] = True
    if args.pass_ in ("backward", "train"):
        if cfg.path != "batched":
            print(f"--pass {args.pass_} needs a batched workload, not {cfg.name}",
                  file=sys.stderr)
            sys.exit(2)
        recompute = args.recompute or cfg.dtype == "mxfp8"
        r = run_backward(M, W, torch, cfg, args.steps, args.warmup, args.seed,
                         recompute=recompute, train=args.pass_ == "train")
        roof = backward_roofline(cfg, r)
        line = {
            "metric": ("MoE layer backward tokens/s" if args.pass_ == "backward"
                       else "MoE layer forward+backward tokens/s"),
            "value": round(r["tokens_per_s"], 1),
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(r["ms_per_step"], 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None,
            "dtype": ("bf16" if cfg.dtype == "bf16"
                      else "mxfp8 (e4m3 + e8m0) operands, fp32 accumulate, bf16 gradients"),
            "data": "synthetic",
            "config": {"workload": f"{cfg.name} {args.pass_}", "T": cfg.T, "H": cfg.H,
                       "E": cfg.E, "k": cfg.k, "I": cfg.I,
                       "preactivations": "recomputed" if recompute else "kept by the forward",
                       "parallelism": "none (1 GPU)"},
            "roofline": roof,
            "kernels": {n: {"avg_us": round(v["avg_us"], 1), "gbs": round(v["gbs"], 1),
                            "tflops": round(v["tflops"], 1)} for n, v in r["per_kernel"].items()},
            "layer": {"hbm_gbs": round(r["layer_gbs"], 1),
                      "hbm_frac": round(r["layer_gbs"] / HBM_PEAK_GBS, 4),
                      "avg_touched_experts": round(r["avg_touched_experts"], 2),
                      "latency_us": round(1e3 * r["ms_per_step"], 2)},
            "cpu_baseline": None,
        }
        print(json.dumps(line), flush=True)
        return
    if cfg.path == "decode":
        r = run_decode(M, W, torch, cfg, args.steps, args.warmup, args.layers, args.seed)
    else:
        r = run_batched(M, W, torch, cfg, args.steps, args.warmup, args.seed, layers=args.layers)
    roof, layer = forward_roofline(cfg, r)
    line = {
        "metric": METRIC, "value": round(r["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "mxfp8 (e4m3 + e8m0), fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k,
                   "I": cfg.I, "weight_sets": r.get("weight_sets", args.layers),
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "layer": layer,
    }
    if "graph" in r:
        line["issue"] = {"mode": "hip graph replay", **r["graph"], "eager": r["eager"]}
    if cfg.path == "decode" and args.layers > 1:
        # the headline cycles weight sets, so each step streams weights no recent step
        # left in the 256 MB last-level cache; this reruns one weight set back to back
        rw = run_decode(M, W, torch, cfg, min(args.steps, 50), args.warmup, 1, args.seed)
        line["warm"] = {"weight_sets": 1, "steps": min(args.steps, 50),
                        "ms_per_step": round(rw["ms_per_step"], 5),
                        "tokens_per_s": round(rw["tokens_per_s"], 1),
                        "gate_up_gbs": round(rw["kernel_gbs"], 1),
                        "gate_up_launch_us": rw["kernel_pct_us"]}
    if args.cpu_seconds > 0:
        log("timing the CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline(
            W, cfg, r["first_batch"], r["first_weights"], args.cpu_seconds,
            n_tokens=None if cfg.path == "decode" else 2)
    else:
        line["cpu_baseline"] = None
    first_w = r.pop("first_weights")
    del first_w, r
    lines = [] if args.lines in ("", "none") else args.lines.split(",")
    if lines:
        line["lines"] = run_lines(M, W, torch, lines, args)
    print(json.dumps(line), flush=True)


def forward_roofline(cfg, r):
    """The dominant kernel's roofline (decode: decode_gate_up against HBM;
    batched: the gate_up GEMM, against HBM or, at 256+ rows per expert, the
    MFMA peak of its dtype) and the whole layer's figures."""
    peak_tf = MFMA_PEAK_TFLOPS[cfg.dtype]
    if cfg.path == "decode":
        kern = r.get("kernel", "decode_gate_up")   # decode_fused: the single-launch layer
        mfma_bound = False
    else:
        kern = "gemm_gate_up"
        mfma_bound = cfg.T * cfg.k / cfg.E >= 256      # weight reuse high enough
    traffic, tprof = traffic_for(kern, cfg.name)
    common = {"kernel": kern, "traffic": traffic, "traffic_unit": "bytes per launch",
              "traffic_source": tprof, "avg_launch_us": round(r["kernel_avg_us"], 2),
              "launch_us": r["kernel_pct_us"]}
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(r["kernel_tflops"], 1), "peak": peak_tf,
                "unit": "TFLOP/s", "frac": round(r["kernel_tflops"] / peak_tf, 4), **common,
                "algorithmic_flops_per_launch": int(r["kernel_flops_per_launch"]),
                "hbm_gbs": round(r["kernel_gbs"], 1)}
    else:
        roof = {"bound": "hbm", "achieved": round(r["kernel_gbs"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(r["kernel_gbs"] / HBM_PEAK_GBS, 4), **common,
                "algorithmic_bytes_per_launch": int(r["kernel_bytes_per_launch"])}
        if "kernel_tflops" in r:
            roof["mfma_tflops"] = round(r["kernel_tflops"], 1)
            roof["mfma_frac"] = round(r["kernel_tflops"] / peak_tf, 4)
    layer = {"hbm_gbs": round(r["layer_gbs"], 1), "hbm_frac": round(r["layer_gbs"] / HBM_PEAK_GBS, 4),
             "avg_touched_experts": round(r["avg_touched_experts"], 2),
             "latency_us": round(1e3 * r["ms_per_step"], 2)}
    if "layer_tflops" in r:
        layer["mfma_tflops"] = round(r["layer_tflops"], 1)
        layer["mfma_frac"] = round(r["layer_tflops"] / peak_tf, 4)
    return roof, layer


# the pages' other shapes, reported beside the headline in the same JSON line
DEFAULT_LINES = ("dsv4-mxfp8-T2048,kimi-bf16-ep64share,dsv4-mxfp8-ep64share,"
                 "qwen3-decode-T1,qwen3-decode-T8,qwen3-decode-T32,q35-zipf-T64,"
                 "kimi-bf16-T2048:backward,kimi-bf16-ep64share:backward,"
                 "dsv4-mxfp8-T2048:backward,dsv4-mxfp8-ep64share:backward")


def run_lines(M, W, torch, names, args):
    """Each workload in turn (its tensors freed before the next): batched lines
    time `--steps` steps, decode lines max(--steps, 100) steps cycling weight
    sets (8 for the Qwen3-style shape, shared by its three batch sizes; 2 for the
    Qwen3.5-shaped one, 25.8 GB)."""
    out = []
    qwen_sets = None
    for name in names:
        name, _, pass_ = name.partition(":")
        cfg = W.get(name)
        t0 = time.perf_counter()
        if pass_ == "backward":
            r = run_backward(M, W, torch, cfg, args.steps, args.warmup, args.seed,
                             recompute=cfg.dtype == "mxfp8")
            roof = backward_roofline(cfg, r)
            out.append({"workload": name, "pass": "backward", "T": cfg.T, "H": cfg.H, "E": cfg.E,
                        "k": cfg.k, "I": cfg.I, "dtype": cfg.dtype, "steps": args.steps,
                        "preactivations": ("recomputed" if cfg.dtype == "mxfp8"
                                           else "kept by the forward"),
                        "ms_per_step": round(r["ms_per_step"], 5),
                        "tokens_per_s": round(r["tokens_per_s"], 1),
                        "roofline": {k_: roof[k_] for k_ in ("bound", "kernel", "achieved", "peak",
                                                             "unit", "frac", "avg_launch_us",
                                                             "traffic", "traffic_source")},
                        "segments_us": {n: round(v["avg_us"], 1)
                                        for n, v in r["per_kernel"].items()}})
            del r
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            log(f"{name} backward: {out[-1]['ms_per_step']:.4f} ms/step, frac {roof['frac']} "
                f"({time.perf_counter() - t0:.1f} s)")
            continue
        if cfg.path == "decode":
            steps = max(args.steps, 100)
            if name.startswith("qwen3-decode"):
                if qwen_sets is None:
                    qwen_sets = decode_weight_sets(W, cfg, 8, args.seed)
                sets = qwen_sets
            else:
                sets = decode_weight_sets(W, cfg, 2, args.seed)
            r = run_decode(M, W, torch, cfg, steps, args.warmup, len(sets), args.seed,
                           weights=sets)
            del sets
        else:
            steps = args.steps
            r = run_batched(M, W, torch, cfg, steps, args.warmup, args.seed, layers=1)
        r.pop("first_weights", None)
        r.pop("first_batch", None)
        roof, layer = forward_roofline(cfg, r)
        out.append({"workload": name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k, "I": cfg.I,
                    "dtype": cfg.dtype, "steps": steps, "weight_sets": r.get("weight_sets"),
                    "ms_per_step": round(r["ms_per_step"], 5),
                    "tokens_per_s": round(r["tokens_per_s"], 1),
                    "roofline": {k_: roof[k_] for k_ in ("bound", "kernel", "achieved", "peak",
                                                         "unit", "frac", "avg_launch_us",
                                                         "traffic", "traffic_source")},
                    "layer": layer})
        if "graph" in r:
            out[-1]["issue"] = {"mode": "hip graph replay", **r["graph"], "eager": r["eager"]}
        del r
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        log(f"{name}: {out[-1]['ms_per_step']:.4f} ms/step, frac {roof['frac']} "
            f"({time.perf_counter() - t0:.1f} s)")
    return out


if __name__ == "__main__":
    main()
