#!/usr/bin/env python3
"""Benchmark of per-head causal local-window attention on one MI355X.

One step = one pass of the whole path over one batch: window intake and work
lists (cached after the first call), the forward kernel and the two backward
kernels (dQ, which also forms the per-row D = dO . O, then dK/dV), on the
1B-scale layer workload
(B=4, H=32, T=4096, d=64, bf16; 8 groups of 4 heads whose windows are drawn
from {512, 1024, 2048, 4096} with P = (.5, .25, .125, .125); seed 0).

Effective FLOPs count in-window query/key pairs only: 4*d per pair forward
(Q K^T and P V) and 10*d per pair backward (Q K^T, dO V^T, P^T dO, dS K,
dS^T Q); the backward kernels recompute Q K^T and dO V^T once more for dQ, which
is not counted.  Pairs per head = sum_{t=1}^{T} min(t, W_h) (plus, for heads
with sink tokens, the sinks each row sees before its window).

--workload 5 times the same step on the streaming-head layer (heads 0-15 full
causal, heads 16-31 sink 128 + recent window 256; "Autonomy-of-Heads" section
5 and 6.1); --workload 6 on a grouped-query layer (32 query heads over 8
key/value heads, d = 128, per-query-head windows); --workload 6s on that layer
for one sequence, and --workload 5s the streaming-head layer for one sequence,
both of which take the split launches.

Prints ONE JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # After idle the device needs some 60 steps (about 30 ms) of this load before its clock settles; the
    # default warm-up covers that, so the timed steps measure the sustained rate.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="3", help="catalogued workload id (default 3: fwd+bwd 1B-scale layer)")
    ap.add_argument("--no-split", action="store_true",
                    help="pass workspaces too small for the split launches (one workgroup per work item), to time "
                         "what splitting buys on layers with few work items")
    ap.add_argument("--cpu-heads", type=int, default=48, help="heads of the oracle CPU-baseline sample (0 = skip)")
    ap.add_argument("--fwd-only", action="store_true", help="time the forward pass only")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a device-to-device copy of a known size (to scale HBM byte counters)")
    ap.add_argument("--diag", action="store_true",
                    help="time a control-update forward: the forward with per-row entropy and output norm, "
                         "then the per-head features and their EMA (prints its own JSON line)")
    ap.add_argument("--decode", action="store_true",
                    help="time one decoding step over the trimmed per-head caches of the workload's layer "
                         "(a separate measurement; prints its own JSON line)")
    return ap.parse_args()


def quiet_gc():
    """Collect once and move every live object out of the collector's generations.  A full collection over
    torch's heap takes 30-60 ms; left alone, one lands inside the timed steps every few hundred library calls
    (each call makes a few small Python objects) and the device idles while the host is paused."""
    import gc
    gc.collect()
    gc.freeze()


def bench_decode(args, wl):
    """Decoding over per-head trimmed K/V caches: the layer's caches hold positions 0..T-2 (a prefill), and
    every timed step decodes the token at position T-1 (every ring full; repeating the step rewrites the same
    row and reads the same bytes).  Bound: HBM.  Algorithmic bytes per step = the cached K and V rows
    (2 * 2 d bytes each; with grouped key/value heads each row once for its group) + q, k_new, v_new read +
    o written + the new K/V rows written + lse."""
    import torch
    import head_causal_local_amd as aah
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    k, v, q = to_dev(wl, "k"), to_dev(wl, "v"), to_dev(wl, "q")
    H_kv = k.shape[1]
    kc, vc = aah.kv_cache_fill(k[:, :, :T - 1].contiguous(), v[:, :, :T - 1].contiguous(), wl.windows, T,
                               sinks=wl.sinks)
    qt, kt, vt = (x[:, :, T - 1].contiguous() for x in (q, k, v))
    pos = torch.full((B,), T - 1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(aah.decode_workspace_size(wl.windows, B, T, d, sinks=wl.sinks, H_kv=H_kv), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(qt)
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        aah.attn_decode(qt, kt, vt, kc, vc, pos, wl.windows, T, scale=wl.scale, out=o, lse=lse, workspace=ws,
                        stream=stream, sinks=wl.sinks)

    quiet_gc()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # Eager: one library call per step from Python (includes the host's per-call cost).
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eager_us = e0.elapsed_time(e1) * 1e3 / args.steps
    # Graph: the same steps captured once and replayed, as a serving loop would run them; this is
    # the device's time per step.
    g = torch.cuda.CUDAGraph()
    gs = torch.cuda.Stream()
    gs.wait_stream(stream)
    with torch.cuda.stream(gs):
        with torch.cuda.graph(g, stream=gs):
            for _ in range(10):
                aah.attn_decode(qt, kt, vt, kc, vc, pos, wl.windows, T, scale=wl.scale, out=o, lse=lse,
                                workspace=ws, stream=gs, sinks=wl.sinks)
    stream.wait_stream(gs)
    torch.cuda.synchronize()
    reps = max(1, args.steps // 10)
    g.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (10 * reps)
    # Every cached row is read at position T - 1 (rings full, sinks before every window).
    rows = aah.kv_cache_rows(wl.windows, T, sinks=wl.sinks, H_kv=H_kv)
    alg = B * (rows * 2 * 2 * d + H * 2 * d + 2 * H_kv * 2 * d + H * 2 * d + 2 * H_kv * 2 * d + H * 4)
    gbs = alg / (us * 1e-6) / 1e9
    out = {
        "metric": "decode step: algorithmic HBM bytes per step / device time per step (graph replay; "
                  "per-head trimmed K/V caches)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (N(0,1) bf16 Q/K/V, seed 0)",
        "config": {"workload": wl.name + " decode at position T-1", "B": B, "H": H, "H_kv": H_kv, "T_max": T, "d": d,
                   "windows": [int(x) for x in wl.windows],
                   **({"sinks": [int(x) for x in wl.sinks]} if wl.sinks is not None else {}),
                   "cache_rows_per_batch_entry": rows,
                   "step_us": round(us, 3), "eager_step_us": round(eager_us, 3),
                   "tokens_per_s": round(B / (us * 1e-6), 1),
                   "algorithmic_bytes_per_step": int(alg)},
        "roofline": {"kernel": f"decode_kernel<{d}, {'true' if H_kv != H else 'false'}>", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(f"decode_kernel<{d}, {'true' if H_kv != H else 'false'}>", args.workload),
                     "avg_launch_us": round(us, 3),
                     "algorithmic_bytes_per_launch": int(alg)},
    }
    print(json.dumps(out))


def bench_diag(args, wl):
    """Controller diagnostics (AAH section 5.3) on a control-update step: the diagnostic forward (same O and
    LSE as the plain forward, plus per-row entropy and output norm) and the head-features call (Q/K/V
    statistics, means of the rows, EMA).  The features call is HBM-bound: its algorithmic bytes are Q, K, V
    read once, the two row arrays read once, and the features / EMA written."""
    import torch
    import head_causal_local_amd as aah
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    q, k, v = to_dev(wl, "q"), to_dev(wl, "k"), to_dev(wl, "v")
    o = torch.empty_like(q)
    lse, ent, nrm = (torch.empty((B, H, T), dtype=torch.float32, device="cuda") for _ in range(3))
    feats = torch.empty((H, aah.N_FEATURES), dtype=torch.float32, device="cuda")
    ema = torch.zeros_like(feats)
    ws = torch.empty(aah.head_features_workspace_size(B, H, T, d), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        aah.attn_fwd(q, k, v, wl.windows, wl.scale, out=o, lse=lse, stream=stream, sinks=wl.sinks)
        mark(1)
        aah.attn_fwd_diag(q, k, v, wl.windows, wl.scale, out=o, lse=lse, row_entropy=ent, row_onorm=nrm,
                          stream=stream, sinks=wl.sinks)
        mark(2)
        aah.head_features(q, k, v, wl.windows, ent, nrm, features_ema=ema, alpha=0.9, out=feats, workspace=ws,
                          stream=stream)
        mark(3)

    quiet_gc()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def span(a, b):
        return float(np.mean([e[a].elapsed_time(e[b]) for e in events]))

    fwd_ms, diag_ms, feat_ms = span(0, 1), span(1, 2), span(2, 3)
    chunks = -(-(T * d) // 32768)
    alg = 3 * B * H * T * d * 2 + 2 * B * H * T * 4 + 3 * H * 9 * 4 + 2 * 3 * H * B * chunks * 32
    gbs = alg / (feat_ms * 1e-3) / 1e9
    pairs_b, _ = aah.window_stats(wl.windows, T, sinks=wl.sinks)
    out = {
        "metric": "control-update diagnostics: head-features call, algorithmic HBM bytes / time",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (N(0,1) bf16 Q/K/V, seed 0)",
        "config": {"workload": wl.name + " control-update forward + head features", "B": B, "H": H, "T": T, "d": d,
                   "fwd_ms": round(fwd_ms, 4), "fwd_diag_ms": round(diag_ms, 4),
                   "diag_overhead_pct": round(100 * (diag_ms / fwd_ms - 1), 2),
                   "fwd_diag_tflops": round(4 * d * B * pairs_b / (diag_ms * 1e-3) / 1e12, 2),
                   "features_us": round(feat_ms * 1e3, 2), "algorithmic_bytes_features": int(alg)},
        "roofline": {"kernel": "head features (qkv_stats_kernel + features_kernel)", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "avg_launch_us": round(feat_ms * 1e3, 2), "algorithmic_bytes_per_launch": int(alg)},
    }
    print(json.dumps(out), flush=True)


COPY_BYTES = 512 * 1024 * 1024


def calibrate_copy(steps):
    """Kernels of known traffic whose counter readings convert FETCH_SIZE / WRITE_SIZE to bytes: a fill that
    writes COPY_BYTES, a plain copy that reads and writes COPY_BYTES, and a sum that only reads them."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    total = torch.zeros((), dtype=torch.float32, device="cuda")
    for _ in range(steps):
        dst.copy_(src)
    for _ in range(steps):
        total += src.sum()
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device fill, copy and sum", "bytes_read": COPY_BYTES,
                      "bytes_written": COPY_BYTES, "launches": steps}), flush=True)


KERNEL_SOURCES = {  # kernel template name -> its source file
    "fwd_bf16_kernel": "head_causal_local_amd/csrc/fwd_bf16.hip",
    "bwd_dkdv_kernel": "head_causal_local_amd/csrc/bwd_bf16.hip",
    "bwd_dq_kernel": "head_causal_local_amd/csrc/bwd_bf16.hip",
    "decode_kernel": "head_causal_local_amd/csrc/decode.hip",
}
KERNEL_HEADERS = ("head_causal_local_amd/csrc/device_common.hpp", "head_causal_local_amd/csrc/kernels.hpp")


def kernel_source_sha(kernel):
    """First 16 hex digits of the SHA-256 of a kernel's source file followed by the headers it includes (the
    key of its rows in profiles/hbm_traffic.txt), or None for a kernel without a listed source."""
    import hashlib
    src = KERNEL_SOURCES.get(kernel.split("<")[0])
    if src is None:
        return None
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in (src,) + KERNEL_HEADERS:
        h.update(open(os.path.join(root, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from profiles/hbm_traffic.txt, if taken on the current
    kernel source."""
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "hbm_traffic.txt")
    sha = kernel_source_sha(kernel)
    if sha is None or not os.path.exists(path):
        return None
    for line in open(path):
        parts = line.split()
        if line.startswith("#"):
            continue
        # <kernel name (may hold spaces)> <workload> <source sha16> <fetch bytes> <write bytes>
        parts = line.rsplit(None, 4)
        if len(parts) == 5 and parts[0] == kernel and parts[1] == str(workload) and parts[2] == sha:
            return int(parts[3]) + int(parts[4])
    return None


def to_dev(wl, key):
    import torch
    return torch.from_numpy(wl.bits[key].view(np.int16)).view(torch.bfloat16).to("cuda")


def cpu_baseline(wl, n_heads, with_bwd):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = os.cpu_count() or 1
    # Sample: the first n_heads (b, h) pairs of batch entry 0, cycling over distinct windows first.
    order = []
    seen = set()
    for h in range(wl.H):
        if int(wl.windows[h]) not in seen:
            seen.add(int(wl.windows[h]))
            order.append(h)
    order += [h for h in range(wl.H) if h not in order]
    heads = order[:n_heads]
    import head_causal_local_amd as aah
    sinks = None if wl.sinks is None else wl.sinks[heads]
    pairs, _ = aah.window_stats(wl.windows[heads], wl.T, sinks=sinks)
    t0 = time.perf_counter()
    for h in heads:
        sl = (slice(0, 1), slice(h, h + 1))
        g = h // (wl.H // wl.k.shape[1])                     # the query head's key/value head
        kv = (slice(0, 1), slice(g, g + 1))
        sk = None if wl.sinks is None else wl.sinks[h:h + 1]
        oracle.attn_fwd_ref(wl.q[sl], wl.k[kv], wl.v[kv], wl.windows[h:h + 1], wl.scale, sinks=sk)
        if with_bwd:
            oracle.attn_bwd_ref(wl.q[sl], wl.k[kv], wl.v[kv], wl.windows[h:h + 1], wl.scale, wl.do[sl], sinks=sk)
    dt = time.perf_counter() - t0
    flops = (4 + (10 if with_bwd else 0)) * wl.d * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"fp64 oracle {'fwd+bwd' if with_bwd else 'fwd'} of {len(heads)} full heads (b=0, "
                      f"h={heads}) of the same workload, {pairs} in-window pairs, effective FLOPs as on the GPU"}


def main():
    args = parse()
    if args.steps < 1 or args.warmup < 0:
        print(f"--steps must be >= 1 and --warmup >= 0 (got {args.steps}, {args.warmup})", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library runs every head of a layer on a single MI355X "
              "(no sharding or collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import head_causal_local_amd as aah
    import synth

    if not torch.cuda.is_available():
        print("no HIP device visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(max(args.steps, 1))
        return

    wid = int(args.workload) if args.workload.isdigit() else args.workload
    wl = synth.make_workload(wid)
    if wl.dtype != "bf16":
        print("bench.py times bf16 workloads", file=sys.stderr)
        sys.exit(2)
    if args.decode:
        bench_decode(args, wl)
        return
    if args.diag:
        bench_diag(args, wl)
        return
    with_bwd = (wl.do is not None) and not args.fwd_only
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    H_kv = wl.k.shape[1]

    # Two resident copies of every input and output, used by alternate steps: a step never finds the
    # previous step's operands still in the device's last-level cache (the inputs of one step, 0.27-0.54 GB
    # on the 1B-scale layer, are about the size of that cache).
    bwd_split_bytes = (aah.bwd_split_workspace_size(wl.windows, B, H, T, d, sinks=wl.sinks, H_kv=H_kv)
                       if with_bwd and not args.no_split else 0)
    fwd_ws = torch.empty(0, dtype=torch.uint8, device="cuda") if args.no_split else None  # None: the binding sizes it

    def buffers():
        q, k, v = to_dev(wl, "q"), to_dev(wl, "k"), to_dev(wl, "v")
        bufs = {"q": q, "k": k, "v": v, "o": torch.empty_like(q),
                "lse": torch.empty((B, H, T), dtype=torch.float32, device="cuda")}
        if with_bwd:
            # The backward's workspace: the per-row arrays, or, where the library splits the backward's long
            # items (few work items: one sequence, few heads), the larger split workspace.
            ws_bytes = max(aah.workspace_size(B, H, T, d, "bf16"), bwd_split_bytes)
            bufs.update(do=to_dev(wl, "do"), dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                        ws=torch.empty(ws_bytes, dtype=torch.uint8, device="cuda"))
        return bufs

    sets = [buffers(), buffers()]
    stream = torch.cuda.current_stream()
    n_ev = 4 if with_bwd else 2

    def step(i, ev=None):
        def mark(j):
            if ev is not None:
                ev[j].record(stream)
        x = sets[i % 2]
        mark(0)
        aah.attn_fwd(x["q"], x["k"], x["v"], wl.windows, wl.scale, out=x["o"], lse=x["lse"], stream=stream,
                     sinks=wl.sinks, workspace=fwd_ws)
        mark(1)
        if with_bwd:
            aah.attn_bwd_dq(x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], wl.windows, x["dq"], x["ws"], wl.scale,
                            stream=stream, sinks=wl.sinks)
            mark(2)
            aah.attn_bwd_dkdv(x["q"], x["k"], x["v"], x["do"], wl.windows, x["dk"], x["dv"], x["ws"], wl.scale,
                              stream=stream, sinks=wl.sinks)
            mark(3)

    quiet_gc()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def span(a, b):
        return np.array([e[a].elapsed_time(e[b]) for e in events])

    fwd_ms = span(0, 1)
    dq_ms = span(1, 2) if with_bwd else np.zeros(1)
    dkdv_ms = span(2, 3) if with_bwd else np.zeros(1)
    bwd_ms = span(1, 3) if with_bwd else np.zeros(1)
    step_dev_ms = span(0, n_ev - 1)  # device time of each step, first launch to last
    ms_per_step = wall * 1e3 / args.steps

    pairs_b, acr = aah.window_stats(wl.windows, T, sinks=wl.sinks)
    pairs = B * pairs_b
    f_fwd = 4 * d * pairs
    f_bwd = 10 * d * pairs if with_bwd else 0
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12
    fwd_tf = f_fwd / (fwd_ms.mean() * 1e-3) / 1e12
    bwd_tf = f_bwd / (bwd_ms.mean() * 1e-3) / 1e12 if with_bwd else None

    # Roofline of the kernel that dominates the step (each step is one launch on `stream`).
    # Algorithmic FLOPs per in-window pair: forward 4 d (Q K^T, P V); dK/dV kernel 8 d
    # (Q K^T, dO V^T, dO^T P, Q^T dS); dQ kernel 2 d (K^T dS^T) -- it also recomputes
    # K Q^T and V dO^T (4 d more MFMA work), which the backward's 10 d does not count.
    # Instantiations the library launches: <d, sinks, diagnostics> forward, <d, sinks> dQ,
    # <d, sinks, grouped heads> dK/dV.
    sink = "true" if wl.sinks is not None and int(np.max(wl.sinks)) > 0 else "false"
    gqa = "true" if H_kv != H else "false"
    fname = f"fwd_bf16_kernel<{d}, {sink}, false>"
    if not args.no_split and aah.fwd_workspace_size(wl.windows, B, H, T, d, sinks=wl.sinks, H_kv=H_kv) > 0:
        fname += f" + fwd_merge_kernel<{d}>"  # split launch: the forward's events hold both kernels
    kernels = [(fname, float(fwd_ms.mean()), f_fwd)]
    if with_bwd:
        # With a split workspace, a backward kernel the library splits is followed by its merge launch, which
        # that kernel's events then also hold.
        merge = " (+ bwd_merge_kernel where split)" if bwd_split_bytes > 0 else ""
        kernels += [(f"bwd_dkdv_kernel<{d}, {sink}, {gqa}>{merge}", float(dkdv_ms.mean()), 8 * d * pairs),
                    (f"bwd_dq_kernel<{d}, {sink}>{merge}", float(dq_ms.mean()), 2 * d * pairs)]
    kname, kms, kflops = max(kernels, key=lambda x: x[1])
    achieved = kflops / (kms * 1e-3) / 1e12
    roof = {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(kname, args.workload),
            "avg_launch_us": round(kms * 1e3, 2), "algorithmic_flops_per_launch": int(kflops)}

    out = {
        "metric": "effective TFLOP/s (in-window pairs only) fwd/bwd, % of bf16 MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (N(0,1) bf16 Q/K/V/dO, seed 0)",
        "config": {
            "workload": wl.name + (" fwd+bwd" if with_bwd else " fwd"),
            "B": B, "H": H, "H_kv": H_kv, "T": T, "d": d,
            "windows": [int(x) for x in wl.windows],
            **({"sinks": [int(x) for x in wl.sinks]} if wl.sinks is not None else {}),
            "in_window_pairs": int(pairs),
            "acr": round(acr, 4),
            "fwd_ms": round(float(fwd_ms.mean()), 4),
            "bwd_ms": round(float(bwd_ms.mean()), 4) if with_bwd else None,
            "bwd_dkdv_ms": round(float(dkdv_ms.mean()), 4) if with_bwd else None,
            "bwd_dq_ms": round(float(dq_ms.mean()), 4) if with_bwd else None,
            "fwd_tflops": round(fwd_tf, 2),
            "bwd_tflops": round(bwd_tf, 2) if with_bwd else None,
            "fwd_pct_bf16_peak": round(100 * fwd_tf / PEAK_BF16_TFLOPS, 2),
            "bwd_pct_bf16_peak": round(100 * bwd_tf / PEAK_BF16_TFLOPS, 2) if with_bwd else None,
            "step_pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
            "step_device_ms_p10_median_p90": [round(float(np.percentile(step_dev_ms, p)), 4) for p in (10, 50, 90)],
            "bwd_split_workspace": bool(bwd_split_bytes > 0),
            "split_launches": not args.no_split,
        },
        "roofline": roof,
    }
    if args.cpu_heads > 0:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_heads, with_bwd)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
