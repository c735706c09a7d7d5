#!/usr/bin/env python3
"""Throughput of the fused, chunked XMC classifier-head training step on one MI355X.

A step is one pass of the whole training hot path over one synthetic batch: label bucketing, the
forward contraction with the sigmoid-BCE gradient epilogue, the input gradient with the pre-update
weights, and the weight gradient fused into SGD with stochastic rounding, chunk by chunk, then the
dX reduction. The default workload is the 3M-label E4M3 head (B=256, D=768, L=3,000,000,
chunk 131,072, lr 0.1), with inputs resident in HBM before timing. The top-k scoring pass is timed
separately (its own object in the JSON line) because the metric is the training step.

Prints one JSON line: samples/s (value), TFLOP/s, MFMA-roofline fraction, HBM use, the dominant
kernel's roofline from live HIP-event timing, and the CPU oracle timed on a bounded sample. The
timed steps carry no event between kernels; the per-kernel averages come from a second pass of the
same number of steps with HIP events around every forward and backward launch (its own ms/step is
reported beside them, since the events add a few microseconds between the kernels they bracket,
with the median of its per-step times). The first warm-up step, with cold caches, is timed on its
own (`first_step_ms`).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "classifier train-step samples/sec + TFLOP/s (% MFMA peak), L=3M D=768 FP8"
PEAK = {"bf16": 2.5e15, "fp8": 5.0e15, "hbm": 8.0e12}   # MI355X dense MFMA and HBM3E peaks


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="e4m3_3m",
                    help="one of tiny, bf16_131k, bf16_670k, e4m3_3m, bf16_8p6m")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-topk", action="store_true")
    ap.add_argument("--topk-n", type=int, default=4096)
    ap.add_argument("--no-kahan", action="store_true")
    ap.add_argument("--kahan-params", type=int, default=110_000_000,
                    help="encoder parameters of the Kahan-compensated BF16 update pass (768-wide, 12 layers)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (3 times) and exit: the "
                         "known-size reference for scaling HBM byte counters")
    return ap.parse_args()


def kahan_bench(n, stream):
    """Kahan-compensated BF16 update of n encoder parameters (BF16 w and c, FP32 g), a separate
    elementwise pass bound by HBM: 12 algorithmic bytes per parameter (w, c, g read; w, c written),
    timed over 10 updates with events on the launch stream."""
    import torch

    import precision_label_chunk_amd as elmo
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    w = (torch.randn(n, device=dev, generator=gen) * 0.02).to(torch.bfloat16).view(torch.int16)
    c = torch.zeros(n, dtype=torch.int16, device=dev)
    g = torch.randn(n, device=dev, generator=gen)
    for _ in range(2):
        elmo.kahan_update(w, c, g, 1e-3)
    torch.cuda.synchronize()
    reps = 10
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        elmo.kahan_update(w, c, g, 1e-3)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 12.0 * n / (ms / 1e3) / 1e9
    del w, c, g
    return {"params": n, "ms": round(ms, 4), "alg_gbs": round(gbs, 1), "peak_gbs": PEAK["hbm"] / 1e9,
            "frac": round(gbs * 1e9 / PEAK["hbm"], 4)}


def kernel_source_hash():
    """SHA-256 over the library's kernel sources: byte counters taken on other sources are stale."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "precision_label_chunk_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` (read + write) from the committed counter summary of this
    workload, or None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    fetch = write = None
    sha = None
    with open(path) as fh:
        for line in fh:
            t = line.split()
            if not t or t[0].startswith("#"):
                continue
            if t[0] == "source_sha256":
                sha = t[1]
            elif t[0].startswith(kernel + "<") and "bytes" in t:
                v = float(t[t.index("bytes") + 1])
                if t[1] == "fetch_size_kib":
                    fetch = v
                elif t[1] == "write_size_kib":
                    write = v
    if sha != kernel_source_hash() or fetch is None or write is None:
        return None
    return {"bytes": fetch + write, "read": fetch, "write": write}


def copy_reference(nbytes):
    """A plain copy of `nbytes` bytes, three times: each launch reads and writes exactly nbytes."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 3}), flush=True)


def cpu_baseline(wl, W_dev, batch, target_s):
    """The oracle as it stands, on the first L' labels of the same weights and batch (all B samples,
    all D features), L' sized for about `target_s` seconds; scaled to samples/s over all L labels."""
    import numpy as np

    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()

    def run(Ls):
        W = W_dev[:Ls].cpu().numpy()
        W = W.view(np.uint16) if W.dtype == np.int16 else W
        keep = batch.ids < Ls
        rows = [keep[batch.row_ptr[b]:batch.row_ptr[b + 1]].sum() for b in range(wl.B)]
        rp = np.zeros(wl.B + 1, np.int32); rp[1:] = np.cumsum(rows)
        t0 = time.perf_counter()
        oracle.step(wl.wfmt, W, batch.X, rp, batch.ids[keep], wl.lr, wl.seed, 0, nthreads=threads)
        return time.perf_counter() - t0

    Ls = min(wl.L, 512)
    t = run(Ls)
    Ls2 = int(min(wl.L, max(Ls, Ls * target_s / max(t, 1e-3))))
    if Ls2 > Ls:
        Ls, t = Ls2, run(Ls2)
    per_label = t / Ls
    return {"value": wl.B / (per_label * wl.L), "unit": "samples/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle step over the first {Ls} of {wl.L} labels (B={wl.B}, D={wl.D}, same weights "
                      f"and batch) took {t:.2f} s; scaled linearly to all labels",
            "seconds": round(t, 3), "labels": Ls}


def cpu_topk_baseline(wl, W_dev, Xe, k, target_s, nq=256):
    """The oracle's top-k of nq of the same held-out queries over the first L' labels of the same
    weights, L' sized for about `target_s` seconds; scaled to queries/s over all L labels."""
    import numpy as np

    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    Xs = np.ascontiguousarray(Xe[:nq])

    def run(Ls):
        W = W_dev[:Ls].cpu().numpy()
        W = W.view(np.uint16) if W.dtype == np.int16 else W
        t0 = time.perf_counter()
        oracle.topk(wl.wfmt, W, Xs, min(k, Ls), nthreads=threads)
        return time.perf_counter() - t0

    Ls = min(wl.L, 4096)
    t = run(Ls)
    Ls2 = int(min(wl.L, max(Ls, Ls * target_s / max(t, 1e-3))))
    if Ls2 > Ls:
        Ls, t = Ls2, run(Ls2)
    return {"value": Xs.shape[0] / (t / Ls * wl.L), "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle top-{k} of {Xs.shape[0]} queries over the first {Ls} of {wl.L} labels took "
                      f"{t:.2f} s; scaled linearly to all labels", "seconds": round(t, 3), "labels": Ls}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: runs on exactly one GPU (--gpus 1); multi-GPU runs are not implemented",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_bytes:
        copy_reference(args.copy_bytes)
        return

    import numpy as np
    import torch

    import precision_label_chunk_amd as elmo
    import workloads as wk

    wl = wk.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    elmo.lib()
    torch.cuda.reset_peak_memory_stats(dev)

    # inputs resident in HBM before timing
    W = wk.make_w_device(wl.L, wl.D, wl.wfmt, seed=wl.seed, device=dev)
    nb = args.warmup + args.steps
    host_batches = [wk.make_batch(wl, step=s) for s in range(nb)]
    batches = []
    for bt in host_batches:
        batches.append((torch.from_numpy(bt.X.view(np.int16)).to(dev), torch.from_numpy(bt.row_ptr).to(dev),
                        torch.from_numpy(bt.ids).to(dev)))
    max_nnz = max(int(b[2].numel()) for b in batches)
    ws = torch.empty((elmo.step_workspace_bytes(wl.B, wl.D, wl.L, wl.chunk, wl.wfmt, max_nnz),), dtype=torch.uint8,
                     device=dev)
    dX = torch.empty((wl.B, wl.D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    # the step's peak HBM counts what is resident while it runs (the library allocates nothing),
    # not the transients of generating the weights
    torch.cuda.reset_peak_memory_stats(dev)
    hbm_parts = {"weights": W.numel() * W.element_size(), "workspace": ws.numel(),
                 "batches": sum(t.numel() * t.element_size() for b in batches for t in b),
                 "dX": dX.numel() * 4}

    # the first warm-up step runs with cold caches (and the library's lazy set-up): timed on its own
    evc = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for s in range(args.warmup):
        X, rp, ids = batches[s]
        if s == 0:
            evc[0].record(torch.cuda.current_stream())
        elmo.step(W, X, rp, ids, wl.lr, wl.seed, s, wl.chunk, dX=dX, workspace=ws)
        if s == 0:
            evc[1].record(torch.cuda.current_stream())
    torch.cuda.synchronize()
    first_ms = evc[0].elapsed_time(evc[1]) if args.warmup else None

    # the timed steps: whole-step throughput, with no event between the step's kernels
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for s in range(args.warmup, nb):
        X, rp, ids = batches[s]
        elmo.step(W, X, rp, ids, wl.lr, wl.seed, s, wl.chunk, dX=dX, workspace=ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_step = total_ms / args.steps

    # the same number of steps again with HIP events around every forward and backward launch (on
    # the step's stream) for the per-kernel averages; the events add a few microseconds between
    # the kernels they bracket, so this pass is timed separately and reported as such
    elmo.kernel_timing(True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i, s in enumerate(range(args.warmup, nb)):
        X, rp, ids = batches[s]
        elmo.step(W, X, rp, ids, wl.lr, wl.seed, nb + s, wl.chunk, dX=dX, workspace=ws)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    elmo.kernel_timing(False)
    kt = elmo.kernel_timing_read()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    events_ms_step = evs[0].elapsed_time(evs[-1]) / args.steps
    h = len(per_step) // 2
    events_median = per_step[h] if len(per_step) % 2 else 0.5 * (per_step[h - 1] + per_step[h])
    peak_hbm = torch.cuda.max_memory_allocated(dev)
    free_b, total_b = torch.cuda.mem_get_info(dev)   # hipMemGetInfo: the device's own view, for comparison

    B, D, L = wl.B, wl.D, wl.L
    flops = 6.0 * B * D * L
    fwd_peak = PEAK["fp8"] if wl.wfmt == wk.W_E4M3 else PEAK["bf16"]
    t_ideal = 2.0 * B * D * L / fwd_peak + 4.0 * B * D * L / PEAK["bf16"]
    alg_bytes = 2.0 * L * D * wl.wbytes
    samples_s = B * args.steps / (total_ms / 1e3)

    # dominant kernel roofline from the live per-launch events
    kern = {}
    for name, per_label, peak in (("bwd", 4.0 * B * D, PEAK["bf16"]), ("fwd", 2.0 * B * D, fwd_peak)):
        ms, n, labels = kt[name]
        if n:
            ach = labels * per_label / (ms / 1e3)
            kern[name] = {"ms_total": ms, "launches": n, "avg_ms": ms / n, "achieved": ach, "peak": peak}
    dom = max(kern, key=lambda k: kern[k]["ms_total"])
    kd = kern[dom]
    kname = "k_bwd_update" if dom == "bwd" else "k_fwd_g"
    tr = measured_traffic(args.workload, kname)
    roofline = {"kernel": kname, "bound": "mfma",
                "achieved": round(kd["achieved"] / 1e12, 2), "peak": round(kd["peak"] / 1e12, 1),
                "unit": "TFLOP/s", "frac": round(kd["achieved"] / kd["peak"], 4),
                "traffic": None if tr is None else int(tr["bytes"]),
                "traffic_read_write": None if tr is None else [int(tr["read"]), int(tr["write"])],
                "avg_launch_ms": round(kd["avg_ms"], 4), "launches": kd["launches"],
                "events_pass_ms_per_step": round(events_ms_step, 4),
                "events_pass_median_ms_per_step": round(events_median, 4),
                "flops_per_label": (4 if dom == "bwd" else 2) * B * D}
    other = [k for k in kern if k != dom]
    if other:
        ko = kern[other[0]]
        roofline["other_kernel"] = {"kernel": "k_fwd_g" if other[0] == "fwd" else "k_bwd_update",
                                    "achieved_tflops": round(ko["achieved"] / 1e12, 2),
                                    "peak_tflops": round(ko["peak"] / 1e12, 1),
                                    "frac": round(ko["achieved"] / ko["peak"], 4),
                                    "avg_launch_ms": round(ko["avg_ms"], 4)}

    out = {"metric": METRIC, "value": round(samples_s, 1), "unit": "samples/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "first_step_ms": None if first_ms is None else round(first_ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "e4m3+bf16" if wl.wfmt == wk.W_E4M3 else "bf16", "data": "synthetic",
           "config": {"workload": wl.name, "B": B, "D": D, "L": L, "chunk": wl.chunk,
                      "weights": "e4m3" if wl.wfmt == wk.W_E4M3 else "bf16", "lr": wl.lr},
           "tflops": round(flops / (ms_step / 1e3) / 1e12, 2),
           "mfma_roofline_frac": round(t_ideal / (ms_step / 1e3), 4),
           "alg_hbm_gbs": round(alg_bytes / (ms_step / 1e3) / 1e9, 1),
           "hbm_frac": round(alg_bytes / (ms_step / 1e3) / PEAK["hbm"], 4),
           "peak_hbm_bytes": int(peak_hbm),
           "peak_hbm_breakdown": {k: int(v) for k, v in hbm_parts.items()},
           "device_used_bytes": int(total_b - free_b),
           "weights_bytes": int(L * D * wl.wbytes),
           "roofline": roofline}

    if not args.no_topk:
        N, k = args.topk_n, (wl.topk or 5)
        Xe_host = wk.make_eval_x(wl, N)
        Xe = torch.from_numpy(Xe_host.view(np.int16)).to(dev)
        tws = torch.empty((elmo.topk_workspace_bytes(N, D, L, k, wl.wfmt),), dtype=torch.uint8, device=dev)
        elmo.topk(W, Xe, k, workspace=tws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        elmo.topk(W, Xe, k, workspace=tws)
        e1.record(stream)
        torch.cuda.synchronize()
        tk = e0.elapsed_time(e1)
        tf = 2.0 * N * D * L
        out["topk"] = {"N": N, "k": k, "ms": round(tk, 3), "samples_s": round(N / (tk / 1e3), 1),
                       "tflops": round(tf / (tk / 1e3) / 1e12, 2),
                       "frac": round(tf / (tk / 1e3) / fwd_peak, 4)}
        if not args.no_cpu_baseline:
            out["topk"]["cpu_baseline"] = cpu_topk_baseline(wl, W, Xe_host, k, args.cpu_seconds / 3)

    if not args.no_kahan:
        out["kahan_update"] = kahan_bench(args.kahan_params, stream)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, W, host_batches[0], args.cpu_seconds)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
