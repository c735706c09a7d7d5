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
own (`first_step_ms`). The same line carries a `bf16_8p6m` object measured the same way on the
8.6M-label BF16 head (B=128, D=768, chunk 262,144, lr 0.05), whose step is bound by HBM, with its
own top-5 pass over 4,096 held-out queries, roofline and CPU baseline, and a `mxfp4_3m` object for
the 3M-label head with MX-scaled FP4 weights (B=256, D=768, chunk 131,072, lr 0.1).
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
                    help="one of tiny, bf16_131k, bf16_670k, e4m3_3m, bf16_8p6m, mxfp4_3m")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-topk", action="store_true")
    ap.add_argument("--topk-n", type=int, default=4096)
    ap.add_argument("--no-kahan", action="store_true")
    ap.add_argument("--second-workload", default="bf16_8p6m",
                    help="workload measured into its own object of the same line ('none' to skip)")
    ap.add_argument("--no-8p6m", action="store_true", help="same as --second-workload none")
    ap.add_argument("--steps-8p6m", type=int, default=10, help="timed steps of the second workload")
    ap.add_argument("--third-workload", default="mxfp4_3m",
                    help="a third workload in its own object of the line ('none' to skip): by default the "
                         "3M-label head with MX-scaled FP4 weights")
    ap.add_argument("--steps-third", type=int, default=10, help="timed steps of the third workload")
    ap.add_argument("--small-workloads", default="bf16_131k,bf16_670k",
                    help="comma-separated further workloads timed without top-k and CPU baseline, or 'none'")
    ap.add_argument("--shard-workloads", default="e4m3_375k,bf16_1075k",
                    help="one GPU's share of the 3M- and 8.6M-label heads split over eight GPUs (none: skip)")
    ap.add_argument("--single-pass-workloads", default="bf16_8p6m_b32,e4m3_3m_b32",
                    help="comma-separated workloads (B <= 32) timed with the single-pass step and the two-kernel "
                         "step side by side, or 'none'")
    ap.add_argument("--steps-single", type=int, default=10, help="timed steps of each single-pass comparison")
    ap.add_argument("--single-pass", action="store_true",
                    help="run the main workload (B <= 32) with the single-pass step (for profiling it alone); "
                         "with --summarize-traffic: the file's commands carry this flag")
    ap.add_argument("--kahan-params", type=int, default=110_000_000,
                    help="encoder parameters of the Kahan-compensated BF16 update pass (768-wide, 12 layers)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (3 times) and exit: the "
                         "known-size reference for scaling HBM byte counters")
    ap.add_argument("--summarize-stats", metavar="DIR",
                    help="no GPU: print the markdown kernel-time table of a rocprofv3 --stats output folder")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="no GPU: print the per-dispatch table of every counter in these rocprofv3 --pmc output "
                         "folders for the step's chunk kernels")
    ap.add_argument("--summarize-traffic", nargs=5, metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                              "COPY_WRITE_DIR"),
                    help="no GPU: print the HBM-bytes-per-launch file (the format bench.py reads for "
                         "roofline.traffic) from four rocprofv3 --pmc output folders")
    return ap.parse_args()


# ---- summaries of rocprofv3 output (CSV), written into profiles/ --------------------------------
def _csv_rows(folder, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {folder}")
    return rows


def summarize_stats(folder):
    """Markdown table of a --kernel-trace --stats run: calls, total and average time per kernel."""
    rows = _csv_rows(folder, "kernel_stats.csv")
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    print("| kernel | calls | total ms | average us | share % |")
    print("|---|---|---|---|---|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].split("(")[0].strip()
        name = name[5:] if name.startswith("void ") else name
        name = name if len(name) <= 70 else name[:67] + "..."
        t = float(r["TotalDurationNs"])
        print(f"| `{name}` | {r['Calls']} | {t / 1e6:.3f} | {float(r['AverageNs']) / 1e3:.2f} | {100 * t / total:.2f} |")


def _counter_per_kernel(folder, counter):
    """{kernel template name: (mean KiB per dispatch, dispatches)} of one counter's pass."""
    per = {}
    for r in _csv_rows(folder, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        name = _kernel_key(r["Kernel_Name"])
        v = per.setdefault(name, {})
        key = r["Dispatch_Id"]
        v[key] = v.get(key, 0.0) + float(r["Counter_Value"])
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in per.items()}


def summarize_counters(folders):
    """Markdown table: every counter of the passes (rows) per chunk kernel (columns), as the mean
    over its dispatches of the device-wide sum per dispatch."""
    table = {}
    for folder in folders:
        for r in _csv_rows(folder, "counter_collection.csv"):
            name = _kernel_key(r["Kernel_Name"])
            if not (name.startswith("k_bwd_update") or name.startswith("k_fwd") or name.startswith("k_step_single")):
                continue
            d = table.setdefault(r["Counter_Name"], {}).setdefault(name, {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    kernels = sorted({k for v in table.values() for k in v})
    print("| counter | " + " | ".join(f"`{k}`" for k in kernels) + " |")
    print("|---|" + "---|" * len(kernels))
    for c in sorted(table):
        cells = []
        for k in kernels:
            v = table[c].get(k)
            cells.append(f"{sum(v.values()) / len(v):.4g}" if v else "")
        print(f"| {c} | " + " | ".join(cells) + " |")


def _kernel_key(name):
    """'k_name<args>' from a demangled kernel name (return type, namespace, parameters and spaces
    dropped)."""
    name = name.split("(")[0].strip()
    if name.startswith("void "):
        name = name[5:]
    return name.replace("elmo::", "").replace(" ", "")


def summarize_traffic(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, single=False):
    """The HBM bytes per launch of each kernel: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
    scaled by what the same counter reads for a plain copy of known size (read and written once)."""
    def copy_factor(folder, counter):
        per = _counter_per_kernel(folder, counter)
        kib, _ = max(per.values(), key=lambda v: v[0])         # the copy kernel dominates the run
        return kib, (1 << 30) / 1024 / kib
    cf, ff = copy_factor(copy_fetch_dir, "FETCH_SIZE")
    cw, fw = copy_factor(copy_write_dir, "WRITE_SIZE")
    import workloads as wk
    print(f"# HBM bytes per launch, workload {wk.WORKLOADS[workload].name}")
    print("# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from one rocprofv3 pass each, scaled by what the same")
    print("# counter reads for a plain 1 GiB device copy (1048576 KiB read and written per launch).")
    print("# commands (from the repository root on the GPU box):")
    for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        print(f"#   export TMPDIR=/tmp && rocprofv3 --pmc {c} -f csv -d {d} -o run -- python3 bench.py --steps 2 "
              f"--warmup 1 --no-cpu-baseline --no-topk --no-kahan --second-workload none --third-workload none "
              f"--single-pass-workloads none --small-workloads none --shard-workloads none --workload {workload}"
              f"{' --single-pass' if single else ''}")
    for c, d in (("FETCH_SIZE", copy_fetch_dir), ("WRITE_SIZE", copy_write_dir)):
        print(f"#   export TMPDIR=/tmp && rocprofv3 --pmc {c} -f csv -d {d} -o run -- python3 bench.py "
              f"--copy-bytes 1073741824")
    print(f"#   python3 bench.py --summarize-traffic {workload} {fetch_dir} {write_dir} {copy_fetch_dir} {copy_write_dir}"
          f"{' --single-pass' if single else ''}")
    print(f"source_sha256 {kernel_source_hash()}")
    print(f"copy_fetch_size_kib {cf:.1f} factor {ff:.4f}")
    print(f"copy_write_size_kib {cw:.1f} factor {fw:.4f}")
    for counter, folder, f, tag in (("FETCH_SIZE", fetch_dir, ff, "fetch_size_kib"),
                                    ("WRITE_SIZE", write_dir, fw, "write_size_kib")):
        for k, (kib, n) in sorted(_counter_per_kernel(folder, counter).items()):
            if k.startswith("k_") or k.startswith("elmo"):
                print(f"{k} {tag} {kib:.1f} bytes {int(kib * 1024 * f)} dispatches {n}")


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
    """A plain copy of `nbytes` bytes, three times: each launch reads and writes exactly nbytes. Also
    reports the copy's own rate (bytes read plus written per second, HIP events around the three
    launches): a practical ceiling for kernels that read and write HBM, beside the spec peak."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 3
    print(json.dumps({"copy_bytes": nbytes, "launches": 3, "ms_per_copy": round(ms, 4),
                      "read_write_gbs": round(2 * nbytes / (ms / 1e3) / 1e9, 1)}), flush=True)


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


def cpu_info():
    """Host CPU model (from /proc/cpuinfo) and logical CPU count."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count()}


def bench_workload(name, steps, warmup, args, with_topk=True, with_cpu=True, single=None):
    """One workload: W resident in HBM, `warmup` untimed steps (the first timed on its own), `steps`
    timed steps with no event between kernels, then the same number again with events around every
    forward and backward launch for the per-kernel averages; the top-k pass; the CPU oracle on a
    bounded sample. Returns the workload's JSON object; frees its device memory."""
    import numpy as np
    import torch

    import precision_label_chunk_amd as elmo
    import workloads as wk

    wl = wk.WORKLOADS[name]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    # single: True = the single-pass entry, False = the two-kernel entry, None = elmo_xmc_step (the
    # faster path for the shape; the pages' workloads have B > 32 and take the two-kernel step)
    sp_arg = single
    runs_single = single if single is not None else (wl.B <= 32 and wl.D in (256, 512, 768))
    torch.cuda.reset_peak_memory_stats(dev)

    # inputs resident in HBM before timing
    W = wk.make_w_device(wl.L, wl.D, wl.wfmt, seed=wl.seed, device=dev)
    nb = warmup + steps
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
    # not the transients of generating the weights, nor the previous workload's workspace, which the
    # binding keeps as its last one (for step_flags) until the next step replaces it
    elmo.last_workspace = None
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    hbm_parts = {"weights": W.numel() * W.element_size(), "workspace": ws.numel(),
                 "batches": sum(t.numel() * t.element_size() for b in batches for t in b),
                 "dX": dX.numel() * 4}

    # the first warm-up step runs with cold caches (and the library's lazy set-up): timed on its own
    evc = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for s in range(warmup):
        X, rp, ids = batches[s]
        if s == 0:
            evc[0].record(stream)
        elmo.step(W, X, rp, ids, wl.lr, wl.seed, s, wl.chunk, dX=dX, workspace=ws, wfmt=wl.wfmt,
                  single_pass=sp_arg)
        if s == 0:
            evc[1].record(stream)
    torch.cuda.synchronize()
    first_ms = evc[0].elapsed_time(evc[1]) if warmup else None

    # the timed steps: whole-step throughput, with no event between the step's kernels
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for s in range(warmup, nb):
        X, rp, ids = batches[s]
        elmo.step(W, X, rp, ids, wl.lr, wl.seed, s, wl.chunk, dX=dX, workspace=ws, wfmt=wl.wfmt,
                  single_pass=sp_arg)
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_step = total_ms / steps

    # the same number of steps again with HIP events around every forward and backward launch (on
    # the step's stream) for the per-kernel averages; the events add a few microseconds between
    # the kernels they bracket, so this pass is timed separately and reported as such
    elmo.kernel_timing(True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i, s in enumerate(range(warmup, nb)):
        X, rp, ids = batches[s]
        elmo.step(W, X, rp, ids, wl.lr, wl.seed, nb + s, wl.chunk, dX=dX, workspace=ws, wfmt=wl.wfmt,
                  single_pass=sp_arg)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    elmo.kernel_timing(False)
    kt = elmo.kernel_timing_read()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    events_ms_step = evs[0].elapsed_time(evs[-1]) / steps
    h = len(per_step) // 2
    events_median = per_step[h] if len(per_step) % 2 else 0.5 * (per_step[h - 1] + per_step[h])
    peak_hbm = torch.cuda.max_memory_allocated(dev)
    # hipMemGetInfo, the device's own view, with torch's cached free blocks returned first: what it
    # reports beyond the live allocations is the runtime's own memory (context, code objects)
    live = torch.cuda.memory_allocated(dev)
    torch.cuda.empty_cache()
    free_b, total_b = torch.cuda.mem_get_info(dev)
    reserved = torch.cuda.memory_reserved(dev)

    B, D, L = wl.B, wl.D, wl.L
    flops = 6.0 * B * D * L
    # the forward's contraction: BF16 x BF16, E4M3 x E4M3, or E4M3 x E2M1 (MXFP4), which the scaled
    # matrix cores run at the FP8 rate (an 8-bit operand sets it)
    fwd_peak = PEAK["bf16"] if wl.wfmt == wk.W_BF16 else PEAK["fp8"]
    t_mfma = 2.0 * B * D * L / fwd_peak + 4.0 * B * D * L / PEAK["bf16"]
    alg_bytes = 2.0 * L * D * wl.wbytes
    t_hbm = alg_bytes / PEAK["hbm"]
    samples_s = B * steps / (total_ms / 1e3)

    # per-kernel rooflines from the live per-launch events. Algorithmic work per label: forward
    # 2 B D flops and D w bytes (W read); backward 4 B D flops and 2 D w bytes (W read and write).
    # A kernel is MFMA- or HBM-bound by its arithmetic intensity against the ridge point.
    # The single-pass kernel (timed in the backward's slot) does the whole step's work per label:
    # 6 B D flops on the BF16 matrix cores and 2 D w bytes (W read and written once).
    kern = {}
    per_kernel = ((("bwd", 6.0 * B * D, 2.0 * D * wl.wbytes, PEAK["bf16"]),) if runs_single else
                  (("bwd", 4.0 * B * D, 2.0 * D * wl.wbytes, PEAK["bf16"]),
                   ("fwd", 2.0 * B * D, 1.0 * D * wl.wbytes, fwd_peak)))
    for kn, per_label_f, per_label_b, peak_f in per_kernel:
        ms, n, labels = kt[kn]
        if not n:
            continue
        sec = ms / 1e3
        hbm_bound = per_label_f / per_label_b < peak_f / PEAK["hbm"]
        if hbm_bound:
            ach, peak, unit = labels * per_label_b / sec, PEAK["hbm"], "GB/s"
        else:
            ach, peak, unit = labels * per_label_f / sec, peak_f, "TFLOP/s"
        kern[kn] = {"ms_total": ms, "launches": n, "avg_ms": ms / n, "achieved": ach, "peak": peak, "unit": unit,
                    "bound": "hbm" if hbm_bound else "mfma", "labels_per_launch": labels / n,
                    "per_label": per_label_b if hbm_bound else per_label_f}
    dom = max(kern, key=lambda k: kern[k]["ms_total"])
    kd = kern[dom]
    # the forward kernel the launcher picks for this workload
    fwd_kernel = ("k_fwd_xs" if wl.wfmt != wk.W_BF16 and D == 768 and B > 128 else
                  "k_fwd_xb" if wl.wfmt == wk.W_BF16 and D == 768 and 64 < B <= 128 else
                  "k_fwd_mx" if wl.wfmt == wk.W_MXFP4 else "k_fwd_g")
    kname = {"bwd": "k_step_single" if runs_single else "k_bwd_update", "fwd": fwd_kernel}
    scale = 1e9 if kd["unit"] == "GB/s" else 1e12
    tr = measured_traffic(name, kname[dom])
    roofline = {"kernel": kname[dom], "bound": kd["bound"],
                "achieved": round(kd["achieved"] / scale, 2), "peak": round(kd["peak"] / scale, 1),
                "unit": kd["unit"], "frac": round(kd["achieved"] / kd["peak"], 4),
                "traffic": None if tr is None else int(tr["bytes"]),
                "traffic_read_write": None if tr is None else [int(tr["read"]), int(tr["write"])],
                "avg_launch_ms": round(kd["avg_ms"], 4), "launches": kd["launches"],
                "labels_per_launch": round(kd["labels_per_launch"], 1),
                "events_pass_ms_per_step": round(events_ms_step, 4),
                "events_pass_median_ms_per_step": round(events_median, 4),
                ("bytes_per_label" if kd["bound"] == "hbm" else "flops_per_label"): int(kd["per_label"])}
    for other in [k for k in kern if k != dom]:
        ko = kern[other]
        so = 1e9 if ko["unit"] == "GB/s" else 1e12
        roofline["other_kernel"] = {"kernel": kname[other], "bound": ko["bound"],
                                    "achieved": round(ko["achieved"] / so, 2), "peak": round(ko["peak"] / so, 1),
                                    "unit": ko["unit"], "frac": round(ko["achieved"] / ko["peak"], 4),
                                    "avg_launch_ms": round(ko["avg_ms"], 4)}

    out = {"ms_per_step": round(ms_step, 4), "samples_s": round(samples_s, 1), "steps": steps, "warmup": warmup,
           "first_step_ms": None if first_ms is None else round(first_ms, 4),
           "config": {"workload": wl.name, "B": B, "D": D, "L": L, "chunk": wl.chunk,
                      "weights": {wk.W_BF16: "bf16", wk.W_E4M3: "e4m3", wk.W_MXFP4: "mxfp4"}[wl.wfmt],
                      "lr": wl.lr},
           "dtype": {wk.W_BF16: "bf16", wk.W_E4M3: "e4m3+bf16", wk.W_MXFP4: "e4m3xe2m1+bf16"}[wl.wfmt],
           "tflops": round(flops / (ms_step / 1e3) / 1e12, 2),
           "mfma_roofline_frac": round(t_mfma / (ms_step / 1e3), 4),
           "alg_hbm_gbs": round(alg_bytes / (ms_step / 1e3) / 1e9, 1),
           "hbm_frac": round(t_hbm / (ms_step / 1e3), 4),
           "roofline_bound": "mfma" if t_mfma >= t_hbm else "hbm",
           "roofline_frac": round(max(t_mfma, t_hbm) / (ms_step / 1e3), 4),
           "peak_hbm_bytes": int(peak_hbm),
           "peak_hbm_breakdown": {k: int(v) for k, v in hbm_parts.items()},
           "peak_hbm_budget_bytes": int(L * D * wl.wbytes + 2 * B * wl.chunk + 64 * 2**20),
           "device_used_bytes": int(total_b - free_b), "live_bytes": int(live),
           "device_used_beyond_live_bytes": int(total_b - free_b - live), "torch_reserved_bytes": int(reserved),
           "weights_bytes": int(L * D * wl.wbytes),
           "roofline": roofline}

    if with_topk:
        N, k = args.topk_n, (wl.topk or 5)
        Xe_host = wk.make_eval_x(wl, N)
        Xe = torch.from_numpy(Xe_host.view(np.int16)).to(dev)
        tws = torch.empty((elmo.topk_workspace_bytes(N, D, L, k, wl.wfmt),), dtype=torch.uint8, device=dev)
        elmo.topk(W, Xe, k, workspace=tws, wfmt=wl.wfmt)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        elmo.topk(W, Xe, k, workspace=tws, wfmt=wl.wfmt)
        e1.record(stream)
        torch.cuda.synchronize()
        tk = e0.elapsed_time(e1)
        tf = 2.0 * N * D * L
        out["topk"] = {"N": N, "k": k, "ms": round(tk, 3), "samples_s": round(N / (tk / 1e3), 1),
                       "tflops": round(tf / (tk / 1e3) / 1e12, 2),
                       "frac": round(tf / (tk / 1e3) / fwd_peak, 4)}
        if with_cpu:
            out["topk"]["cpu_baseline"] = cpu_topk_baseline(wl, W, Xe_host, k, args.cpu_seconds / 3)
        del Xe, tws

    if with_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, W, host_batches[0], args.cpu_seconds)

    del W, ws, dX, batches
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.summarize_stats:
        summarize_stats(args.summarize_stats)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, single=args.single_pass)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: runs on exactly one GPU (--gpus 1); multi-GPU runs are not implemented",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_bytes:
        copy_reference(args.copy_bytes)
        return

    import torch

    import precision_label_chunk_amd as elmo

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    elmo.lib()

    main_w = bench_workload(args.workload, args.steps, args.warmup, args, with_topk=not args.no_topk,
                            with_cpu=not args.no_cpu_baseline, single=True if args.single_pass else None)
    out = {"metric": METRIC, "value": main_w["samples_s"], "unit": "samples/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_w["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": main_w["dtype"], "data": "synthetic", "config": main_w["config"]}
    for key in ("first_step_ms", "tflops", "mfma_roofline_frac", "alg_hbm_gbs", "hbm_frac", "peak_hbm_bytes",
                "peak_hbm_breakdown", "peak_hbm_budget_bytes", "device_used_bytes", "live_bytes",
                "device_used_beyond_live_bytes", "torch_reserved_bytes",
                "weights_bytes", "roofline", "topk", "cpu_baseline"):
        if key in main_w:
            out[key] = main_w[key]

    if not args.no_kahan:
        out["kahan_update"] = kahan_bench(args.kahan_params, torch.cuda.current_stream())

    # the second label space the method is measured on (default: 8.6M labels in BF16 with B = 128,
    # bound by HBM), in an object of its own keyed by the workload's name
    second = "none" if args.no_8p6m else args.second_workload
    extra = [(second, args.steps_8p6m), (args.third_workload, args.steps_third)]
    for name, nsteps in extra:
        if name != "none":
            out[name] = bench_workload(name, nsteps, 2, args, with_topk=not args.no_topk,
                                       with_cpu=not args.no_cpu_baseline)

    # the 131k- and 670k-label BF16 heads (B = 256), each in an object of its own
    for name in [w for w in args.small_workloads.split(",") if w and w != "none"]:
        out[name] = bench_workload(name, args.steps_third, 2, args, with_topk=False, with_cpu=False)

    # one GPU's share of each head split by label ranges over eight GPUs: the kernels at a shard's
    # real shape (the one exchange such a split needs, an all-reduce of dX, is not run here)
    shards = [w for w in args.shard_workloads.split(",") if w and w != "none"]
    if shards:
        out["label_shard_of_8"] = {name: bench_workload(name, args.steps_third, 2, args, with_topk=False, with_cpu=False)
                                   for name in shards}

    # the single-pass step beside the two-kernel step on the same small-batch workloads
    sp = [w for w in args.single_pass_workloads.split(",") if w and w != "none"]
    if sp:
        out["single_pass"] = {}
        for name in sp:
            one = bench_workload(name, args.steps_single, 2, args, with_topk=False, with_cpu=False, single=True)
            two = bench_workload(name, args.steps_single, 2, args, with_topk=False, with_cpu=False, single=False)
            out["single_pass"][name] = {
                "single_pass": one, "two_kernel": two,
                "speedup": round(two["ms_per_step"] / one["ms_per_step"], 3)}

    info = cpu_info()
    for obj in [out] + [out.get(name, {}) for name, _ in extra]:
        for cb in (obj.get("cpu_baseline"), obj.get("topk", {}).get("cpu_baseline")):
            if cb is not None:
                cb.update(info)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
