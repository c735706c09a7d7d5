"""The benchmark's output contract on small workloads: one JSON line with the metric, the
whole-step throughput, the dominant kernel's roofline from live event timing, the top-k pass and
the CPU oracle baselines (with their bounded samples and the host CPU), the second and third
workloads' objects measured the same way, a further workload's object without top-k, and the
single-pass step beside the two-kernel step on a 32-sample workload."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line_on_the_tiny_workload():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3", "--warmup", "1",
           "--topk-n", "64", "--kahan-params", "100000", "--cpu-seconds", "0.3", "--second-workload", "bf16_131k",
           "--steps-8p6m", "2", "--third-workload", "mxfp4_131k", "--steps-third", "2",
           "--small-workloads", "bf16_670k", "--single-pass-workloads", "e4m3_3m_b32", "--steps-single", "2",
           "--shard-workloads", "e4m3_375k"]
    print("  " + " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "topk",
                "kahan_update", "first_step_ms", "peak_hbm_bytes"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
    # the device's own count of used memory, torch's cached blocks returned, covers the live allocations
    assert d["device_used_bytes"] >= d["live_bytes"] > 0
    assert d["config"]["workload"] == "xmc-bf16-L4096-D64-B32"
    ro = d["roofline"]
    # B = 32, D = 64: the backward's 4 B D flops per 2 D w bytes (32 flop/B) sit below the ridge point
    assert ro["bound"] == "hbm" and ro["unit"] == "GB/s" and ro["peak"] == 8000.0
    assert ro["achieved"] > 0 and ro["frac"] == pytest.approx(ro["achieved"] / ro["peak"], rel=1e-2, abs=1e-4)
    assert ro["launches"] == 3 * 4                          # 4 chunks per step, one launch each
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["nproc"] >= 1 and "cpu_model" in cb
    tk = d["topk"]
    assert tk["N"] == 64 and tk["k"] == 5 and tk["ms"] > 0 and tk["cpu_baseline"]["value"] > 0
    assert d["kahan_update"]["params"] == 100000
    s2 = d["bf16_131k"]
    assert s2["config"]["workload"] == "xmc-bf16-L131072-D768-B256" and s2["samples_s"] > 0
    # (B = 256, BF16: the backward moves 2 D w = 3,072 bytes per 786,432 flops, 256 flop/B: below the ridge)
    assert s2["roofline"]["bound"] == "hbm" and s2["roofline"]["launches"] == 2 * 4
    assert s2["cpu_baseline"]["value"] > 0 and s2["topk"]["ms"] > 0 and s2["peak_hbm_bytes"] > 0
    s3 = d["mxfp4_131k"]
    assert s3["config"]["weights"] == "mxfp4" and s3["samples_s"] > 0 and s3["topk"]["ms"] > 0
    # (B = 256, MXFP4: the backward moves 2 * 17 D / 32 bytes per 4 B D flops, 964 flop/B: above the
    # BF16 ridge point; at 256 samples and D = 768 the forward is the stationary-feature kernel)
    assert s3["roofline"]["bound"] == "mfma" and s3["roofline"]["other_kernel"]["kernel"] == "k_fwd_xs"
    s4 = d["bf16_670k"]
    assert s4["config"]["L"] == 670000 and s4["samples_s"] > 0 and "topk" not in s4
    sp = d["single_pass"]["e4m3_3m_b32"]
    assert sp["single_pass"]["roofline"]["kernel"] == "k_step_single" and sp["single_pass"]["roofline"]["bound"] == "hbm"
    assert sp["two_kernel"]["roofline"]["kernel"] == "k_bwd_update"
    assert sp["speedup"] == pytest.approx(sp["two_kernel"]["ms_per_step"] / sp["single_pass"]["ms_per_step"], rel=1e-2)
    sh = d["label_shard_of_8"]["e4m3_375k"]
    assert sh["config"]["L"] == 375000 and sh["config"]["B"] == 256 and sh["samples_s"] > 0
    assert sh["roofline"]["kernel"] == "k_bwd_update" and sh["roofline"]["launches"] == 2 * 3   # 3 chunks per step
