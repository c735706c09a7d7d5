"""The benchmark's output contract on a small workload: one JSON line with the metric, the
whole-step throughput, the dominant kernel's roofline from live event timing, the top-k pass and
the CPU oracle baselines (with their bounded samples)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line_on_the_tiny_workload():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3", "--warmup", "1",
           "--topk-n", "64", "--kahan-params", "100000", "--cpu-seconds", "0.3"]
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
    assert d["config"]["workload"] == "xmc-bf16-L4096-D64-B32"
    ro = d["roofline"]
    assert ro["bound"] == "mfma" and ro["unit"] == "TFLOP/s" and ro["peak"] == 2500.0
    assert ro["achieved"] > 0 and ro["frac"] == pytest.approx(ro["achieved"] / ro["peak"], rel=1e-2, abs=1e-4)
    assert ro["launches"] == 3 * 4                          # 4 chunks per step, one launch each
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    tk = d["topk"]
    assert tk["N"] == 64 and tk["k"] == 5 and tk["ms"] > 0 and tk["cpu_baseline"]["value"] > 0
    assert d["kahan_update"]["params"] == 100000
