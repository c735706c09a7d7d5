"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host code only) and run
over every exported function on small inputs and edge cases (tests/oracle_sanitize.c): no invalid
memory access, leak or undefined arithmetic, and the properties the driver checks hold."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_address_and_ub_sanitizers():
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    d = tempfile.mkdtemp()
    exe = os.path.join(d, "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "elmo_oracle.c"), os.path.join(HERE, "oracle_sanitize.c"), "-lm", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 and "asan" in (res.stderr or "").lower():
        pytest.skip("sanitizer runtime not available: " + res.stderr[-300:])
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    shutil.rmtree(d, ignore_errors=True)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "ok" in run.stdout
