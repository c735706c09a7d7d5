"""Build step for the HIP library: compiles every source under csrc/ for gfx950 into
libelmo_xmc.so next to this file (in-tree, so it travels with the source tree)."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libelmo_xmc.so")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    "-ffp-contract=off",                        # every rounding point stays where the source puts it
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def sources():
    csrc = os.path.join(HERE, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.hip"))) + sorted(glob.glob(os.path.join(csrc, "*.cpp")))


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    # a kernel template whose host stub was silently not instantiated shows up as an undefined
    # symbol of this library: refuse such a build instead of failing at load time
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in nm.stdout.splitlines() if "elmo" in ln]
    if missing:
        raise RuntimeError("libelmo_xmc.so has undefined library symbols: " + ", ".join(missing[:5]))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
