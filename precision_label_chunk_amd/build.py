"""Build step for the HIP library: compiles every source under csrc/ for gfx950 into
libelmo_xmc.so next to this file (in-tree, so it travels with the source tree).

Each source is compiled to its own object (in parallel, under _build/ at the repository root),
then the objects are linked; no translation unit calls device code of another, so no relocatable
device code is needed."""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libelmo_xmc.so")
OBJDIR = os.path.join(ROOT, "_build")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-ffp-contract=off",                        # every rounding point stays where the source puts it
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


# sources compiled once per variant (each variant defines the macros listed)
VARIANTS = {
    "step_chunks.hip": [{"ELMO_MB": mb, "ELMO_WF": wf} for wf in (0, 1, 2) for mb in (32, 64, 128, 256)],
}


def sources():
    csrc = os.path.join(HERE, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.hip"))) + sorted(glob.glob(os.path.join(csrc, "*.cpp")))


def units():
    """(source, object name, -D flags) for every object of the library."""
    out = []
    for src in sources():
        base = os.path.basename(src)
        for v in VARIANTS.get(base, [None]):
            if v is None:
                out.append((src, base + ".o", []))
            else:
                tag = "_".join(f"{k}{val}" for k, val in v.items())
                out.append((src, f"{base}.{tag}.o", [f"-D{k}={val}" for k, val in v.items()]))
    return out


def _compile(hipcc, unit):
    src, name, defs = unit
    obj = os.path.join(OBJDIR, name)
    res = subprocess.run([hipcc, *HIPCC_FLAGS, *defs, "-c", src, "-o", obj], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} {' '.join(defs)}:\n" + res.stdout + res.stderr)
    return obj


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJDIR, exist_ok=True)
    us = units()
    jobs = max(1, min(len(us), int(os.environ.get("MAX_JOBS", "8") or 8)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda u: _compile(hipcc, u), us))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
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
