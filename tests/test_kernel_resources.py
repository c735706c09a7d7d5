"""Register budget of the step kernels (no GPU): the compiler's resource report for every
instantiation of the kernels on the timed step paths must show no scratch memory. A spill inside a
tile loop turns register traffic into memory traffic in the hot loop (and an accumulator array
indexed at run time, when an unroll fails, lands in scratch the same way). Each object is compiled
here for gfx950 with the library's own flags."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from precision_label_chunk_amd import build as B

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(os.path.dirname(B.__file__), "csrc")
INCLUDE = os.path.join(os.path.dirname(os.path.dirname(B.__file__)), "include")

# (source, defines): the weight formats and padded batches of the measured workloads
UNITS = [
    ("step_chunks.hip", {"ELMO_MB": 256, "ELMO_WF": 1}),   # 3M E4M3, B = 256
    ("step_chunks.hip", {"ELMO_MB": 256, "ELMO_WF": 2}),   # 3M MXFP4, B = 256
    ("step_chunks.hip", {"ELMO_MB": 256, "ELMO_WF": 0}),   # BF16 above 128 samples
    ("step_chunks.hip", {"ELMO_MB": 128, "ELMO_WF": 0}),   # 8.6M BF16, B = 128
    ("step_single.hip", {}),                               # single pass, B <= 32
]
# kernels on a timed path; the diagnostic forms (logits written out: ZOUT) and the long top-k
# lists are not
HOT = re.compile(r"k_bwd_update|k_step_single|k_fwd_(xs|xb|g|mx)I.*Lb0EEEv|k_dx_reduce|k_label_")


def _report(unit, tmp):
    src, defs = unit
    obj = os.path.join(tmp, src + "".join(f"_{k}{v}" for k, v in defs.items()) + ".o")
    cmd = [HIPCC, *B.HIPCC_FLAGS, *[f"-D{k}={v}" for k, v in defs.items()], "-I", INCLUDE, "-c",
           os.path.join(CSRC, src), "-o", obj, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, name = [], None
    for ln in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", ln)
        if m and name:
            out.append((name, int(m.group(1))))
    return out


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not installed")
def test_timed_step_kernels_use_no_scratch(tmp_path):
    with ThreadPoolExecutor(len(UNITS)) as ex:
        reports = list(ex.map(lambda u: _report(u, str(tmp_path)), UNITS))
    hot = [(n, s) for rep in reports for n, s in rep if HOT.search(n)]
    assert len(hot) >= 20, f"expected the step kernels in the reports, found {len(hot)}"
    spilled = [(n, s) for n, s in hot if s != 0]
    assert not spilled, f"step kernels using scratch: {spilled}"
