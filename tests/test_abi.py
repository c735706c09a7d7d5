"""The C-ABI library loads and exports every entry point that include/elmo_xmc.h declares, and
rejects invalid arguments on the host (no GPU needed: validation happens before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "elmo_xmc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(elmo_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    import precision_label_chunk_amd as elmo
    if not os.path.exists(elmo.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return elmo.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["elmo_xmc_step", "elmo_xmc_topk", "elmo_xmc_step_workspace_bytes", "elmo_xmc_topk_workspace_bytes",
              "elmo_xmc_logits", "elmo_numerics_probe", "elmo_status_str", "elmo_abi_version", "elmo_xmc_step_flags",
              "elmo_kahan_update", "elmo_xmc_step_single_pass", "elmo_xmc_step_two_kernel"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), f"missing export {n}"


def test_status_strings_and_version(L):
    assert L.elmo_abi_version() == 1
    assert L.elmo_status_str(0) == b"ok"
    assert L.elmo_status_str(-4).startswith(b"workspace")


@pytest.mark.parametrize("B,D,Lab,chunk,wd", [(0, 768, 1000, 128, 0), (257, 768, 1000, 128, 0), (4, 96, 1000, 128, 0),
                                              (4, 2048, 1000, 128, 0), (4, 768, 0, 128, 0), (4, 768, 1000, 0, 0),
                                              (4, 768, 1000, 128, 7), (4, 768, 2**31, 128, 0),
                                              (4, 192, 1000, 128, 2), (4, 640, 1000, 128, 2)])   # MXFP4: D % 256
def test_workspace_query_rejects_bad_shapes(L, B, D, Lab, chunk, wd):
    assert L.elmo_xmc_step_workspace_bytes(B, D, Lab, chunk, wd, 10) == 0


def test_step_rejects_invalid_arguments_before_launch(L):
    null = None
    # unknown format
    assert L.elmo_xmc_step(null, 5, 1000, 768, null, 4, null, null, 0, 0.1, 0, 0, 128, null, null, null, 0, null) == -3
    # bad shapes
    assert L.elmo_xmc_step(null, 0, 1000, 100, null, 4, null, null, 0, 0.1, 0, 0, 128, null, null, null, 0, null) == -2
    # null pointers
    assert L.elmo_xmc_step(null, 0, 1000, 128, null, 4, null, null, 0, 0.1, 0, 0, 128, null, null, null, 0, null) == -1
    # non-finite learning rate
    p = ctypes.c_void_p(4096)
    assert L.elmo_xmc_step(p, 0, 1000, 128, p, 4, p, p, 1, float("nan"), 0, 0, 128, p, null, p, 1 << 30, null) == -1
    # misaligned pointer
    q = ctypes.c_void_p(4097)
    assert L.elmo_xmc_step(q, 0, 1000, 128, p, 4, p, p, 1, 0.1, 0, 0, 128, p, null, p, 1 << 30, null) == -1
    # workspace too small (validation precedes any device work)
    assert L.elmo_xmc_step(p, 0, 1000, 128, p, 4, p, p, 1, 0.1, 0, 0, 128, p, null, p, 16, null) == -4
    # MXFP4 rows need D % 256 == 0
    assert L.elmo_xmc_step(p, 2, 1000, 192, p, 4, p, p, 1, 0.1, 0, 0, 128, p, null, p, 1 << 30, null) == -2
    assert L.elmo_xmc_step_workspace_bytes(4, 256, 1000, 128, 2, 10) > 0


def test_topk_rejects_invalid_arguments(L):
    null = None
    assert L.elmo_xmc_topk(null, 0, 1000, 128, null, 4, 0, null, null, null, 0, null) == -2
    assert L.elmo_xmc_topk(null, 0, 1000, 128, null, 4, 65, null, null, null, 0, null) == -2      # k > 64
    assert L.elmo_xmc_topk(null, 0, 10, 128, null, 4, 11, null, null, null, 0, null) == -2
    assert L.elmo_xmc_topk(null, 0, 1000, 128, null, 4, 5, null, null, null, 0, null) == -1
    assert L.elmo_xmc_topk_workspace_bytes(4, 128, 1000, 0, 0) == 0
    assert L.elmo_xmc_topk_workspace_bytes(4, 128, 1000, 5, 2) == 0       # MXFP4 with D % 256 != 0
    assert L.elmo_xmc_topk(null, 2, 1000, 128, null, 4, 5, null, null, null, 0, null) == -2


def test_numerics_probe_rejects_bad_op(L):
    assert L.elmo_numerics_probe(10, None, None, ctypes.c_void_p(4096), 1, 0, 0, None) == -1
    assert L.elmo_numerics_probe(8, ctypes.c_void_p(4096), None, ctypes.c_void_p(4096), 1, 0, 0, None) == -1
    assert L.elmo_numerics_probe(3, ctypes.c_void_p(4096), None, ctypes.c_void_p(4096), 1, 0, 0, None) == -1


def test_kahan_update_rejects_invalid_arguments(L):
    L.elmo_kahan_update.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_float, ctypes.c_void_p]
    p = ctypes.c_void_p(4096)
    assert L.elmo_kahan_update(p, p, p, -1, 0.1, None) == -2
    assert L.elmo_kahan_update(None, None, None, 0, 0.1, None) == 0          # empty: nothing to do
    assert L.elmo_kahan_update(None, p, p, 8, 0.1, None) == -1
    assert L.elmo_kahan_update(p, p, ctypes.c_void_p(4098), 8, 0.1, None) == -1   # misaligned g
    assert L.elmo_kahan_update(ctypes.c_void_p(4097), p, p, 8, 0.1, None) == -1   # misaligned w


def test_single_pass_step_rejects_shapes_it_does_not_build(L):
    null = None
    p = ctypes.c_void_p(4096)
    f = L.elmo_xmc_step_single_pass
    f.restype = ctypes.c_int
    # the same host validation as elmo_xmc_step
    assert f(null, 5, 1000, 768, null, 4, null, null, 0, 0.1, 0, 0, 128, null, null, null, null, 0, null) == -3
    assert f(null, 0, 1000, 100, null, 4, null, null, 0, 0.1, 0, 0, 128, null, null, null, null, 0, null) == -2
    assert f(p, 0, 1000, 768, p, 4, p, p, 1, float("nan"), 0, 0, 128, p, null, null, p, 1 << 30, null) == -1
    # built for B <= 32 and D in {256, 512, 768} only: other valid shapes are unsupported, nothing runs
    assert f(p, 0, 1000, 768, p, 33, p, p, 1, 0.1, 0, 0, 128, p, null, null, p, 1 << 30, null) == -6
    assert f(p, 1, 1000, 640, p, 8, p, p, 1, 0.1, 0, 0, 128, p, null, null, p, 1 << 30, null) == -6
    assert f(p, 0, 1000, 1024, p, 8, p, p, 1, 0.1, 0, 0, 128, p, null, null, p, 1 << 30, null) == -6
    # workspace too small for a supported shape; a misaligned gradient-code output
    assert f(p, 0, 1000, 768, p, 32, p, p, 1, 0.1, 0, 0, 128, p, null, null, p, 16, null) == -4
    assert f(p, 0, 1000, 768, p, 32, p, p, 1, 0.1, 0, 0, 128, p, null, ctypes.c_void_p(4097), p, 1 << 30,
             null) == -1


def test_workspace_holds_the_single_pass_partials():
    """At padded batch 32 and D = 768 the workspace has room for one dX partial (32 x 768 FP32) per
    single-pass work-group, up to one per CU (or per 32-label tile of the chunk, if fewer)."""
    import precision_label_chunk_amd as elmo
    small = elmo.step_workspace_bytes(32, 768, 4096, 1024, 0, 100)
    big = elmo.step_workspace_bytes(32, 768, 8_600_000, 262_144, 0, 100)
    assert small >= 32 * (32 * 768 * 4)
    assert big >= 256 * (32 * 768 * 4)


def test_two_kernel_step_validates_like_the_step(L):
    null = None
    p = ctypes.c_void_p(4096)
    f = L.elmo_xmc_step_two_kernel
    assert f(null, 5, 1000, 768, null, 4, null, null, 0, 0.1, 0, 0, 128, null, null, null, 0, null) == -3
    assert f(null, 0, 1000, 100, null, 4, null, null, 0, 0.1, 0, 0, 128, null, null, null, 0, null) == -2
    assert f(p, 0, 1000, 768, p, 4, p, p, 1, float("nan"), 0, 0, 128, p, null, p, 1 << 30, null) == -1
    assert f(p, 0, 1000, 768, p, 32, p, p, 1, 0.1, 0, 0, 128, p, null, p, 16, null) == -4
