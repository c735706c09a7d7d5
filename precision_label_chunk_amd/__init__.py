"""Python binding of libelmo_xmc (the MI355X XMC classifier-head step and top-k scoring).

Argument marshalling only: every step of the computation runs in the HIP kernels behind the C ABI
declared in include/elmo_xmc.h. PyTorch supplies device memory and the current stream.

    import precision_label_chunk_amd as elmo
    dX, loss = elmo.step(W, X, row_ptr, ids, lr=0.05, seed=0, step=0, chunk=32768, want_loss=True)
    idx, score = elmo.topk(W, X_eval, k=5)

W: [L, D] torch tensor of weight codes on the GPU, updated in place: int16/uint16/bfloat16 for
BF16 weights, uint8/float8_e4m3fn for OCP E4M3 weights; MX-scaled FP4 weights are uint8 rows of
D/2 code bytes and D/32 scale bytes ([L, 17 D / 32]) and need wfmt=ELMO_W_MXFP4. X: [B, D] BF16
codes (int16/uint16/bfloat16). row_ptr/ids: int32 CSR positive labels on the GPU.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libelmo_xmc.so")

ELMO_W_BF16 = 0
ELMO_W_E4M3 = 1
ELMO_W_MXFP4 = 2
FLAG_LABEL_RANGE = 1
FLAG_ROW_PTR = 2

_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape", -3: "unknown weight format",
           -4: "workspace missing or too small", -5: "HIP runtime error", -6: "not supported",
           -7: "step too large for the allocation-free entry point's static scratch"}


class ElmoError(RuntimeError):
    def __init__(self, name, status):
        super().__init__(f"{name} failed: {_STATUS.get(status, status)} ({status})")
        self.status = status


_lib = None
last_workspace = None    # workspace of the latest step() call (its first word holds the flags)


def lib():
    """The loaded HIP library. Raises if it has not been built: there is no fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is missing; build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, u64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                                     ctypes.c_float, ctypes.c_size_t)
        L.elmo_abi_version.restype = i32
        L.elmo_status_str.argtypes = [i32]; L.elmo_status_str.restype = ctypes.c_char_p
        L.elmo_xmc_step_workspace_bytes.argtypes = [i32, i32, i64, i64, i32, i64]
        L.elmo_xmc_step_workspace_bytes.restype = sz
        L.elmo_xmc_step.argtypes = [P, i32, i64, i32, P, i32, P, P, i64, f32, u64, u64, i64, P, P, P, sz, P]
        L.elmo_xmc_step.restype = i32
        L.elmo_xmc_step_two_kernel.argtypes = L.elmo_xmc_step.argtypes
        L.elmo_xmc_step_two_kernel.restype = i32
        L.elmo_xmc_step_single_pass.argtypes = [P, i32, i64, i32, P, i32, P, P, i64, f32, u64, u64, i64, P, P, P,
                                                P, sz, P]
        L.elmo_xmc_step_single_pass.restype = i32
        L.elmo_xmc_step_flags.argtypes = [P, P, P]; L.elmo_xmc_step_flags.restype = i32
        L.elmo_xmc_step_noalloc.argtypes = [P, i32, i64, i32, P, i32, P, P, i64, f32, u64, u64, i64, P, P, P]
        L.elmo_xmc_step_noalloc.restype = i32
        L.elmo_xmc_topk_workspace_bytes.argtypes = [i32, i32, i64, i32, i32]
        L.elmo_xmc_topk_workspace_bytes.restype = sz
        L.elmo_xmc_topk.argtypes = [P, i32, i64, i32, P, i32, i32, P, P, P, sz, P]
        L.elmo_xmc_topk.restype = i32
        L.elmo_xmc_logits.argtypes = [P, i32, i64, i32, i64, i64, P, i32, P, P, sz, P]
        L.elmo_xmc_logits.restype = i32
        L.elmo_xmc_forward.argtypes = [P, i32, i64, i32, P, i32, P, P, i64, i64, i64, P, P, P, sz, P]
        L.elmo_xmc_forward.restype = i32
        L.elmo_xmc_kernel_timing.argtypes = [i32]; L.elmo_xmc_kernel_timing.restype = i32
        L.elmo_xmc_kernel_timing_read.argtypes = [P, P, P]; L.elmo_xmc_kernel_timing_read.restype = i32
        L.elmo_numerics_probe.argtypes = [i32, P, P, P, i64, u64, u64, P]
        L.elmo_numerics_probe.restype = i32
        L.elmo_kahan_update.argtypes = [P, P, P, i64, f32, P]; L.elmo_kahan_update.restype = i32
        _lib = L
    return _lib


def _chk(name, rc):
    if rc != 0:
        raise ElmoError(name, rc)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def wdtype_of(W: torch.Tensor) -> int:
    if W.dtype in (torch.int16, torch.uint16, torch.bfloat16):
        return ELMO_W_BF16
    if W.dtype in (torch.uint8, torch.float8_e4m3fn):
        return ELMO_W_E4M3
    raise TypeError(f"unsupported weight dtype {W.dtype}")


def _wdims(W: torch.Tensor, wfmt):
    """(format, L, D) of a weight tensor: by dtype, or MXFP4 rows of 17 D / 32 bytes when asked."""
    if wfmt is None or wfmt != ELMO_W_MXFP4:
        wd = wdtype_of(W)
        if wfmt is not None and wfmt != wd:
            raise TypeError(f"weight dtype {W.dtype} does not hold format {wfmt}")
        return wd, W.shape[0], W.shape[1]
    if W.dtype != torch.uint8 or W.dim() != 2 or (W.shape[1] * 32) % 17:
        raise TypeError("MXFP4 weights are uint8 rows of D/2 code bytes and D/32 scale bytes")
    return ELMO_W_MXFP4, W.shape[0], W.shape[1] * 32 // 17


def _check_dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous CUDA tensors")


def step_workspace_bytes(B, D, L, chunk, wdtype, max_nnz):
    return int(lib().elmo_xmc_step_workspace_bytes(B, D, L, chunk, wdtype, max_nnz))


def step(W, X, row_ptr, ids, lr, seed, step, chunk, want_loss=False, dX=None, workspace=None, wfmt=None,
         single_pass=None, g_out=None):
    """One fused training step; W is updated in place. Returns (dX [B, D] float32, loss tensor|None).
    single_pass=None calls elmo_xmc_step (the faster path for the shape), False
    elmo_xmc_step_two_kernel, True elmo_xmc_step_single_pass (B <= 32, D in 256/512/768); g_out (an
    int16 [B, L] device tensor) then receives the gradient codes it used."""
    _check_dev(W, X, row_ptr, ids)
    wd, L, D = _wdims(W, wfmt)
    B = X.shape[0]
    nnz = int(ids.numel())
    if dX is None:
        dX = torch.empty((B, D), dtype=torch.float32, device=W.device)
    loss = torch.empty((1,), dtype=torch.float32, device=W.device) if want_loss else None
    need = step_workspace_bytes(B, D, L, chunk, wd, nnz)
    if need == 0:
        raise ElmoError("elmo_xmc_step_workspace_bytes", -2)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=W.device)
    if single_pass:
        name = "elmo_xmc_step_single_pass"
        if g_out is not None:
            _check_dev(g_out)
            if g_out.dtype != torch.int16 or tuple(g_out.shape) != (B, L):
                raise ValueError("g_out must be an int16 [B, L] device tensor")
        rc = lib().elmo_xmc_step_single_pass(_ptr(W), wd, L, D, _ptr(X), B, _ptr(row_ptr),
                                             _ptr(ids) if nnz else None, nnz, float(lr), int(seed), int(step),
                                             int(chunk), _ptr(dX), _ptr(loss), _ptr(g_out), _ptr(workspace),
                                             workspace.numel(), _stream())
    else:
        if g_out is not None:
            raise ValueError("g_out is a diagnostic of the single-pass step")
        name = "elmo_xmc_step" if single_pass is None else "elmo_xmc_step_two_kernel"
        rc = getattr(lib(), name)(_ptr(W), wd, L, D, _ptr(X), B, _ptr(row_ptr), _ptr(ids) if nnz else None,
                                  nnz, float(lr), int(seed), int(step), int(chunk), _ptr(dX), _ptr(loss),
                                  _ptr(workspace), workspace.numel(), _stream())
    _chk(name, rc)
    global last_workspace
    last_workspace = workspace
    return dX, loss


def step_noalloc(W, X, row_ptr, ids, lr, seed, step, chunk, dX, loss=None, wfmt=None):
    """The same step through the allocation-free entry point (static scratch inside the library):
    dX [B, D] float32 and the optional loss [1] float32 are caller-allocated outputs."""
    _check_dev(W, X, row_ptr, ids, dX, loss)
    wd, L, D = _wdims(W, wfmt)
    B = X.shape[0]
    nnz = int(ids.numel())
    rc = lib().elmo_xmc_step_noalloc(_ptr(W), wd, L, D, _ptr(X), B, _ptr(row_ptr), _ptr(ids) if nnz else None,
                                     nnz, float(lr), int(seed), int(step), int(chunk), _ptr(dX), _ptr(loss), _stream())
    _chk("elmo_xmc_step_noalloc", rc)
    return dX, loss


def step_flags(workspace) -> int:
    out = ctypes.c_uint32(0)
    _chk("elmo_xmc_step_flags", lib().elmo_xmc_step_flags(_ptr(workspace), ctypes.byref(out), _stream()))
    return int(out.value)


def topk_workspace_bytes(N, D, L, k, wdtype):
    return int(lib().elmo_xmc_topk_workspace_bytes(N, D, L, k, wdtype))


def topk(W, X, k, workspace=None, want_score=True, wfmt=None):
    """Top-k labels per row of X by FP32 logit (ties to the smaller label). Returns (idx, score)."""
    _check_dev(W, X)
    wd, L, D = _wdims(W, wfmt)
    N = X.shape[0]
    idx = torch.empty((N, k), dtype=torch.int32, device=W.device)
    score = torch.empty((N, k), dtype=torch.float32, device=W.device) if want_score else None
    need = topk_workspace_bytes(N, D, L, k, wd)
    if need == 0:
        raise ElmoError("elmo_xmc_topk_workspace_bytes", -2)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=W.device)
    _chk("elmo_xmc_topk", lib().elmo_xmc_topk(_ptr(W), wd, L, D, _ptr(X), N, k, _ptr(idx), _ptr(score),
                                              _ptr(workspace), workspace.numel(), _stream()))
    return idx, score


def logits(W, X, l0, l1, wfmt=None):
    """FP32 logits [B, l1 - l0] from the step's forward kernel (diagnostic)."""
    _check_dev(W, X)
    wd, L, D = _wdims(W, wfmt)
    B = X.shape[0]
    Z = torch.empty((B, l1 - l0), dtype=torch.float32, device=W.device)
    need = step_workspace_bytes(B, D, L, l1 - l0, wd, 0)
    ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=W.device)
    _chk("elmo_xmc_logits", lib().elmo_xmc_logits(_ptr(W), wd, L, D, l0, l1, _ptr(X), B, _ptr(Z), _ptr(ws),
                                                  ws.numel(), _stream()))
    return Z


def forward(W, X, row_ptr, ids, l0, l1, want_z=True, want_g=True, wfmt=None):
    """The step's forward kernel over labels [l0, l1): (Z float32 | None, G int16 BF16 codes | None),
    each [B, l1 - l0]. Weights are not modified (diagnostic)."""
    _check_dev(W, X, row_ptr, ids)
    wd, L, D = _wdims(W, wfmt)
    B = X.shape[0]
    nnz = int(ids.numel()) if ids is not None else 0
    Z = torch.empty((B, l1 - l0), dtype=torch.float32, device=W.device) if want_z else None
    G = torch.empty((B, l1 - l0), dtype=torch.int16, device=W.device) if want_g else None
    need = step_workspace_bytes(B, D, L, l1 - l0, wd, nnz)
    ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=W.device)
    _chk("elmo_xmc_forward", lib().elmo_xmc_forward(_ptr(W), wd, L, D, _ptr(X), B, _ptr(row_ptr),
                                                    _ptr(ids) if nnz else None, nnz, l0, l1, _ptr(Z), _ptr(G),
                                                    _ptr(ws), ws.numel(), _stream()))
    return Z, G


def kernel_timing(enable: bool):
    """Bracket each forward / backward kernel launch of later steps with HIP events."""
    _chk("elmo_xmc_kernel_timing", lib().elmo_xmc_kernel_timing(1 if enable else 0))


def kernel_timing_read():
    """{'fwd': (ms, launches, labels), 'bwd': (...)} summed since the last read (synchronises)."""
    ms = (ctypes.c_double * 2)(); n = (ctypes.c_int64 * 2)(); lab = (ctypes.c_double * 2)()
    _chk("elmo_xmc_kernel_timing_read", lib().elmo_xmc_kernel_timing_read(ms, n, lab))
    return {"fwd": (ms[0], n[0], lab[0]), "bwd": (ms[1], n[1], lab[1])}


def kahan_update(w, c, g, lr):
    """Kahan-compensated BF16 update of encoder parameters in place: w, c (int16 tensors of BF16
    codes) and g (float32), same number of elements, on the GPU (see elmo_xmc.h)."""
    _check_dev(w, c, g)
    assert w.dtype == torch.int16 and c.dtype == torch.int16 and g.dtype == torch.float32
    assert w.is_contiguous() and c.is_contiguous() and g.is_contiguous()
    n = w.numel()
    assert c.numel() == n and g.numel() == n
    _chk("elmo_kahan_update", lib().elmo_kahan_update(_ptr(w), _ptr(c), _ptr(g), n, float(lr), _stream()))
    return w, c


def numerics_probe(op, in0=None, in1=None, n=None, seed=0, step=0, idx0=0):
    """Device codec / SR / RNG / gradient applied elementwise (test hook; see elmo_xmc.h)."""
    out_dtype = {0: torch.int16, 1: torch.uint8, 2: torch.float32, 3: torch.int16, 4: torch.uint8,
                 5: torch.int32, 6: torch.int16, 7: torch.int32, 8: torch.float32, 9: torch.float32,
                 10: torch.uint8, 11: torch.uint8, 12: torch.int32, 13: torch.float32, 14: torch.int32}[op]
    if n is None:
        n = {11: in0.numel() // 32, 13: 1, 14: in0.numel() // 2}.get(op, in0.numel())
    dev = in0.device if in0 is not None else torch.device("cuda")
    size = {7: 2 * n, 11: 33 * n, 12: 4 * n, 13: 1024}.get(op, n)
    out = torch.empty((size,), dtype=out_dtype, device=dev)
    if op == 5:
        host = ctypes.c_uint64(idx0)
        rc = lib().elmo_numerics_probe(op, ctypes.cast(ctypes.byref(host), ctypes.c_void_p), None, _ptr(out), n,
                                       int(seed), int(step), _stream())
    else:
        _check_dev(in0, in1)
        rc = lib().elmo_numerics_probe(op, _ptr(in0), _ptr(in1), _ptr(out), n, int(seed), int(step), _stream())
    _chk("elmo_numerics_probe", rc)
    return out
