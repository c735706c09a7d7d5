"""CPU oracle for the ELMO classifier-head step (ctypes binding of ``elmo_oracle.c``).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP product path never imports it and shares no code
with it.

The C source follows the ELMO pages ("ELMO: Efficiency via Low-precision and Peak Memory Optimization
in Large Output Spaces": atlas.scime.ai summary, "Approach" and "Surprising findings"; arXiv
2510.11168 abstract). The readings it implements where the pages are silent are listed in the
C header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "elmo_oracle.c")
_LIB = os.path.join(_HERE, "libelmo_oracle.so")

W_BF16 = 0
W_E4M3 = 1
W_MXFP4 = 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE arithmetic: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        u8, u16, u32, u64, i32, i64 = (ctypes.c_uint8, ctypes.c_uint16, ctypes.c_uint32,
                                       ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64)
        P = ctypes.c_void_p
        L.orc_bf16_value.argtypes = [u16]; L.orc_bf16_value.restype = ctypes.c_double
        L.orc_bf16_rne.argtypes = [ctypes.c_float]; L.orc_bf16_rne.restype = u16
        L.orc_e4m3_value.argtypes = [u8]; L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_rne_sat.argtypes = [ctypes.c_double]; L.orc_e4m3_rne_sat.restype = u8
        L.orc_sr_bf16.argtypes = [ctypes.c_float, u32]; L.orc_sr_bf16.restype = u16
        L.orc_sr_e4m3.argtypes = [ctypes.c_float, u32]; L.orc_sr_e4m3.restype = u8
        L.orc_philox4x32.argtypes = [P, P, ctypes.c_int, P]; L.orc_philox4x32.restype = None
        L.orc_r16.argtypes = [u64, u64, u64]; L.orc_r16.restype = u32
        L.orc_grad_code.argtypes = [ctypes.c_float, ctypes.c_int]; L.orc_grad_code.restype = u16
        for name in ("orc_bf16_rne_array", "orc_e4m3_rne_sat_array"):
            getattr(L, name).argtypes = [P, P, i64]; getattr(L, name).restype = None
        for name in ("orc_sr_bf16_array", "orc_sr_e4m3_array"):
            getattr(L, name).argtypes = [P, P, P, i64]; getattr(L, name).restype = None
        L.orc_r16_array.argtypes = [u64, u64, u64, P, i64]; L.orc_r16_array.restype = None
        L.orc_step.argtypes = [ctypes.c_int, P, i64, ctypes.c_int, P, ctypes.c_int, P, P,
                               ctypes.c_float, u64, u64, P, P, P, P, ctypes.c_int]
        L.orc_update_from_g.argtypes = [ctypes.c_int, P, i64, ctypes.c_int, P, ctypes.c_int, P, ctypes.c_float,
                                        u64, u64, P, P, ctypes.c_int]
        L.orc_logits.argtypes = [ctypes.c_int, P, i64, ctypes.c_int, P, ctypes.c_int, P,
                                 ctypes.c_int, P, ctypes.c_int]
        L.orc_update_rows.argtypes = [ctypes.c_int, P, i64, ctypes.c_int, P, ctypes.c_int, P, P,
                                      ctypes.c_float, u64, u64, P, ctypes.c_int, P, P, P, ctypes.c_int]
        L.orc_update_rows_from_g.argtypes = [ctypes.c_int, P, i64, ctypes.c_int, P, ctypes.c_int, P,
                                             ctypes.c_float, u64, u64, P, ctypes.c_int, P, ctypes.c_int]
        L.orc_dx_rows.argtypes = [ctypes.c_int, P, i64, ctypes.c_int, P, ctypes.c_int, P, P, P,
                                  ctypes.c_int, P, ctypes.c_int]
        L.orc_grad_exact.argtypes = [i64, ctypes.c_int, ctypes.c_int, P, P, P, P, P, P, P, P]
        L.orc_kahan_update.argtypes = [i64, P, P, P, ctypes.c_float]; L.orc_kahan_update.restype = None
        L.orc_e2m1_value.argtypes = [u8]; L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [u8]; L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_sr_e2m1.argtypes = [ctypes.c_double, u32]; L.orc_sr_e2m1.restype = u8
        L.orc_mx_block_exponent.argtypes = [ctypes.c_float]; L.orc_mx_block_exponent.restype = ctypes.c_int
        L.orc_mx_quantize_block.argtypes = [P, P, P, P]; L.orc_mx_quantize_block.restype = None
        L.orc_mx_row_bytes.argtypes = [ctypes.c_int]; L.orc_mx_row_bytes.restype = i64
        L.orc_topk.argtypes = [ctypes.c_int, P, i64, ctypes.c_int, P, ctypes.c_int, ctypes.c_int,
                               P, P, ctypes.c_int]
        for name in ("orc_step", "orc_update_from_g", "orc_logits", "orc_update_rows", "orc_update_rows_from_g",
                     "orc_dx_rows", "orc_grad_exact",
                     "orc_topk"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _chk(rc, name):
    if rc != 0:
        raise RuntimeError(f"oracle {name} failed with status {rc}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def wdtype_np(wfmt):
    return np.uint16 if wfmt == W_BF16 else np.uint8


def dims(wfmt, W):
    """(L, D) of a weight array: [L][D] codes, or for MXFP4 [L][D/2 + D/32] bytes per row."""
    L, c = W.shape
    if wfmt == W_MXFP4:
        assert (c * 32) % 17 == 0, "MXFP4 rows hold D/2 + D/32 bytes"
        return L, c * 32 // 17
    return L, c


def row_units(wfmt, D):
    """array columns of one weight row: D codes, or D/2 + D/32 bytes for MXFP4"""
    return D // 2 + D // 32 if wfmt == W_MXFP4 else D


# ---- scalar / elementwise codecs ---------------------------------------------------------------

def bf16_value(codes):
    c = _c(codes, np.uint16)
    return np.array([lib().orc_bf16_value(int(v)) for v in c.ravel()]).reshape(c.shape)


def bf16_rne(x):
    x = _c(x, np.float32); out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_rne_array(_p(x), _p(out), x.size); return out


def e4m3_value(codes):
    c = _c(codes, np.uint8)
    return np.array([lib().orc_e4m3_value(int(v)) for v in c.ravel()]).reshape(c.shape)


def e4m3_rne_sat(x):
    x = _c(x, np.float64); out = np.empty(x.shape, np.uint8)
    lib().orc_e4m3_rne_sat_array(_p(x), _p(out), x.size); return out


def sr_bf16(t, r):
    t = _c(t, np.float32); r = _c(np.broadcast_to(r, t.shape), np.uint32)
    out = np.empty(t.shape, np.uint16); lib().orc_sr_bf16_array(_p(t), _p(r), _p(out), t.size)
    return out


def sr_e4m3(t, r):
    t = _c(t, np.float32); r = _c(np.broadcast_to(r, t.shape), np.uint32)
    out = np.empty(t.shape, np.uint8); lib().orc_sr_e4m3_array(_p(t), _p(r), _p(out), t.size)
    return out


def philox4x32(ctr, key, rounds=10):
    c = _c(ctr, np.uint32); k = _c(key, np.uint32); out = np.empty(4, np.uint32)
    lib().orc_philox4x32(_p(c), _p(k), rounds, _p(out)); return out


def r16(seed, step, idx0, n):
    out = np.empty(n, np.uint32); lib().orc_r16_array(seed, step, idx0, _p(out), n); return out


def grad_code(z, y):
    return lib().orc_grad_code(float(z), int(y))


def e2m1_value(codes):
    if np.ndim(codes) == 0:
        return lib().orc_e2m1_value(int(codes))
    c = _c(codes, np.uint8)
    return np.array([lib().orc_e2m1_value(int(v)) for v in c.ravel()]).reshape(c.shape)


def e8m0_value(codes):
    if np.ndim(codes) == 0:
        return lib().orc_e8m0_value(int(codes))
    c = _c(codes, np.uint8)
    return np.array([lib().orc_e8m0_value(int(v)) for v in c.ravel()]).reshape(c.shape)


def sr_e2m1(v, r):
    v = np.asarray(v, np.float64); r = np.broadcast_to(np.asarray(r, np.uint32), v.shape)
    return np.array([lib().orc_sr_e2m1(float(a), int(b)) for a, b in zip(v.ravel(), r.ravel())],
                    np.uint8).reshape(v.shape)


def mx_block_exponent(amax):
    return int(lib().orc_mx_block_exponent(float(amax)))


def mx_quantize_block(t, r):
    """32 FP32 values and their 16-bit draws -> (32 element codes, scale code)"""
    t = _c(np.asarray(t, np.float32).ravel(), np.float32); r = _c(np.asarray(r, np.uint32).ravel(), np.uint32)
    assert t.size == 32 and r.size == 32
    codes = np.empty(32, np.uint8); scale = np.empty(1, np.uint8)
    lib().orc_mx_quantize_block(_p(t), _p(r), _p(codes), _p(scale))
    return codes, int(scale[0])


def mx_decode(W, D=None):
    """binary64 values [L][D] of MXFP4 rows W [L][D/2 + D/32] (the oracle's element and scale decoders)"""
    W = _c(W, np.uint8)
    L, D = dims(W_MXFP4, W)
    e = _value_lut(W_MXFP4)
    sc = _scale_lut()
    codes = np.empty((L, D), np.uint8)
    codes[:, 0::2] = W[:, :D // 2] & 15
    codes[:, 1::2] = W[:, :D // 2] >> 4
    return e[codes] * np.repeat(sc[W[:, D // 2:]], 32, axis=1)


# ---- the step ----------------------------------------------------------------------------------

def step(wfmt, W, X, row_ptr, ids, lr, seed, step_, want_z=False, want_g=False, want_loss=False,
         nthreads=0):
    """Returns (W_new, dX, loss|None, Z|None, G|None); W is not modified."""
    Wn = np.array(W, dtype=wdtype_np(wfmt), order="C", copy=True)
    L, D = dims(wfmt, Wn)
    X = _c(X, np.uint16); B = X.shape[0]
    rp = _c(row_ptr, np.int32); ids = _c(ids, np.int32)
    dX = np.empty((B, D), np.float32)
    Z = np.empty((B, L), np.float32) if want_z else None
    G = np.empty((B, L), np.uint16) if want_g else None
    loss = ctypes.c_double(0.0)
    rc = lib().orc_step(wfmt, _p(Wn), L, D, _p(X), B, _p(rp), _p(ids) if ids.size else None,
                        float(lr), seed, step_, _p(dX),
                        ctypes.cast(ctypes.pointer(loss), ctypes.c_void_p) if want_loss else None,
                        _p(Z), _p(G), nthreads)
    _chk(rc, "step")
    return Wn, dX, (loss.value if want_loss else None), Z, G


def update_from_g(wfmt, W, X, G, lr, seed, step_, nthreads=0, want_t=False):
    """Updated codes given gradient codes G [B][L]; with want_t also the FP32 values t [L][D] that
    were stochastically rounded: returns W_new or (W_new, T)."""
    W = _c(W, wdtype_np(wfmt)); L, D = dims(wfmt, W); X = _c(X, np.uint16); B = X.shape[0]
    G = _c(G, np.uint16)
    assert G.shape == (B, L)
    out = np.empty_like(W)
    T = np.empty((L, D), np.float32) if want_t else None
    _chk(lib().orc_update_from_g(wfmt, _p(W), L, D, _p(X), B, _p(G), float(lr), seed, step_, _p(out), _p(T),
                                 nthreads), "update_from_g")
    return (out, T) if want_t else out


def logits(wfmt, W, X, js, nthreads=0):
    W = _c(W, wdtype_np(wfmt)); L, D = dims(wfmt, W); X = _c(X, np.uint16); B = X.shape[0]
    js = _c(js, np.int64); Z = np.empty((B, js.size), np.float32)
    _chk(lib().orc_logits(wfmt, _p(W), L, D, _p(X), B, _p(js), js.size, _p(Z), nthreads), "logits")
    return Z


def update_rows(wfmt, W, X, row_ptr, ids, lr, seed, step_, js, nthreads=0, want_detail=False):
    """Updated codes of weight rows js [nj][D]; with want_detail also their gradient codes G [B][nj]
    and the FP32 values t [nj][D] before rounding: returns Wrows or (Wrows, G, T)."""
    W = _c(W, wdtype_np(wfmt)); L, D = dims(wfmt, W); X = _c(X, np.uint16); B = X.shape[0]
    rp = _c(row_ptr, np.int32); ids = _c(ids, np.int32); js = _c(js, np.int64)
    out = np.empty((js.size, row_units(wfmt, D)), wdtype_np(wfmt))
    G = np.empty((B, js.size), np.uint16) if want_detail else None
    T = np.empty((js.size, D), np.float32) if want_detail else None
    _chk(lib().orc_update_rows(wfmt, _p(W), L, D, _p(X), B, _p(rp), _p(ids) if ids.size else None,
                               float(lr), seed, step_, _p(js), js.size, _p(out), _p(G), _p(T), nthreads),
         "update_rows")
    return (out, G, T) if want_detail else out


def update_rows_from_g(wfmt, W, X, G, lr, seed, step_, js, nthreads=0):
    """Updated codes of weight rows js given the gradient codes G [B][len(js)] of those labels."""
    W = _c(W, wdtype_np(wfmt)); L, D = dims(wfmt, W); X = _c(X, np.uint16); B = X.shape[0]
    js = _c(js, np.int64); G = _c(G, np.uint16)
    assert G.shape == (B, js.size)
    out = np.empty((js.size, row_units(wfmt, D)), wdtype_np(wfmt))
    _chk(lib().orc_update_rows_from_g(wfmt, _p(W), L, D, _p(X), B, _p(G), float(lr), seed, step_, _p(js), js.size,
                                      _p(out), nthreads), "update_rows_from_g")
    return out


def dx_rows(wfmt, W, X, row_ptr, ids, bs, nthreads=0):
    W = _c(W, wdtype_np(wfmt)); L, D = dims(wfmt, W); X = _c(X, np.uint16); B = X.shape[0]
    rp = _c(row_ptr, np.int32); ids = _c(ids, np.int32); bs = _c(bs, np.int32)
    out = np.empty((bs.size, D), np.float32)
    _chk(lib().orc_dx_rows(wfmt, _p(W), L, D, _p(X), B, _p(rp), _p(ids) if ids.size else None,
                           _p(bs), bs.size, _p(out), nthreads), "dx_rows")
    return out


def grad_exact(W, X, Y):
    W = _c(W, np.float64); X = _c(X, np.float64); Y = _c(Y, np.float64)
    L, D = W.shape; B = X.shape[0]
    Z = np.empty((B, L)); G = np.empty((B, L)); dX = np.empty((B, D)); dW = np.empty((L, D))
    loss = ctypes.c_double(0.0)
    _chk(lib().orc_grad_exact(L, D, B, _p(W), _p(X), _p(Y), _p(Z), _p(G), _p(dX), _p(dW),
                              ctypes.cast(ctypes.pointer(loss), ctypes.c_void_p)), "grad_exact")
    return Z, G, dX, dW, loss.value


# ---- all-label logits and ranking for many queries at full size -------------------------------

_LUT = {}


def _value_lut(wfmt):
    """Decoded value of every code, from the oracle's own decoders (65,536 BF16, 256 E4M3 or 16 E2M1
    codes)."""
    if wfmt not in _LUT:
        if wfmt == W_BF16:
            _LUT[wfmt] = bf16_value(np.arange(65536, dtype=np.uint16))
        elif wfmt == W_E4M3:
            _LUT[wfmt] = e4m3_value(np.arange(256, dtype=np.uint8))
        else:
            _LUT[wfmt] = e2m1_value(np.arange(16, dtype=np.uint8))
    return _LUT[wfmt]


def _scale_lut():
    if "e8m0" not in _LUT:
        _LUT["e8m0"] = e8m0_value(np.arange(256, dtype=np.uint8))
    return _LUT["e8m0"]


def forward_x_values(wfmt, X):
    """The forward operand of queries X (BF16 codes) as binary64 values: X itself for BF16 weights,
    E4M3-RNE(X) for E4M3 weights (the training forward's cast)."""
    xv = _value_lut(W_BF16)[_c(X, np.uint16)]
    if wfmt in (W_E4M3, W_MXFP4):
        xv = _value_lut(W_E4M3)[e4m3_rne_sat(xv)]
    return xv


def logits_dense(wfmt, W, X, block=1 << 16):
    """FP32 logits of queries X [N][D] against every label of W [L][D]: the same definition as
    orc_logits (z = FP32 of the binary64 sum of the exact products x~_k w_jk), with the sums taken by
    numpy's binary64 matrix product (a library routine) over blocks of labels instead of a loop. It
    differs from orc_logits only in the order of the binary64 additions, which can move z across an
    FP32 rounding boundary only when the sum lies within ~D 2^-53 of it (pinned against orc_logits).
    Returns Z [N][L] float32."""
    W = np.ascontiguousarray(W)
    L = W.shape[0]
    xv = forward_x_values(wfmt, X)
    Z = np.empty((xv.shape[0], L), np.float32)
    for j0 in range(0, L, block):
        j1 = min(L, j0 + block)
        wv = mx_decode(W[j0:j1]) if wfmt == W_MXFP4 else _value_lut(wfmt)[W[j0:j1]]
        Z[:, j0:j1] = (xv @ wv.T).astype(np.float32)
    return Z


def rank_scores(Z, k):
    """Top-k of each row of the score matrix Z [N][L] under the order (score desc, label asc, NaN
    after every number): candidates are the labels whose score is at least the row's k-th largest
    (NaN counted as -inf), ranked by numpy's lexsort. Returns idx [N][k] int32, score [N][k] float32."""
    Z = np.asarray(Z, np.float32)
    N, L = Z.shape
    idx = np.empty((N, k), np.int32)
    sc = np.empty((N, k), np.float32)
    for n in range(N):
        s = Z[n]
        nan = np.isnan(s)
        key = np.where(nan, -np.inf, s)
        vk = np.partition(key, L - k)[L - k]
        cand = np.nonzero(key >= vk)[0]
        order = np.lexsort((cand, nan[cand], -key[cand]))[:k]
        idx[n] = cand[order]
        sc[n] = s[cand[order]]
    return idx, sc


def topk(wfmt, W, X, k, nthreads=0):
    W = _c(W, wdtype_np(wfmt)); L, D = dims(wfmt, W); X = _c(X, np.uint16); N = X.shape[0]
    idx = np.empty((N, k), np.int32); score = np.empty((N, k), np.float32)
    _chk(lib().orc_topk(wfmt, _p(W), L, D, _p(X), N, k, _p(idx), _p(score), nthreads), "topk")
    return idx, score


def kahan_update(w, c, g, lr):
    """One Kahan-compensated BF16 update of parameters w with compensation c (uint16 BF16 codes)
    by gradient g (float32); returns the new (w, c)."""
    w = np.array(w, np.uint16, copy=True).ravel(); c = np.array(c, np.uint16, copy=True).ravel()
    g = _c(np.asarray(g, np.float32).ravel(), np.float32)
    assert w.size == c.size == g.size
    lib().orc_kahan_update(w.size, _p(w), _p(c), _p(g), float(lr))
    return w, c
