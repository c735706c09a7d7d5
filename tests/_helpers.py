"""Comparison helpers shared by the GPU parity tests (tolerances follow the stated bar:
logits and dX within 1e-2 relative for BF16 weights and 6e-2 for E4M3 weights, with an RMS floor;
updated weights >= 99.9% bit-equal and every other element within one unit of the storage format)."""
import numpy as np
import torch

import workloads as wk

RTOL = {wk.W_BF16: 1e-2, wk.W_E4M3: 6e-2}


def signed_code(codes, wfmt):
    c = codes.astype(np.int64)
    if wfmt == wk.W_BF16:
        return np.where(c & 0x8000, -(c & 0x7FFF), c & 0x7FFF)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def is_nan_code(codes, wfmt):
    c = codes.astype(np.int64)
    if wfmt == wk.W_BF16:
        return ((c & 0x7F80) == 0x7F80) & ((c & 0x7F) != 0)
    return (c & 0x7F) == 0x7F


def weight_report(got, ref, wfmt):
    """(fraction bit-equal with +-0 equal, max code distance, NaN count)"""
    d = np.abs(signed_code(got, wfmt) - signed_code(ref, wfmt))
    return float((d == 0).mean()), int(d.max()) if d.size else 0, int(is_nan_code(got, wfmt).sum())


def code_value(codes, wfmt):
    if wfmt == wk.W_BF16:
        return torch.from_numpy(np.ascontiguousarray(codes, np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def update_error_bound(G, X, lr, B):
    """Elementwise bound on |t_device - t_oracle| from the device's FP32 accumulation of
    dW = sum_b g_b x_b over B terms (standard recursive-summation bound gamma_B * sum |g_b x_b|,
    gamma_n = n u / (1 - n u), u = 2^-24), times lr, doubled for safety."""
    u = 2.0 ** -24
    gam = B * u / (1 - B * u)
    S = np.abs(code_value(G, wk.W_BF16)).T @ np.abs(code_value(X, wk.W_BF16))   # [L, D]
    return 2.0 * abs(float(np.float32(lr))) * gam * S


def assert_weights_match(got, ref, wfmt, min_equal=0.999, abs_bound=None):
    """>= min_equal bit-equal (+-0 equal); every other element within one code of the storage
    format, or, where the format's spacing is finer than the FP32 arithmetic's own error bound on
    the update (weights next to zero), within that bound."""
    d = np.abs(signed_code(got, wfmt) - signed_code(ref, wfmt))
    eq = float((d == 0).mean())
    nan = int(is_nan_code(got, wfmt).sum())
    assert nan == 0, f"{nan} NaN weight codes"
    ok = d <= 1
    if abs_bound is not None and not ok.all():
        bad = ~ok
        vg, vr = code_value(got[bad], wfmt), code_value(ref[bad], wfmt)
        ok[bad] = np.abs(vg - vr) <= abs_bound[bad]
    assert ok.all(), f"{int((~ok).sum())} weights off by more than one code (max {d.max()}), equal {eq:.6f}"
    assert eq >= min_equal, f"only {eq:.6f} of weights bit-equal"
    return eq


def assert_grad_codes_match(got, ref, max_rate=1e-3):
    """BF16 gradient codes: each within one unit, at most `max_rate` of them different."""
    d = np.abs(signed_code(got, wk.W_BF16) - signed_code(ref, wk.W_BF16))
    assert d.max() <= 1, f"gradient code distance {d.max()}"
    rate = float((d != 0).mean())
    assert rate <= max_rate, f"gradient code flip rate {rate:.2e}"
    return rate


def rel_err(got, ref):
    got = np.asarray(got, np.float64); ref = np.asarray(ref, np.float64)
    floor = np.sqrt((ref ** 2).mean()) if ref.size else 1.0
    return np.abs(got - ref) / np.maximum(np.abs(ref), max(floor, 1e-30))


def assert_close(got, ref, rtol):
    e = rel_err(got, ref)
    assert np.all(np.isfinite(got)), "non-finite values"
    assert e.max() <= rtol, f"max relative error {e.max():.3e} > {rtol}"
    return float(e.max())


def to_dev_codes(W, dev="cuda"):
    if W.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(W).view(np.int16)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(W)).to(dev)


def from_dev_codes(t):
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def batch_to_dev(bt, dev="cuda"):
    X = torch.from_numpy(np.ascontiguousarray(bt.X).view(np.int16)).to(dev)
    rp = torch.from_numpy(np.ascontiguousarray(bt.row_ptr, np.int32)).to(dev)
    ids = torch.from_numpy(np.ascontiguousarray(bt.ids, np.int32)).to(dev)
    return X, rp, ids
