"""Comparison helpers shared by the GPU parity tests (tolerances follow the stated bar:
logits and dX within 1e-2 relative for BF16 weights and 6e-2 for E4M3 and MXFP4 weights, with an RMS floor;
updated weights >= 99.9% bit-equal and every other element within one unit of the storage format,
or explained by a named, bounded difference of the FP32 arithmetic before the rounding; top-k
indices exact where the ranking is decided by more than the measured logit error)."""
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


def _outward_f32(v64, direction):
    """binary32 value nearest v64 on the side `direction` (-1: <= v64, +1: >= v64)."""
    f = v64.astype(np.float32)
    if direction < 0:
        return np.where(f.astype(np.float64) > v64, np.nextafter(f, np.float32(-np.inf)), f)
    return np.where(f.astype(np.float64) < v64, np.nextafter(f, np.float32(np.inf)), f)


def classify_weights(orc, Wg, Wr, T, R, wfmt, X, Gg, Gr, lr):
    """Sort the device's updated weights Wg [n][D] against the oracle's own (free-running) step Wr
    for the same n labels. T [n][D]: the oracle's FP32 values t before the stochastic rounding;
    R [n][D]: the elements' 16-bit draws; Gg, Gr [B][n]: the device's and the oracle's BF16 gradient
    codes of those labels; X [B][D] the features.

    Stochastic rounding with a fixed draw is monotone in t, so a device t within D of the oracle's t
    can only give a code in [SR(t - D), SR(t + D)] (both ends from the oracle's rounding). Classes of
    the elements that are not bit-equal, in order:
      a  one code away (the stated bar);
      b  in a label row whose gradient codes differ from the oracle's (a BF16 rounding of
         sigmoid(z) - y decided the other way by the FP32 logit and sigmoid, about one FP32 unit from
         the binary64 value), inside [SR(t - D_b), SR(t + D_b)] with
         D_b = lr sum_b |g_dev - g_orc| |x_bk| + D_c;
      c  inside [SR(t - D_c), SR(t + D_c)] with D_c = 2 lr (gamma_B + 2^-23) sum_b |g x| + 2^-22 |t|,
         the recursive-summation bound of the device's FP32 accumulation of dW over B terms
         (gamma_B = B u / (1 - B u), u = 2^-24, doubled) plus the binary32 roundings of dW and t:
         reached only where the format's spacing is finer than that bound (weights next to zero);
    anything else is unexplained. Returns a dict of counts (and 'fail_mask')."""
    B = X.shape[0]
    lr32 = abs(float(np.float32(lr)))
    gg = code_value(Gg, wk.W_BF16)
    gr = code_value(Gr, wk.W_BF16)
    xa = np.abs(code_value(X, wk.W_BF16))
    u = 2.0 ** -24
    gam = B * u / (1 - B * u)
    S = np.maximum(np.abs(gg), np.abs(gr)).T @ xa
    T64 = T.astype(np.float64)
    dc = 2.0 * lr32 * (gam + 2.0 ** -23) * S + 2.0 ** -22 * np.abs(T64)
    db = dc + lr32 * (np.abs(gg - gr).T @ xa)
    flipped = (np.asarray(Gg) != np.asarray(Gr)).any(axis=0)
    sr = orc.sr_bf16 if wfmt == wk.W_BF16 else orc.sr_e4m3

    def admissible(delta):
        lo = signed_code(sr(_outward_f32(T64 - delta, -1), R), wfmt)
        hi = signed_code(sr(_outward_f32(T64 + delta, +1), R), wfmt)
        return lo, hi

    sg = signed_code(Wg, wfmt)
    d = np.abs(sg - signed_code(Wr, wfmt))
    rest = d >= 2
    lo_c, hi_c = admissible(dc)
    lo_b, hi_b = admissible(db)
    in_b = flipped[:, None] & (sg >= lo_b) & (sg <= hi_b)
    in_c = (sg >= lo_c) & (sg <= hi_c)
    cls_b = rest & in_b
    cls_c = rest & ~in_b & in_c
    fail = rest & ~in_b & ~in_c
    return {"n": int(d.size), "equal": int((d == 0).sum()), "a": int((d == 1).sum()), "b": int(cls_b.sum()),
            "c": int(cls_c.sum()), "fail": int(fail.sum()), "max_dist": int(d.max()) if d.size else 0,
            "flipped_rows": int(flipped.sum()), "nan": int(is_nan_code(Wg, wfmt).sum()), "fail_mask": fail}


def assert_weights_free_running(orc, Wg, Wr, T, R, wfmt, X, Gg, Gr, lr, min_equal=0.999, label=""):
    """The stated weight bar against the oracle's own step: >= min_equal bit-equal, no NaN code, and
    every other element in class a, b or c of classify_weights; prints the count of each class."""
    c = classify_weights(orc, Wg, Wr, T, R, wfmt, X, Gg, Gr, lr)
    eq = c["equal"] / max(c["n"], 1)
    print(f"  W free-running{label}: equal {eq:.6f} of {c['n']}  a(1 code) {c['a']}  b(flipped G row) {c['b']}"
          f"  c(FP32 bound) {c['c']}  unexplained {c['fail']}  max code distance {c['max_dist']}"
          f"  rows with flipped G {c['flipped_rows']}", flush=True)
    assert c["nan"] == 0, f"{c['nan']} NaN weight codes"
    assert c["fail"] == 0, f"{c['fail']} weights outside every bound (max code distance {c['max_dist']})"
    assert eq >= min_equal, f"only {eq:.6f} of weights bit-equal"
    return c


def check_topk_rows(idx_g, sc_g, idx_r, sc_r, Zg_rows, Zr_rows, label=""):
    """Top-k of the device against the oracle's, row by row. Zg_rows / Zr_rows: the device's and the
    oracle's FP32 logits of those rows over all labels. Per row, tol = 2 max|Zg - Zr| (the measured
    logit error, floored at one FP32 unit of the row's largest score). Every row must:
      - list k distinct labels in (score desc, label asc) order of its own scores, NaN last;
      - give, for each label, the device's logit of that label (bit for bit) and a score within tol of
        the oracle's logit of it;
      - contain every label whose oracle score beats the oracle's k-th score by more than tol;
      - match the oracle's indices exactly unless two oracle scores within tol of each other
        straddle a difference (the tolerant path, counted and printed).
    Returns the number of rows that took the tolerant path."""
    N, k = idx_r.shape
    tolerant = 0
    for n in range(N):
        ig, sg = idx_g[n], sc_g[n]
        assert len(set(ig.tolist())) == k, (n, ig)
        for i in range(k - 1):
            a, b = sg[i], sg[i + 1]
            ok = (np.isnan(b) and not np.isnan(a)) or (np.isnan(a) and np.isnan(b) and ig[i] < ig[i + 1]) \
                or (a > b) or (a == b and ig[i] < ig[i + 1])
            assert ok, f"row {n}: order broken at {i}: ({a}, {ig[i]}) then ({b}, {ig[i + 1]})"
        zr, zg = Zr_rows[n], Zg_rows[n]
        fin = np.isfinite(zr) & np.isfinite(zg)
        err = float(np.abs(zg[fin].astype(np.float64) - zr[fin]).max()) if fin.any() else 0.0
        top = float(np.nanmax(np.abs(zr))) if np.isfinite(zr).any() else 1.0
        tol = max(2.0 * err, float(np.spacing(np.float32(top))))
        assert np.array_equal(sg.view(np.uint32), zg[ig].view(np.uint32)), f"row {n}: scores are not its logits"
        fin_s = np.isfinite(zr[ig])
        assert np.all(np.abs(sg[fin_s].astype(np.float64) - zr[ig][fin_s]) <= tol), f"row {n}: score off by > {tol}"
        if np.array_equal(ig, idx_r[n]):
            continue
        tolerant += 1
        kth = sc_r[n, -1]
        if np.isfinite(kth):
            must = np.nonzero(zr > kth + tol)[0]
            assert set(must.tolist()) <= set(ig.tolist()), f"row {n}: missing clearly better labels"
            assert np.all(zr[ig][fin_s] >= kth - tol), f"row {n}: a label far below the k-th"
    print(f"  top-{k}{label}: {N} rows, {tolerant} on the tolerant path", flush=True)
    return tolerant


# ---- MX-scaled FP4 weights (rows of D/2 code bytes and D/32 E8M0 scale bytes) --------------------
RTOL[wk.W_MXFP4] = 6e-2


def mx_split(W):
    """(element codes [n][D] uint8, scale codes [n][D/32] int64) of MXFP4 rows."""
    W = np.ascontiguousarray(W, np.uint8)
    D = W.shape[1] * 32 // 17
    c = np.empty((W.shape[0], D), np.uint8)
    c[:, 0::2] = W[:, :D // 2] & 15
    c[:, 1::2] = W[:, :D // 2] >> 4
    return c, W[:, D // 2:].astype(np.int64)


def mx_signed(c):
    """E2M1 codes as signed magnitude indices (monotone in the value; +-0 both 0)"""
    c = np.asarray(c).astype(np.int64)
    return np.where(c & 8, -(c & 7), c & 7)


def mx_weight_report(got, ref):
    """(fraction of elements with equal scale and equal value index, NaN-scale blocks in got)"""
    cg, sg = mx_split(got)
    cr, sr = mx_split(ref)
    eq = (np.repeat(sg, 32, 1) == np.repeat(sr, 32, 1)) & (mx_signed(cg) == mx_signed(cr))
    return float(eq.mean()), int((sg == 255).sum())


def classify_weights_mx(orc, Wg, Wr, T, R, X, Gg, Gr, lr):
    """classify_weights for MXFP4 rows. An element is equal when its block scale and its value index
    equal the oracle's, class a when the scale is equal and the index one away. Otherwise it is
    explained (class b or c, with the deltas D_b, D_c of classify_weights) when the device's values
    t within D of the oracle's can give both the device's block scale and its code: the block's
    largest |t| then lies in [max_k min|t_k +- D_k|, max_k max|t_k +- D_k|], the shared exponent is
    monotone in it, so the device's must lie between the exponents of those two ends; and with that
    exponent X fixed, SR(t / 2^X) with a fixed draw is monotone in t, so the device's code must lie in
    [SR((t - D) / 2^X), SR((t + D) / 2^X)] (the oracle's rounding at both ends)."""
    B = X.shape[0]
    cg, sg = mx_split(Wg)
    cr, sr = mx_split(Wr)
    n, D = cg.shape
    nb = D // 32
    lr32 = abs(float(np.float32(lr)))
    gg = code_value(Gg, wk.W_BF16)
    gr = code_value(Gr, wk.W_BF16)
    xa = np.abs(code_value(X, wk.W_BF16))
    u = 2.0 ** -24
    gam = B * u / (1 - B * u)
    T64 = T.astype(np.float64)
    S = np.maximum(np.abs(gg), np.abs(gr)).T @ xa
    dc = 2.0 * lr32 * (gam + 2.0 ** -23) * S + 2.0 ** -22 * np.abs(T64)
    db = dc + lr32 * (np.abs(gg - gr).T @ xa)
    flipped = (np.asarray(Gg) != np.asarray(Gr)).any(axis=0)
    sge, sre = np.repeat(sg, 32, 1), np.repeat(sr, 32, 1)
    ig, ir = mx_signed(cg), mx_signed(cr)
    equal = (sge == sre) & (ig == ir)
    a = (sge == sre) & (np.abs(ig - ir) == 1)
    rest = ~equal & ~a & (sge != 255)
    rr, kk = np.nonzero(rest)

    def explained(delta):
        ok = np.zeros(rr.size, bool)
        blocks = sorted(set(zip(rr.tolist(), (kk // 32).tolist())))
        sc_ok = {}
        for (j, b) in blocks:
            t = T64[j, 32 * b:32 * b + 32]; d = delta[j, 32 * b:32 * b + 32]
            lo = _outward_f32(t - d, -1).astype(np.float64); hi = _outward_f32(t + d, +1).astype(np.float64)
            mlo = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(lo), np.abs(hi)))
            mhi = np.maximum(np.abs(lo), np.abs(hi))
            xlo = orc.mx_block_exponent(np.float32(mlo.max()))
            xhi = orc.mx_block_exponent(np.float32(mhi.max()))
            sc_ok[(j, b)] = xlo <= sg[j, b] - 127 <= xhi
        for i, (j, k) in enumerate(zip(rr.tolist(), kk.tolist())):
            if not sc_ok[(j, k // 32)]:
                continue
            x = int(sg[j, k // 32]) - 127
            lo = float(_outward_f32(np.array([T64[j, k] - delta[j, k]]), -1)[0])
            hi = float(_outward_f32(np.array([T64[j, k] + delta[j, k]]), +1)[0])
            clo = mx_signed(orc.sr_e2m1(np.array([lo * 2.0 ** -x]), R[j, k]))[0]
            chi = mx_signed(orc.sr_e2m1(np.array([hi * 2.0 ** -x]), R[j, k]))[0]
            ok[i] = clo <= ig[j, k] <= chi
        return ok

    in_b = flipped[rr] & explained(db)
    in_c = explained(dc)
    cls_b = in_b
    cls_c = ~in_b & in_c
    fail = np.zeros((n, D), bool)
    fail[rr[~in_b & ~in_c], kk[~in_b & ~in_c]] = True
    d = np.abs(ig - ir)
    return {"n": int(n * D), "equal": int(equal.sum()), "a": int(a.sum()), "b": int(cls_b.sum()),
            "c": int(cls_c.sum()), "fail": int(fail.sum()), "max_dist": int(d.max()) if d.size else 0,
            "scale_diff_blocks": int((sg != sr).sum()), "flipped_rows": int(flipped.sum()),
            "nan_blocks": int((sg == 255).sum()), "fail_mask": fail}


def assert_weights_free_running_mx(orc, Wg, Wr, T, R, X, Gg, Gr, lr, min_equal=0.999, label=""):
    c = classify_weights_mx(orc, Wg, Wr, T, R, X, Gg, Gr, lr)
    eq = c["equal"] / max(c["n"], 1)
    print(f"  W free-running{label}: equal {eq:.6f} of {c['n']}  a(1 code) {c['a']}  b(flipped G row) {c['b']}"
          f"  c(FP32 bound) {c['c']}  unexplained {c['fail']}  blocks with another scale {c['scale_diff_blocks']}"
          f"  rows with flipped G {c['flipped_rows']}", flush=True)
    assert c["nan_blocks"] == 0, f"{c['nan_blocks']} NaN weight blocks"
    assert c["fail"] == 0, f"{c['fail']} weights outside every bound"
    assert eq >= min_equal, f"only {eq:.6f} of weights equal"
    return c
