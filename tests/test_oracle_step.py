"""Pins of the oracle's training step, loss gradient and top-k scoring.

* Finite differences of the summed sigmoid-BCE loss (the loss is not printed on the pages; it is the
  reading documented with the build) in the unquantised binary64 mode.
* The closed form G = sigmoid(Z) - Y against scipy's expit, and the W = 0 special case.
* The three contractions against numpy binary64 matmul of the torch-decoded operands.
* The SGD + stochastic-rounding update against an exact rational recomputation.
* Invariants: lr = 0, label-set semantics, sampled entry points equal to the full step.
* Top-k against numpy lexsort / argmax, with exact ties from duplicated weight rows.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import workloads as wk


def _bf16_val(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def _e4m3_val(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _wval(wfmt, W):
    return _bf16_val(W) if wfmt == wk.W_BF16 else _e4m3_val(W)


def _dense_y(B, L, rp, ids):
    Y = np.zeros((B, L))
    for b in range(B):
        Y[b, ids[rp[b]:rp[b + 1]]] = 1.0
    return Y


def _small_case(wfmt, B=9, D=64, L=300, seed=0, lam=3.0):
    wl = wk.scaled(wk.WORKLOADS["bf16_131k"], B=B, D=D, L=L, wfmt=wfmt, lam=lam, seed=seed)
    bt = wk.make_batch(wl)
    W = wk.make_weights(wl)
    return wl, W, bt


# ---------------------------------------------------------------------------------------------- #
def test_finite_difference_gradients(orc):
    g = np.random.default_rng(5)
    B, D, L = 3, 5, 7
    W = g.standard_normal((L, D)); X = g.standard_normal((B, D))
    Y = (g.random((B, L)) < 0.3).astype(np.float64)
    Z, G, dX, dW, loss = orc.grad_exact(W, X, Y)
    h = 1e-6
    for j in range(L):
        for k in range(D):
            Wp = W.copy(); Wp[j, k] += h; Wm = W.copy(); Wm[j, k] -= h
            fd = (orc.grad_exact(Wp, X, Y)[4] - orc.grad_exact(Wm, X, Y)[4]) / (2 * h)
            assert abs(fd - dW[j, k]) <= 1e-6 * max(1.0, abs(dW[j, k]))
    for b in range(B):
        for k in range(D):
            Xp = X.copy(); Xp[b, k] += h; Xm = X.copy(); Xm[b, k] -= h
            fd = (orc.grad_exact(W, Xp, Y)[4] - orc.grad_exact(W, Xm, Y)[4]) / (2 * h)
            assert abs(fd - dX[b, k]) <= 1e-6 * max(1.0, abs(dX[b, k]))
    # dL/dZ through a bias-like perturbation: shifting z_bj by h is the same as adding h / x_bk * e_jk
    # to W when only x_bk is non-zero; check directly on a one-hot X instead
    X1 = np.zeros((B, D)); X1[:, 0] = 1.0
    Z1, G1, *_ = orc.grad_exact(W, X1, Y)
    for b in range(B):
        for j in range(L):
            Wp = W.copy(); Wp[j, 0] += h; Wm = W.copy(); Wm[j, 0] -= h
            Yb = Y.copy()
            lp = orc.grad_exact(Wp, X1, Yb)[4]; lm = orc.grad_exact(Wm, X1, Yb)[4]
            # with X1, z_bj = W[j, 0] for every b, so the derivative sums over b
            if b == 0:
                assert abs((lp - lm) / (2 * h) - G1[:, j].sum()) <= 1e-6
    # loss definition: sum of softplus(z) - y z
    assert abs(loss - (np.logaddexp(0, Z) - Y * Z).sum()) <= 1e-12 * abs(loss)


def test_gradient_code_matches_expit(orc):
    g = np.random.default_rng(6)
    z = np.concatenate([g.standard_normal(4000) * 3, g.uniform(-80, 80, 4000),
                        [0.0, -0.0, 1e-8, -1e-8, 88.0, -88.0, 200.0, -200.0]]).astype(np.float32)
    for y in (0, 1):
        ref64 = scipy.special.expit(z.astype(np.float64)) if y == 0 else -scipy.special.expit(-z.astype(np.float64))
        ref = torch.from_numpy(ref64.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        got = np.array([orc.grad_code(float(v), y) for v in z], np.uint16)
        # scipy's expit and binary64 exp may differ in the last binary64 bit: allow mismatches only
        # where the binary32 value sits on a rounding boundary, i.e. none in practice
        assert (got != ref).sum() <= 1


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_zero_weights_closed_form(orc, wfmt):
    wl, W, bt = _small_case(wfmt)
    W0 = np.zeros_like(W)
    lr = 0.05
    Wn, dX, loss, Z, G = orc.step(wfmt, W0, bt.X, bt.row_ptr, bt.ids, lr, 1, 0, want_z=True, want_g=True,
                                  want_loss=True)
    Y = _dense_y(wl.B, wl.L, bt.row_ptr, bt.ids)
    assert np.all(Z == 0.0)
    assert np.array_equal(_bf16_val(G), 0.5 - Y)
    assert np.all(dX == 0.0)
    x = _bf16_val(bt.X)
    dW = ((0.5 - Y).T @ x).astype(np.float32)      # exact in binary64 at these sizes
    t = (-np.float64(np.float32(lr)) * dW.astype(np.float64)).astype(np.float32)
    new = _wval(wfmt, Wn)
    # stochastic rounding lands on one of the two neighbours of t
    tab = _bf16_val(np.arange(0, 0x7F80, dtype=np.uint16)) if wfmt == wk.W_BF16 else _e4m3_val(np.arange(0x7F, dtype=np.uint8))
    a = np.abs(t.astype(np.float64))
    i = np.searchsorted(tab, a, side="right") - 1
    lo = tab[i]; hi = tab[np.minimum(i + 1, tab.size - 1)]
    assert np.all((np.abs(new) == lo) | (np.abs(new) == hi))
    assert abs(loss - wl.B * wl.L * np.log(2.0)) <= 1e-9 * loss


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_contractions_match_numpy_matmul(orc, wfmt):
    wl, W, bt = _small_case(wfmt, B=17, D=128, L=257)
    lr = np.float32(0.05)
    Wn, dX, loss, Z, G = orc.step(wfmt, W, bt.X, bt.row_ptr, bt.ids, lr, 3, 2, want_z=True, want_g=True)
    w = _wval(wfmt, W)
    x = _bf16_val(bt.X)
    xt = x if wfmt == wk.W_BF16 else _e4m3_val(
        torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    Zref = (xt @ w.T).astype(np.float32)
    assert np.array_equal(Z, Zref)
    g = _bf16_val(G)
    Y = _dense_y(wl.B, wl.L, bt.row_ptr, bt.ids)
    # G against expit of the oracle's own FP32 logits
    ref64 = np.where(Y > 0, -scipy.special.expit(-Z.astype(np.float64)), scipy.special.expit(Z.astype(np.float64)))
    gref = _bf16_val(torch.from_numpy(ref64.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    assert (g != gref).sum() <= 1
    assert np.array_equal(dX, (g @ w).astype(np.float32))
    dW = (g.T @ x).astype(np.float32)
    # update: t = FP32(w - lr * dW) rounded once; SR with the oracle's random bits
    rng_rows = orc.r16(3, 2, 0, wl.L * wl.D).reshape(wl.L, wl.D)
    sample = np.random.default_rng(0).integers(0, wl.L * wl.D, 3000)
    for s in sample:
        j, k = divmod(int(s), wl.D)
        exact = Fraction(float(w[j, k])) - Fraction(float(lr)) * Fraction(float(dW[j, k]))
        t = _round_f32(exact)
        if wfmt == wk.W_BF16:
            want = orc.sr_bf16(np.array([t], np.float32), np.array([rng_rows[j, k]], np.uint32))[0]
        else:
            want = orc.sr_e4m3(np.array([t], np.float32), np.array([rng_rows[j, k]], np.uint32))[0]
        assert Wn[j, k] == want


def _round_f32(fr: Fraction) -> np.float32:
    """Correctly rounded (nearest-even) binary32 of a rational."""
    f = np.float32(float(fr))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - fr)
        if best is None or d < best[0] or (d == best[0] and (int(np.float32(c).view(np.uint32)) & 1) == 0):
            best = (d, c)
    return np.float32(best[1])


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_lr_zero_leaves_weights_unchanged(orc, wfmt):
    wl, W, bt = _small_case(wfmt)
    Wn, *_ = orc.step(wfmt, W, bt.X, bt.row_ptr, bt.ids, 0.0, 1, 0)
    # equal values; a negative zero may come back positive (IEEE: -0 * g + -0 is +0 for g < 0)
    assert np.array_equal(_wval(wfmt, Wn), _wval(wfmt, W))
    zero_flip = Wn != W
    assert np.all(_wval(wfmt, W)[zero_flip] == 0.0)


def test_label_set_semantics(orc):
    wl, W, bt = _small_case(wk.W_BF16, B=6, L=120)
    g = np.random.default_rng(9)
    rows = [bt.ids[bt.row_ptr[b]:bt.row_ptr[b + 1]] for b in range(wl.B)]
    rows2 = [g.permutation(np.concatenate([r, r[: len(r) // 2 + 1]])) for r in rows]  # shuffled, duplicated
    rows2[2] = np.zeros(0, np.int32)                                                   # an empty row
    rows1 = [np.unique(r) for r in rows2]
    def csr(rs):
        rp = np.zeros(len(rs) + 1, np.int32); rp[1:] = np.cumsum([len(r) for r in rs])
        return rp, (np.concatenate(rs).astype(np.int32) if sum(map(len, rs)) else np.zeros(0, np.int32))
    a = orc.step(0, W, bt.X, *csr(rows1), 0.05, 4, 1)
    b = orc.step(0, W, bt.X, *csr(rows2), 0.05, 4, 1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    with pytest.raises(RuntimeError):
        rp, ids = csr(rows1); ids = ids.copy(); ids[0] = wl.L
        orc.step(0, W, bt.X, rp, ids, 0.05, 4, 1)


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_sampled_entry_points_equal_full_step(orc, wfmt):
    wl, W, bt = _small_case(wfmt, B=11, D=64, L=333)
    Wn, dX, _, Z, _ = orc.step(wfmt, W, bt.X, bt.row_ptr, bt.ids, wl.lr, 5, 3, want_z=True)
    js = np.array([0, 1, 17, 200, 332], np.int64)
    assert np.array_equal(orc.logits(wfmt, W, bt.X, js), Z[:, js])
    assert np.array_equal(orc.update_rows(wfmt, W, bt.X, bt.row_ptr, bt.ids, wl.lr, 5, 3, js), Wn[js])
    bs = np.array([0, 4, 10], np.int32)
    d = orc.dx_rows(wfmt, W, bt.X, bt.row_ptr, bt.ids, bs)
    # same definition, different binary64 summation order: equal up to one binary32 ulp
    assert np.all(np.abs(d - dX[bs]) <= np.spacing(np.abs(dX[bs])))


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_update_from_g_is_the_weight_half_of_the_step(orc, wfmt):
    wl, W, bt = _small_case(wfmt, B=10, D=64, L=150)
    Wn, _, _, _, G = orc.step(wfmt, W, bt.X, bt.row_ptr, bt.ids, wl.lr, 8, 2, want_g=True)
    assert np.array_equal(orc.update_from_g(wfmt, W, bt.X, G, wl.lr, 8, 2), Wn)


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_update_rows_from_g_is_the_sampled_weight_half(orc, wfmt):
    wl, W, bt = _small_case(wfmt, B=9, D=64, L=260)
    Wn, _, _, _, G = orc.step(wfmt, W, bt.X, bt.row_ptr, bt.ids, wl.lr, 6, 4, want_g=True)
    js = np.array([0, 3, 128, 259], np.int64)
    assert np.array_equal(orc.update_rows_from_g(wfmt, W, bt.X, G[:, js], wl.lr, 6, 4, js), Wn[js])
    # other codes give the row update of those codes (global RNG index of each row kept)
    G2 = G.copy(); G2[:, js] ^= 1
    assert np.array_equal(orc.update_rows_from_g(wfmt, W, bt.X, G2[:, js], wl.lr, 6, 4, js),
                          orc.update_from_g(wfmt, W, bt.X, G2, wl.lr, 6, 4)[js])


def test_saturated_dyadic_step_is_exact(orc):
    """X, W in {+-2^-3} with a dominant first column make |z| >= 116, so the FP32 sigmoid is exactly
    0 or 1 and every intermediate is exact; the result is predicted without the oracle."""
    g = np.random.default_rng(11)
    B, D, L = 8, 64, 96
    xs = g.choice([-1.0, 1.0], (B, D)) * 0.125
    ws = g.choice([-1.0, 1.0], (L, D)) * 0.125
    xs[:, 0] = g.choice([-128.0, 128.0], B)
    ws[:, 0] = g.choice([-1.0, 1.0], L)
    X = wk.to_bf16_codes(xs); W = wk.to_bf16_codes(ws)
    Y = (g.random((B, L)) < 0.2)
    rp = np.zeros(B + 1, np.int32); rp[1:] = np.cumsum(Y.sum(1))
    ids = np.concatenate([np.nonzero(Y[b])[0] for b in range(B)]).astype(np.int32)
    lr = 2.0**-10
    Wn, dX, _, Z, G = orc.step(0, W, X, rp, ids, lr, 0, 0, want_z=True, want_g=True)
    z = xs @ ws.T
    assert np.all(np.abs(z) >= 116) and np.array_equal(Z, z.astype(np.float32))
    gexp = (z > 0).astype(np.float64) - Y
    assert np.array_equal(_bf16_val(G), gexp)
    assert np.array_equal(dX, (gexp @ ws).astype(np.float32))
    t = ws - lr * (gexp.T @ xs)                    # exact dyadic rationals
    new = _bf16_val(Wn)
    tab = _bf16_val(np.arange(0, 0x7F80, dtype=np.uint16))
    i = np.searchsorted(tab, np.abs(t), side="right") - 1
    assert np.all((np.abs(new) == tab[i]) | (np.abs(new) == tab[i + 1]))
    exact = tab[i] == np.abs(t)
    assert np.array_equal(new[exact], t[exact])


# ---------------------------------------------------------------------------------------------- #
@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_topk_matches_lexsort(orc, wfmt):
    wl, W, bt = _small_case(wfmt, B=13, D=64, L=500)
    W = W.copy()
    W[100] = W[7]; W[499] = W[7]; W[250] = W[3]   # exact ties: the smaller label must win
    k = 6
    idx, score = orc.topk(wfmt, W, bt.X, k)
    w = _wval(wfmt, W); x = _bf16_val(bt.X)
    xt = x if wfmt == wk.W_BF16 else _e4m3_val(
        torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    S = (xt @ w.T).astype(np.float32)
    for n in range(S.shape[0]):
        order = np.lexsort((np.arange(wl.L), -S[n].astype(np.float64)))[:k]
        assert np.array_equal(idx[n], order)
        assert np.array_equal(score[n], S[n, order])
    idx1, _ = orc.topk(wfmt, W, bt.X, 1)
    assert np.array_equal(idx1[:, 0], np.argmax(S, axis=1))


def test_topk_nan_ranks_last(orc):
    wl, W, bt = _small_case(wk.W_BF16, B=4, D=64, L=50)
    W = W.copy(); W[:, 0] = 0x7FC0                # every score NaN ...
    W[10] = wk.to_bf16_codes(np.full(64, 0.01))   # ... except rows 10 and 20
    W[20] = wk.to_bf16_codes(np.full(64, -0.01))
    idx, score = orc.topk(0, W, bt.X, 4)
    assert np.all(np.sort(idx[:, :2], axis=1) == [10, 20])
    assert np.all(np.isnan(score[:, 2:])) and np.array_equal(idx[:, 2:], np.tile([0, 1], (4, 1)))


# ---------------------------------------------------------------------------------------------- #
@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_update_t_outputs_are_the_rounded_values(orc, wfmt):
    """The FP32 value t the oracle hands to stochastic rounding: t = fmaf(-lr, dW, w) with dW the
    binary32 rounding of the exact sum (recomputed here with exact rationals), and the stored code is
    the stochastic rounding of exactly that t with the element's draw."""
    wl, W, bt = _small_case(wfmt, B=7, D=64, L=40)
    lr, seed, step = 0.05, 3, 1
    Wn, _, _, _, G = orc.step(wfmt, W, bt.X, bt.row_ptr, bt.ids, lr, seed, step, want_g=True)
    Wu, T = orc.update_from_g(wfmt, W, bt.X, G, lr, seed, step, want_t=True)
    assert np.array_equal(Wu, Wn)
    g = _bf16_val(G); x = _bf16_val(bt.X); w = _wval(wfmt, W)
    lr32 = Fraction(float(np.float32(lr)))
    for (j, k) in [(0, 0), (3, 17), (39, 63), (20, 5)]:
        dw = float(np.float32(float(sum(Fraction(g[b, j]) * Fraction(x[b, k]) for b in range(7)))))
        t = float(np.float32(float(Fraction(w[j, k]) - lr32 * Fraction(dw))))
        assert T[j, k] == np.float32(t)
    R = orc.r16(seed, step, 0, W.size).reshape(W.shape)
    sr = orc.sr_bf16 if wfmt == wk.W_BF16 else orc.sr_e4m3
    assert np.array_equal(sr(T, R), Wn)
    js = np.array([0, 5, 39], np.int64)
    Wr, Gr, Tr = orc.update_rows(wfmt, W, bt.X, bt.row_ptr, bt.ids, lr, seed, step, js, want_detail=True)
    assert np.array_equal(Wr, Wn[js]) and np.array_equal(Gr, G[:, js]) and np.array_equal(Tr, T[js])


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_dense_logits_and_ranking_match_the_loops(orc, wfmt):
    """The blocked binary64 matrix-product form of the logits equals orc_logits (same definition,
    other summation order: at most one FP32 unit, almost always bit-equal), and the ranking of a score
    matrix by lexsort equals orc_topk, exact ties (duplicated rows) and NaN included."""
    wl, W, bt = _small_case(wfmt, B=21, D=128, L=3000, seed=4)
    W = W.copy()
    W[2999] = W[5]; W[1000] = W[5]; W[77] = W[1500]
    X = wk.make_eval_x(wl, 21)
    Zd = orc.logits_dense(wfmt, W, X, block=700)
    Zl = orc.logits(wfmt, W, X, np.arange(wl.L))
    assert np.all(np.abs(Zd.astype(np.float64) - Zl) <= np.spacing(np.abs(Zl)))
    assert (Zd == Zl).mean() >= 0.9999
    for k in (1, 5, 64):
        i_ref, s_ref = orc.topk(wfmt, W, X, k)
        i_d, s_d = orc.rank_scores(Zl, k)
        assert np.array_equal(i_d, i_ref) and np.array_equal(s_d, s_ref)
    Zn = Zl.copy(); Zn[:, 10:] = np.nan; Zn[0, 3] = -np.inf
    i_n, _ = orc.rank_scores(Zn, 12)
    assert np.array_equal(i_n[1], np.concatenate([np.argsort(-Zl[1, :10], kind="stable"), [10, 11]]))
    assert list(i_n[0][:10]) == [j for j in np.lexsort((np.arange(10), -Zn[0, :10].astype(np.float64)))]


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_nan_propagation(orc, wfmt):
    """NaN follows IEEE arithmetic through the step: a NaN weight makes its label's logits, gradient
    codes and updated row NaN and every dX element NaN (each sums over that label); a NaN feature
    makes its sample's logits and dX row NaN and, through dW = G^T X, every updated weight NaN."""
    wl, W, bt = _small_case(wfmt, B=6, D=64, L=50)
    nan_code = 0x7FC0 if wfmt == wk.W_BF16 else 0x7F
    Wb = W.copy(); Wb[13, 9] = nan_code
    Wn, dX, _, Z, G = orc.step(wfmt, Wb, bt.X, bt.row_ptr, bt.ids, 0.05, 1, 0, want_z=True, want_g=True)
    isnan = np.isnan(_wval(wfmt, Wn))
    assert isnan[13].all() and not isnan[np.arange(50) != 13].any()
    assert np.isnan(Z[:, 13]).all() and np.isfinite(np.delete(Z, 13, axis=1)).all()
    assert np.isnan(_bf16_val(G[:, 13])).all() and np.isnan(dX).all()
    Xb = bt.X.copy(); Xb[2, 40] = 0x7FC0
    Wn, dX, _, Z, _ = orc.step(wfmt, W, Xb, bt.row_ptr, bt.ids, 0.05, 1, 0, want_z=True)
    assert np.isnan(_wval(wfmt, Wn)).all()
    assert np.isnan(Z[2]).all() and np.isfinite(np.delete(Z, 2, axis=0)).all()
    assert np.isnan(dX[2]).all() and np.isfinite(np.delete(dX, 2, axis=0)).all()


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_sample_permutation_invariance(orc, wfmt):
    """Permuting the samples (feature rows with their label rows) permutes dX's rows exactly (each is
    a sum over labels, in the same order) and leaves the weights unchanged except where the new order
    of the binary64 sum over samples moves dW across a binary32 rounding boundary (rare)."""
    wl, W, bt = _small_case(wfmt, B=12, D=64, L=200)
    perm = np.random.default_rng(3).permutation(12)
    rows = [bt.ids[bt.row_ptr[b]:bt.row_ptr[b + 1]] for b in perm]
    rp = np.zeros(13, np.int32); rp[1:] = np.cumsum([len(r) for r in rows])
    ids = np.concatenate(rows).astype(np.int32)
    Wa, dXa, _, _, _ = orc.step(wfmt, W, bt.X, bt.row_ptr, bt.ids, 0.05, 2, 0)
    Wp, dXp, _, _, _ = orc.step(wfmt, W, bt.X[perm], rp, ids, 0.05, 2, 0)
    d = np.abs(np.asarray(Wa, np.int64) - np.asarray(Wp, np.int64))
    assert (d == 0).mean() >= 0.9999
    assert np.array_equal(dXa[perm], dXp)
