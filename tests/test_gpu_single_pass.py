"""Parity of the single-pass step (elmo_xmc_step_single_pass: one kernel per chunk, the gradient kept
on chip, the weights read and written once) against the CPU oracle, through the C ABI, with the same
bar as the two-kernel step: the device's gradient codes (its diagnostic copy) within one BF16 unit
of the oracle's and at most 1e-3 of them different, the updated weights against the oracle's own
step (>= 99.9% bit-equal, every other element in a named class), dX within the stated tolerance and
the summed loss within 1e-4. Cases span several 32-label tiles and work-groups, ragged tails, more
work-groups than tiles and several chunks, in every weight format."""
import numpy as np
import pytest
import torch

import workloads as wk
from tests._helpers import (RTOL, assert_close, assert_grad_codes_match, assert_weights_free_running,
                            assert_weights_free_running_mx, batch_to_dev, is_nan_code, mx_weight_report,
                            to_dev_codes, weight_report)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def elmo():
    import precision_label_chunk_amd as m
    m.lib()
    return m


def _case(B, D, L, wfmt, lam=3.0, seed=0):
    base = wk.WORKLOADS["mxfp4_3m" if wfmt == wk.W_MXFP4 else "bf16_131k"]
    kw = {} if wfmt == wk.W_MXFP4 else {"wfmt": wfmt, "zipf_s": 1.0}
    wl = wk.scaled(base, B=B, D=D, L=L, lam=lam, seed=seed, **kw)
    return wl, wk.make_weights(wl), wk.make_batch(wl)


def _run(elmo, W0, bt, wfmt, lr, seed, step, chunk, single=True, want_loss=False):
    W = to_dev_codes(W0)
    X, rp, ids = batch_to_dev(bt)
    B, L = bt.X.shape[0], W0.shape[0]
    g = torch.zeros((B, L), dtype=torch.int16, device="cuda") if single else None
    print(f"  {'single-pass' if single else 'two-kernel'} step B={B} L={L} wfmt={wfmt} chunk={chunk}", flush=True)
    dX, loss = elmo.step(W, X, rp, ids, lr, seed, step, chunk, want_loss=want_loss, single_pass=single, g_out=g,
                         wfmt=elmo.ELMO_W_MXFP4 if wfmt == wk.W_MXFP4 else None)
    torch.cuda.synchronize()
    a = W.cpu().numpy()
    Wg = a.view(np.uint16) if a.dtype == np.int16 else a
    Gg = g.cpu().numpy().view(np.uint16) if single else None
    return Wg, dX.cpu().numpy(), (float(loss.item()) if want_loss else None), Gg


CASES = [  # B, D, L, chunk, wfmt
    (32, 768, 4096, 1024, wk.W_BF16),      # 32 tiles per chunk, four chunks
    (32, 768, 3000, 1024, wk.W_E4M3),      # ragged last chunk (952 labels) and last tile
    (32, 768, 2500, 512, wk.W_MXFP4),
    (1, 256, 300, 128, wk.W_BF16),         # one sample; three chunks, the last of 44 labels
    (17, 512, 1000, 1000, wk.W_E4M3),      # chunk rounded down to 896, ragged second chunk
    (32, 256, 777, 5000, wk.W_BF16),       # chunk larger than L
    (5, 768, 70, 128, wk.W_BF16),          # one chunk of three tiles, the last ragged
    (32, 768, 1337, 128, wk.W_E4M3),       # eleven chunks of four tiles each
    (24, 512, 1500, 384, wk.W_MXFP4),
    (32, 768, 20000, 20000, wk.W_BF16),    # 625 tiles over 256 work-groups (two or three each)
]


def check_single(orc, W0, bt, wfmt, lr, seed, step, Wg, dXg, lossg, Gg):
    L = W0.shape[0]
    Wr, dXr, lossr, _, Gr = orc.step(wfmt, W0, bt.X, bt.row_ptr, bt.ids, lr, seed, step, want_g=True,
                                     want_loss=lossg is not None)
    flips = assert_grad_codes_match(Gg, Gr)
    _, T = orc.update_from_g(wfmt, W0, bt.X, Gr, lr, seed, step, want_t=True)
    if wfmt == wk.W_MXFP4:
        D = T.shape[1]
        R = orc.r16(seed, step, 0, L * D).reshape(L, D)
        assert_weights_free_running_mx(orc, Wg, Wr, T, R, bt.X, Gg, Gr, lr)
        eq_tf, nan_tf = mx_weight_report(Wg, orc.update_from_g(wfmt, W0, bt.X, Gg, lr, seed, step))
        assert nan_tf == 0
    else:
        R = orc.r16(seed, step, 0, W0.size).reshape(W0.shape)
        assert_weights_free_running(orc, Wg, Wr, T, R, wfmt, bt.X, Gg, Gr, lr)
        eq_tf, _, _ = weight_report(Wg, orc.update_from_g(wfmt, W0, bt.X, Gg, lr, seed, step), wfmt)
    assert eq_tf >= 0.999, f"weights given the device's gradient codes only {eq_tf:.6f} equal"
    e = assert_close(dXg, dXr, RTOL[wfmt])
    if lossg is not None:
        assert abs(lossg - lossr) <= 1e-4 * abs(lossr)
    print(f"  G flips {flips:.2e}  W given device G: equal {eq_tf:.6f}  dX rel {e:.2e}", flush=True)


@pytest.mark.parametrize("B,D,L,chunk,wfmt", CASES)
def test_single_pass_matches_oracle(elmo, orc, B, D, L, chunk, wfmt):
    wl, W0, bt = _case(B, D, L, wfmt)
    lr, seed, step = 0.05, 11, 3
    Wg, dXg, lossg, Gg = _run(elmo, W0, bt, wfmt, lr, seed, step, chunk, want_loss=True)
    check_single(orc, W0, bt, wfmt, lr, seed, step, Wg, dXg, lossg, Gg)


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3, wk.W_MXFP4])
def test_single_pass_agrees_with_two_kernel_step(elmo, wfmt):
    """The two paths share the update arithmetic and the dW summation order: every label row whose
    gradient codes agree (all but a handful) has bit-identical updated weights; dX agrees to the
    FP32 summation order."""
    wl, W0, bt = _case(32, 768, 6000, wfmt, lam=5.0)
    lr, seed, step = 0.05, 2, 7
    Ws, dXs, _, Gs = _run(elmo, W0, bt, wfmt, lr, seed, step, 2048)
    Wt, dXt, _, _ = _run(elmo, W0, bt, wfmt, lr, seed, step, 2048, single=False)
    X, rp, ids = batch_to_dev(bt)
    _, G2 = elmo.forward(to_dev_codes(W0), X, rp, ids, 0, W0.shape[0],
                         wfmt=elmo.ELMO_W_MXFP4 if wfmt == wk.W_MXFP4 else None)
    G2 = G2.cpu().numpy().view(np.uint16)
    same = (Gs == G2).all(axis=0)
    print(f"  rows with equal gradient codes: {int(same.sum())} of {same.size}", flush=True)
    assert same.mean() >= 0.99
    assert np.array_equal(Ws[same], Wt[same])
    assert_close(dXs, dXt, 1e-4)


def test_single_pass_repeat_runs_are_bitwise_identical(elmo):
    wl, W0, bt = _case(32, 768, 5000, wk.W_E4M3)
    a = _run(elmo, W0, bt, wk.W_E4M3, 0.1, 1, 1, 1024, want_loss=True)
    b = _run(elmo, W0, bt, wk.W_E4M3, 0.1, 1, 1, 1024, want_loss=True)
    for x, y in zip(a, b):
        assert np.array_equal(np.asarray(x), np.asarray(y))


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_single_pass_chunk_size_invariance(elmo, wfmt):
    """Chunking changes which tiles share a work-group and chunk, never the arithmetic of a weight:
    the weights are bit-identical across chunk sizes (the logits of a tile are summed in the same
    fixed order whatever work-group holds it)."""
    wl, W0, bt = _case(29, 512, 3000, wfmt)
    outs = [_run(elmo, W0, bt, wfmt, 0.1, 5, 1, c) for c in (128, 1000, 3000, 1 << 20)]
    for Wg, dXg, _, Gg in outs[1:]:
        assert np.array_equal(Gg, outs[0][3])
        assert np.array_equal(Wg, outs[0][0])
        assert_close(dXg, outs[0][1], 1e-5)


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_single_pass_nan_propagates_as_in_the_oracle(elmo, orc, wfmt):
    """A NaN weight makes its label's updated row NaN and every dX element NaN; the other rows meet
    the weight bar."""
    wl, W0, bt = _case(20, 256, 1500, wfmt)
    lr, seed, step = 0.05, 3, 1
    nan_code = 0x7FC0 if wfmt == wk.W_BF16 else 0x7F
    Wb = W0.copy(); Wb[700, 33] = nan_code
    Wg, dXg, _, Gg = _run(elmo, Wb, bt, wfmt, lr, seed, step, 512)
    Wr, dXr, _, _, Gr = orc.step(wfmt, Wb, bt.X, bt.row_ptr, bt.ids, lr, seed, step, want_g=True)
    assert np.array_equal(is_nan_code(Wg, wfmt), is_nan_code(Wr, wfmt))
    assert is_nan_code(Wg[700], wfmt).all()
    assert np.isnan(dXg).all() and np.isnan(dXr).all()
    assert np.array_equal(is_nan_code(Gg, wk.W_BF16), is_nan_code(Gr, wk.W_BF16))
    keep = np.arange(W0.shape[0]) != 700
    _, T = orc.update_from_g(wfmt, Wb, bt.X, Gr, lr, seed, step, want_t=True)
    R = orc.r16(seed, step, 0, W0.size).reshape(W0.shape)
    assert_weights_free_running(orc, Wg[keep], Wr[keep], T[keep], R[keep], wfmt, bt.X, Gg[:, keep], Gr[:, keep], lr,
                                label=" (rows without NaN)")


def test_single_pass_no_labels(elmo, orc):
    wl, W0, bt = _case(32, 768, 2000, wk.W_BF16)
    empty = wk.Batch(bt.X, np.zeros(33, np.int32), np.zeros(0, np.int32))
    Wg, dXg, lossg, Gg = _run(elmo, W0, empty, wk.W_BF16, 0.05, 4, 2, 1024, want_loss=True)
    check_single(orc, W0, empty, wk.W_BF16, 0.05, 4, 2, Wg, dXg, lossg, Gg)


@pytest.mark.parametrize("B,D,wfmt", [(32, 768, wk.W_BF16), (7, 256, wk.W_MXFP4), (33, 768, wk.W_E4M3),
                                      (32, 640, wk.W_BF16)])
def test_default_step_takes_the_faster_path(elmo, B, D, wfmt):
    """elmo_xmc_step runs the single pass where it is built (B <= 32, D in 256/512/768) and the two
    kernels elsewhere: its weights and dX are bit-identical to the entry point of that path."""
    wl, W0, bt = _case(B, D, 1500, wfmt)
    fmt = elmo.ELMO_W_MXFP4 if wfmt == wk.W_MXFP4 else None
    single = B <= 32 and D in (256, 512, 768)
    outs = []
    for sp in (None, single if single else False):
        W = to_dev_codes(W0)
        X, rp, ids = batch_to_dev(bt)
        print(f"  B={B} D={D} wfmt={wfmt} single_pass={sp}", flush=True)
        dX, _ = elmo.step(W, X, rp, ids, 0.05, 3, 2, 512, wfmt=fmt, single_pass=sp)
        torch.cuda.synchronize()
        outs.append((W.cpu().numpy(), dX.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])
