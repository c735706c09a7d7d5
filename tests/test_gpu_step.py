"""Training-step parity of the HIP path (through the C ABI) against the CPU oracle, element by element,
at sizes that span several tiles and a ragged tail, plus invariants and edge cases."""
import numpy as np
import pytest
import torch

import workloads as wk
from tests._helpers import (RTOL, assert_close, assert_grad_codes_match, assert_weights_free_running, batch_to_dev,
                            code_value, from_dev_codes, rel_err, to_dev_codes, weight_report)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def elmo():
    import precision_label_chunk_amd as m
    m.lib()
    return m


def _case(B, D, L, wfmt, lam=3.0, seed=0, x_kind="rownorm"):
    wl = wk.scaled(wk.WORKLOADS["bf16_131k"], B=B, D=D, L=L, wfmt=wfmt, lam=lam, seed=seed, x_kind=x_kind,
                   zipf_s=1.0)
    return wl, wk.make_weights(wl), wk.make_batch(wl)


def _run(elmo, W0, bt, wfmt, lr, seed, step, chunk, want_loss=False):
    W = to_dev_codes(W0)
    X, rp, ids = batch_to_dev(bt)
    print(f"  step B={bt.X.shape[0]} D={W0.shape[1]} L={W0.shape[0]} wfmt={wfmt} chunk={chunk}", flush=True)
    dX, loss = elmo.step(W, X, rp, ids, lr, seed, step, chunk, want_loss=want_loss)
    torch.cuda.synchronize()
    return from_dev_codes(W), dX.cpu().numpy(), (float(loss.item()) if want_loss else None)


CASES = [  # B, D, L, chunk, wfmt
    (32, 64, 4096, 1024, wk.W_BF16),       # the tiny oracle configuration
    (32, 128, 4096, 1024, wk.W_E4M3),      # its FP8 variant
    (1, 64, 300, 128, wk.W_BF16),          # one sample, L below three tiles, ragged
    (17, 192, 1000, 1000, wk.W_BF16),      # chunk rounded down to 896, ragged second chunk
    (100, 256, 2500, 512, wk.W_E4M3),
    (200, 128, 777, 5000, wk.W_BF16),      # chunk larger than L
    (129, 64, 1500, 256, wk.W_E4M3),       # D = 64 in FP8: half a staged K slice
    (256, 768, 3000, 1024, wk.W_E4M3),     # full batch and width
    (256, 768, 2100, 1024, wk.W_BF16),
    (64, 1024, 700, 384, wk.W_BF16),       # largest D
    # E4M3 with 129..256 samples and D = 768: the forward with the features held in registers
    (200, 768, 1000, 1000, wk.W_E4M3),     # chunk rounded down to 896, ragged second chunk
    (129, 768, 70, 128, wk.W_E4M3),        # one chunk of two 64-label tiles, the second ragged
    (256, 768, 5000, 65536, wk.W_E4M3),    # chunk larger than L
    (160, 768, 1337, 128, wk.W_E4M3),      # eleven chunks of one 128-label tile each
    # BF16 with 65..128 samples and D = 768: the forward with BF16 features held in registers
    (128, 768, 3000, 1024, wk.W_BF16),
    (100, 768, 1337, 256, wk.W_BF16),      # ragged last chunk and last 32-label tile
    (65, 768, 70, 128, wk.W_BF16),         # one chunk of three 32-label tiles, the last ragged
]


def _gpu_forward(elmo, W0, bt, L):
    X, rp, ids = batch_to_dev(bt)
    Z, G = elmo.forward(to_dev_codes(W0), X, rp, ids, 0, L)
    return Z.cpu().numpy(), G.cpu().numpy().view(np.uint16)


def check_step(elmo, orc, W0, bt, wfmt, lr, seed, step, Wg, dXg, lossg=None):
    """Parity of one GPU step against the oracle.
    Logits and dX: elementwise relative error with an RMS floor. Gradient codes: every code within
    one BF16 unit and at most 1e-3 of them different (FP32 logit and sigmoid rounding decides a
    BF16 rounding only near a tie). Weights against the oracle's own step (free-running): >= 99.9%
    bit-equal, every other element one code away or inside the bound of a named difference of the
    FP32 arithmetic before the rounding (a flipped gradient code of its label, or the FP32
    accumulation of dW next to zero), each class counted. Diagnostic: the oracle's weight half run on
    the device's own gradient codes isolates the update kernel (>= 99.9% bit-equal there too)."""
    L = W0.shape[0]
    Wr, dXr, lossr, Zr, Gr = orc.step(wfmt, W0, bt.X, bt.row_ptr, bt.ids, lr, seed, step, want_z=True, want_g=True,
                                      want_loss=lossg is not None)
    Zg, Gg = _gpu_forward(elmo, W0, bt, L)
    ez = assert_close(Zg, Zr, RTOL[wfmt])
    flips = assert_grad_codes_match(Gg, Gr)
    _, T = orc.update_from_g(wfmt, W0, bt.X, Gr, lr, seed, step, want_t=True)
    R = orc.r16(seed, step, 0, W0.size).reshape(W0.shape)
    assert_weights_free_running(orc, Wg, Wr, T, R, wfmt, bt.X, Gg, Gr, lr)
    eq_tf, mx_tf, _ = weight_report(Wg, orc.update_from_g(wfmt, W0, bt.X, Gg, lr, seed, step), wfmt)
    assert eq_tf >= 0.999, f"weights given the device's gradient codes only {eq_tf:.6f} equal"
    e = assert_close(dXg, dXr, RTOL[wfmt])
    if lossg is not None:
        assert abs(lossg - lossr) <= 1e-4 * abs(lossr)
    print(f"  Z rel {ez:.2e}  G flips {flips:.2e}  W given device G: equal {eq_tf:.6f} max dist {mx_tf}"
          f"  dX rel {e:.2e}", flush=True)
    if wfmt == wk.W_E4M3:
        # context only: the FP8 logits against logits of the unquantised BF16 features (the effect
        # of casting X to E4M3, which the 6e-2 tolerance leaves room for)
        Zu = code_value(bt.X, wk.W_BF16) @ code_value(W0, wfmt).T
        print(f"  FP8 logits vs unquantised-X logits: max rel {rel_err(Zg, Zu).max():.2e}", flush=True)


@pytest.mark.parametrize("B,D,L,chunk,wfmt", CASES)
def test_step_matches_oracle(elmo, orc, B, D, L, chunk, wfmt):
    wl, W0, bt = _case(B, D, L, wfmt)
    lr, seed, step = 0.05, 11, 3
    Wg, dXg, lossg = _run(elmo, W0, bt, wfmt, lr, seed, step, chunk, want_loss=True)
    check_step(elmo, orc, W0, bt, wfmt, lr, seed, step, Wg, dXg, lossg)


@pytest.mark.parametrize("B,D,wfmt", [(20, 128, wk.W_BF16), (200, 768, wk.W_E4M3), (100, 768, wk.W_BF16)])
def test_logits_subrange(elmo, orc, B, D, wfmt):
    wl, W0, bt = _case(B, D, 1000, wfmt)
    Wd, Xd = to_dev_codes(W0), batch_to_dev(bt)[0]
    for l0, l1 in [(333, 901), (0, 1), (999, 1000), (130, 131), (0, 1000)]:
        js = np.arange(l0, l1)
        Zg = elmo.logits(Wd, Xd, l0, l1).cpu().numpy()
        Zr = orc.logits(wfmt, W0, bt.X, js)
        assert_close(Zg, Zr, RTOL[wfmt])


@pytest.mark.parametrize("B,D,wfmt", [(48, 128, wk.W_BF16), (48, 128, wk.W_E4M3), (256, 768, wk.W_E4M3),
                                      (128, 768, wk.W_BF16)])
def test_chunk_size_invariance(elmo, B, D, wfmt):
    wl, W0, bt = _case(B, D, 2000, wfmt)
    outs = [_run(elmo, W0, bt, wfmt, 0.1, 5, 1, c) for c in (128, 1000, 2000, 1 << 20)]
    for Wg, dXg, _ in outs[1:]:
        assert np.array_equal(Wg, outs[0][0])               # weights: bit-identical
        assert_close(dXg, outs[0][1], 1e-5)                  # dX: FP32 summation order only


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_lr_zero_keeps_weights(elmo, wfmt):
    wl, W0, bt = _case(40, 128, 1500, wfmt)
    Wg, _, _ = _run(elmo, W0, bt, wfmt, 0.0, 1, 0, 512)
    eq, mx, _ = weight_report(Wg, W0, wfmt)
    assert eq == 1.0 and mx == 0                             # +-0 counted equal


def test_repeat_runs_are_bitwise_identical(elmo):
    wl, W0, bt = _case(256, 768, 2500, wk.W_E4M3, lam=20)
    runs = [_run(elmo, W0, bt, wk.W_E4M3, 0.1, 3, 9, 1024) for _ in range(3)]
    for Wg, dXg, _ in runs[1:]:
        assert np.array_equal(Wg, runs[0][0])
        assert np.array_equal(dXg, runs[0][1])


def test_resume_equals_uninterrupted(elmo):
    """The step keeps no state: W after steps 0..3 run in one loop equals W after 0..1 then 2..3
    from a copy (a checkpoint is W plus the next step index)."""
    wl, W0, _ = _case(64, 128, 1200, wk.W_BF16)
    batches = [wk.make_batch(wl, step=s) for s in range(4)]
    W = to_dev_codes(W0)
    for s in range(4):
        X, rp, ids = batch_to_dev(batches[s]); elmo.step(W, X, rp, ids, 0.05, 7, s, 512)
    W2 = to_dev_codes(W0)
    for s in range(2):
        X, rp, ids = batch_to_dev(batches[s]); elmo.step(W2, X, rp, ids, 0.05, 7, s, 512)
    ckpt = W2.cpu()
    W3 = ckpt.cuda()
    for s in range(2, 4):
        X, rp, ids = batch_to_dev(batches[s]); elmo.step(W3, X, rp, ids, 0.05, 7, s, 512)
    torch.cuda.synchronize()
    assert torch.equal(W.cpu(), W3.cpu())


def test_teacher_forced_multi_step(elmo, orc):
    wl, W0, _ = _case(32, 64, 4096, wk.W_BF16, x_kind="gauss_sqrtD")
    W = to_dev_codes(W0)
    for s in range(3):
        bt = wk.make_batch(wl, step=s)
        Wprev = from_dev_codes(W)
        X, rp, ids = batch_to_dev(bt)
        dX, _ = elmo.step(W, X, rp, ids, 0.05, 0, s, 1024)
        torch.cuda.synchronize()
        check_step(elmo, orc, Wprev, bt, wk.W_BF16, 0.05, 0, s, from_dev_codes(W), dX.cpu().numpy())


def _csr(rows):
    rp = np.zeros(len(rows) + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ids = np.concatenate(rows).astype(np.int32) if rp[-1] else np.zeros(0, np.int32)
    return rp, ids


def test_label_set_semantics_and_empty_rows(elmo):
    wl, W0, bt = _case(24, 64, 900, wk.W_BF16)
    g = np.random.default_rng(1)
    rows = [bt.ids[bt.row_ptr[b]:bt.row_ptr[b + 1]] for b in range(24)]
    messy = [g.permutation(np.concatenate([r, r[:2]])) for r in rows]
    messy[3] = np.zeros(0, np.int32); messy[23] = np.zeros(0, np.int32)
    clean = [np.unique(r) for r in messy]
    a = _run(elmo, W0, wk.Batch(bt.X, *_csr(clean)), wk.W_BF16, 0.05, 2, 0, 256)
    b = _run(elmo, W0, wk.Batch(bt.X, *_csr(messy)), wk.W_BF16, 0.05, 2, 0, 256)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_no_labels_at_all(elmo, orc):
    wl, W0, bt = _case(8, 64, 500, wk.W_E4M3)
    rp = np.zeros(9, np.int32); ids = np.zeros(0, np.int32)
    b0 = wk.Batch(bt.X, rp, ids)
    Wg, dXg, _ = _run(elmo, W0, b0, wk.W_E4M3, 0.05, 2, 0, 256)
    check_step(elmo, orc, W0, b0, wk.W_E4M3, 0.05, 2, 0, Wg, dXg)


def test_out_of_range_labels_are_flagged_and_skipped(elmo, orc):
    wl, W0, bt = _case(16, 64, 800, wk.W_BF16)
    ids = bt.ids.copy(); ids[0] = 800; ids[5] = -3
    W = to_dev_codes(W0)
    X, rp, idd = batch_to_dev(wk.Batch(bt.X, bt.row_ptr, ids))
    dX, _ = elmo.step(W, X, rp, idd, 0.05, 2, 0, 256)
    flags = elmo.step_flags(elmo.last_workspace)
    assert flags & elmo.FLAG_LABEL_RANGE
    keep = np.ones(ids.size, bool); keep[[0, 5]] = False
    rows = [ids[bt.row_ptr[b]:bt.row_ptr[b + 1]][keep[bt.row_ptr[b]:bt.row_ptr[b + 1]]] for b in range(16)]
    rp2, ids2 = _csr(rows)
    check_step(elmo, orc, W0, wk.Batch(bt.X, rp2, ids2), wk.W_BF16, 0.05, 2, 0, from_dev_codes(W), dX.cpu().numpy())


def test_clean_labels_raise_no_flag(elmo):
    wl, W0, bt = _case(16, 64, 800, wk.W_BF16)
    W = to_dev_codes(W0); X, rp, ids = batch_to_dev(bt)
    elmo.step(W, X, rp, ids, 0.05, 2, 0, 256)
    assert elmo.step_flags(elmo.last_workspace) == 0


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_saturated_dyadic_step_is_exact(elmo, orc, wfmt):
    """|z| >= 116 makes the sigmoid exactly 0 or 1 in FP32 and every sum exact: the GPU must match
    100% of the weight codes and give exact logits and dX."""
    g = np.random.default_rng(11)
    B, D, L = 64, 128, 1000
    xs = g.choice([-1.0, 1.0], (B, D)) * 0.125
    ws = g.choice([-1.0, 1.0], (L, D)) * 0.125
    xs[:, 0] = g.choice([-128.0, 128.0], B)
    ws[:, 0] = g.choice([-1.0, 1.0], L)
    X = wk.to_bf16_codes(xs)
    W0 = wk.to_bf16_codes(ws) if wfmt == wk.W_BF16 else wk.to_e4m3_codes(ws)
    Y = g.random((B, L)) < 0.1
    rp, ids = _csr([np.nonzero(Y[b])[0] for b in range(B)])
    bt = wk.Batch(X, rp, ids)
    Wg, dXg, _ = _run(elmo, W0, bt, wfmt, 2.0**-10, 4, 2, 256)
    Wr, dXr, _, Zr, _ = orc.step(wfmt, W0, X, rp, ids, 2.0**-10, 4, 2, want_z=True)
    assert np.array_equal(dXg, dXr)
    eq, mx, _ = weight_report(Wg, Wr, wfmt)
    assert eq == 1.0
    Zg = elmo.logits(to_dev_codes(W0), batch_to_dev(bt)[0], 0, L).cpu().numpy()
    assert np.array_equal(Zg, Zr)


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_nan_propagates_as_in_the_oracle(elmo, orc, wfmt):
    """A NaN weight makes its label's row NaN and every dX element NaN (IEEE arithmetic through the
    logit, the gradient and both sums) and leaves the other rows to the weight bar; a NaN feature
    makes every updated weight and its sample's dX row NaN, the other dX rows finite and close."""
    from tests._helpers import is_nan_code
    wl, W0, bt = _case(40, 128, 1500, wfmt)
    lr, seed, step = 0.05, 3, 1
    nan_code = 0x7FC0 if wfmt == wk.W_BF16 else 0x7F
    Wb = W0.copy(); Wb[700, 33] = nan_code
    Wg, dXg, _ = _run(elmo, Wb, bt, wfmt, lr, seed, step, 512)
    Wr, dXr, _, _, Gr = orc.step(wfmt, Wb, bt.X, bt.row_ptr, bt.ids, lr, seed, step, want_g=True)
    assert np.array_equal(is_nan_code(Wg, wfmt), is_nan_code(Wr, wfmt))
    assert is_nan_code(Wg[700], wfmt).all()
    assert np.isnan(dXg).all() and np.isnan(dXr).all()
    keep = np.arange(W0.shape[0]) != 700
    _, Gg = _gpu_forward(elmo, Wb, bt, W0.shape[0])
    assert np.array_equal(is_nan_code(Gg, wk.W_BF16), is_nan_code(Gr, wk.W_BF16))
    _, T = orc.update_from_g(wfmt, Wb, bt.X, Gr, lr, seed, step, want_t=True)
    R = orc.r16(seed, step, 0, W0.size).reshape(W0.shape)
    assert_weights_free_running(orc, Wg[keep], Wr[keep], T[keep], R[keep], wfmt, bt.X, Gg[:, keep], Gr[:, keep], lr,
                                label=" (rows without NaN)")
    Xb = bt.X.copy(); Xb[5, 17] = 0x7FC0
    btn = wk.Batch(Xb, bt.row_ptr, bt.ids)
    Wg, dXg, _ = _run(elmo, W0, btn, wfmt, lr, seed, step, 512)
    Wr, dXr, _, _, _ = orc.step(wfmt, W0, Xb, bt.row_ptr, bt.ids, lr, seed, step)
    assert is_nan_code(Wg, wfmt).all() and is_nan_code(Wr, wfmt).all()
    assert np.isnan(dXg[5]).all() and np.isnan(dXr[5]).all()
    rows = np.arange(40) != 5
    assert_close(dXg[rows], dXr[rows], RTOL[wfmt])


def test_sample_permutation_dyadic_exact(elmo, orc):
    """Permuting the samples with exact arithmetic (saturated dyadic inputs): weights bit-identical,
    dX rows permuted exactly."""
    g = np.random.default_rng(12)
    B, D, L = 96, 128, 900
    xs = g.choice([-1.0, 1.0], (B, D)) * 0.125
    ws = g.choice([-1.0, 1.0], (L, D)) * 0.125
    xs[:, 0] = g.choice([-128.0, 128.0], B)
    ws[:, 0] = g.choice([-1.0, 1.0], L)
    X = wk.to_bf16_codes(xs); W0 = wk.to_bf16_codes(ws)
    Y = g.random((B, L)) < 0.05
    rows = [np.nonzero(Y[b])[0] for b in range(B)]
    perm = g.permutation(B)
    a = _run(elmo, W0, wk.Batch(X, *_csr(rows)), wk.W_BF16, 2.0**-10, 4, 2, 256)
    b = _run(elmo, W0, wk.Batch(X[perm], *_csr([rows[p] for p in perm])), wk.W_BF16, 2.0**-10, 4, 2, 256)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1][perm], b[1])


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_sample_permutation_general(elmo, orc, wfmt):
    """Permuting the samples of a general batch: the permuted step meets the weight bar against the
    oracle's step on the permuted batch, its dX rows are the unpermuted run's rows permuted (to the
    FP32 summation order), and the two runs' weights differ only where the FP32 order of the dW sum
    over samples moves a rounding (>= 99.9% bit-equal)."""
    wl, W0, bt = _case(100, 256, 2500, wfmt, lam=6.0)
    perm = np.random.default_rng(21).permutation(100)
    rows = [bt.ids[bt.row_ptr[p]:bt.row_ptr[p + 1]] for p in perm]
    btp = wk.Batch(bt.X[perm], *_csr(rows))
    lr, seed, step = 0.05, 6, 2
    Wa, dXa, _ = _run(elmo, W0, bt, wfmt, lr, seed, step, 1024)
    Wp, dXp, _ = _run(elmo, W0, btp, wfmt, lr, seed, step, 1024)
    check_step(elmo, orc, W0, btp, wfmt, lr, seed, step, Wp, dXp)
    assert_close(dXp, dXa[perm], 1e-5)
    eq, mx, _ = weight_report(Wp, Wa, wfmt)
    print(f"  permuted vs unpermuted weights: equal {eq:.6f}, max code distance {mx}", flush=True)
    assert eq >= 0.999


def test_bf16_logits_have_the_same_bits_in_every_forward(elmo):
    """Every BF16 forward sums a logit as one MFMA chain over the features in order (the tiled
    forward at 256 and at 32 padded samples, the stationary-feature forward at 65-128, and the
    tiled top-k scan): the same queries' logits, computed in batches that take different forward
    kernels, are bit-identical."""
    wl = wk.scaled(wk.WORKLOADS["bf16_131k"], B=256, D=768, L=3000)
    W0 = wk.make_weights(wl)
    X = wk.make_batch(wl).X
    Wd = to_dev_codes(W0)
    Z = {}
    for n in (256, 100, 20):
        print(f"  BF16 logits of {n} queries over {W0.shape[0]} labels", flush=True)
        Xd = torch.from_numpy(np.ascontiguousarray(X[:n]).view(np.int16)).cuda()
        Z[n] = elmo.logits(Wd, Xd, 0, W0.shape[0]).cpu().numpy()
    assert np.array_equal(Z[256][:100].view(np.uint32), Z[100].view(np.uint32))
    assert np.array_equal(Z[256][:20].view(np.uint32), Z[20].view(np.uint32))
