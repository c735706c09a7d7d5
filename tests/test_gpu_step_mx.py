"""Training-step parity of the HIP path for MX-scaled FP4 weights (E2M1 elements, one E8M0 scale per
32 features, the format the summary page's Limitations leave to micro-tensor scaling) against the
CPU oracle, through the C ABI: logits, gradient codes, dX and the updated blocks (scale and codes),
at sizes that span several tiles and a ragged tail, plus invariants and edge cases."""
import numpy as np
import pytest
import torch

import workloads as wk
from tests._helpers import (RTOL, assert_close, assert_grad_codes_match, assert_weights_free_running_mx,
                            batch_to_dev, mx_split, mx_weight_report, to_dev_codes)

pytestmark = pytest.mark.gpu
MX = wk.W_MXFP4


@pytest.fixture(scope="module")
def elmo():
    import precision_label_chunk_amd as m
    m.lib()
    return m


def _case(B, D, L, lam=3.0, seed=0):
    wl = wk.scaled(wk.WORKLOADS["mxfp4_3m"], B=B, D=D, L=L, lam=lam, seed=seed)
    return wl, wk.make_weights(wl), wk.make_batch(wl)


def _run(elmo, W0, bt, lr, seed, step, chunk, want_loss=False):
    W = torch.from_numpy(np.ascontiguousarray(W0)).cuda()
    X, rp, ids = batch_to_dev(bt)
    D = W0.shape[1] * 32 // 17
    print(f"  mx step B={bt.X.shape[0]} D={D} L={W0.shape[0]} chunk={chunk}", flush=True)
    # (the two-kernel step, also at the shapes where elmo_xmc_step takes the single pass; that path
    # has its own tests)
    dX, loss = elmo.step(W, X, rp, ids, lr, seed, step, chunk, want_loss=want_loss, wfmt=elmo.ELMO_W_MXFP4,
                         single_pass=False)
    torch.cuda.synchronize()
    return W.cpu().numpy(), dX.cpu().numpy(), (float(loss.item()) if want_loss else None)


def _gpu_forward(elmo, W0, bt, L):
    X, rp, ids = batch_to_dev(bt)
    Z, G = elmo.forward(to_dev_codes(W0), X, rp, ids, 0, L, wfmt=elmo.ELMO_W_MXFP4)
    return Z.cpu().numpy(), G.cpu().numpy().view(np.uint16)


CASES = [  # B, D, L, chunk
    (32, 256, 4096, 1024),
    (1, 256, 300, 128),         # one sample, ragged
    (100, 512, 2500, 512),
    (17, 256, 1000, 1000),      # chunk rounded down to 896, ragged second chunk
    (200, 256, 777, 5000),      # chunk larger than L
    (256, 768, 3000, 1024),     # full batch and width
    (129, 768, 1500, 256),
    (64, 1024, 700, 384),       # largest D
]


def check_step(elmo, orc, W0, bt, lr, seed, step, Wg, dXg, lossg=None):
    """As the BF16 / E4M3 parity check, with the weights compared block by block: scale and element
    codes against the oracle's own step (free-running, classes a / b / c of the block form), and
    against the oracle's update given the device's gradient codes (>= 99.9% equal)."""
    L = W0.shape[0]
    Wr, dXr, lossr, Zr, Gr = orc.step(MX, W0, bt.X, bt.row_ptr, bt.ids, lr, seed, step, want_z=True, want_g=True,
                                      want_loss=lossg is not None)
    Zg, Gg = _gpu_forward(elmo, W0, bt, L)
    ez = assert_close(Zg, Zr, RTOL[MX])
    flips = assert_grad_codes_match(Gg, Gr)
    _, T = orc.update_from_g(MX, W0, bt.X, Gr, lr, seed, step, want_t=True)
    D = T.shape[1]
    R = orc.r16(seed, step, 0, L * D).reshape(L, D)
    assert_weights_free_running_mx(orc, Wg, Wr, T, R, bt.X, Gg, Gr, lr)
    eq_tf, nan_tf = mx_weight_report(Wg, orc.update_from_g(MX, W0, bt.X, Gg, lr, seed, step))
    assert eq_tf >= 0.999 and nan_tf == 0, f"weights given the device's gradient codes only {eq_tf:.6f} equal"
    e = assert_close(dXg, dXr, RTOL[MX])
    if lossg is not None:
        assert abs(lossg - lossr) <= 1e-4 * abs(lossr)
    print(f"  Z rel {ez:.2e}  G flips {flips:.2e}  W given device G: equal {eq_tf:.6f}  dX rel {e:.2e}", flush=True)


@pytest.mark.parametrize("B,D,L,chunk", CASES)
def test_mx_step_matches_oracle(elmo, orc, B, D, L, chunk):
    wl, W0, bt = _case(B, D, L)
    lr, seed, step = 0.05, 11, 3
    Wg, dXg, lossg = _run(elmo, W0, bt, lr, seed, step, chunk, want_loss=True)
    check_step(elmo, orc, W0, bt, lr, seed, step, Wg, dXg, lossg)


def test_mx_logits_subrange(elmo, orc):
    wl, W0, bt = _case(200, 768, 1000)
    Wd, Xd = to_dev_codes(W0), batch_to_dev(bt)[0]
    for l0, l1 in [(333, 901), (0, 1), (999, 1000), (130, 131), (0, 1000)]:
        Zg = elmo.logits(Wd, Xd, l0, l1, wfmt=elmo.ELMO_W_MXFP4).cpu().numpy()
        assert_close(Zg, orc.logits(MX, W0, bt.X, np.arange(l0, l1)), RTOL[MX])


@pytest.mark.parametrize("B,D", [(48, 256), (256, 768)])
def test_mx_chunk_size_invariance(elmo, B, D):
    wl, W0, bt = _case(B, D, 2000)
    outs = [_run(elmo, W0, bt, 0.1, 5, 1, c) for c in (128, 1000, 2000, 1 << 20)]
    for Wg, dXg, _ in outs[1:]:
        assert np.array_equal(Wg, outs[0][0])
        assert_close(dXg, outs[0][1], 1e-5)


def test_mx_lr_zero_keeps_values(elmo, orc):
    """With lr = 0, t is the decoded weight itself: every block's value is kept exactly (its scale
    may move where the block's largest magnitude is below 4, with the codes rescaled to match)."""
    wl, W0, bt = _case(40, 256, 1500)
    Wg, _, _ = _run(elmo, W0, bt, 0.0, 1, 0, 512)
    assert np.array_equal(orc.mx_decode(Wg), orc.mx_decode(W0))


def test_mx_saturated_dyadic_step_is_exact(elmo, orc):
    """|z| >= 116 makes the sigmoid exactly 0 or 1 and, with dyadic features and weights, every sum
    exact: the device must give the oracle's blocks bit for bit, and exact logits and dX."""
    g = np.random.default_rng(11)
    B, D, L = 64, 256, 1000
    lr, seed, step = 2.0 ** -6, 5, 3
    xs = g.choice([-1.0, 1.0], (B, D)) * 0.125
    xs[:, 0] = g.choice([-128.0, 128.0], B)
    codes = g.integers(0, 16, (L, D)).astype(np.uint8)
    codes[:, 0] = g.choice([4, 12], L)
    W0 = np.empty((L, D // 2 + D // 32), np.uint8)
    W0[:, :D // 2] = codes[:, 0::2] | (codes[:, 1::2] << 4)
    W0[:, D // 2:] = 126
    X = wk.to_bf16_codes(xs)
    Y = g.random((B, L)) < 0.1
    rp = np.zeros(B + 1, np.int32); rp[1:] = np.cumsum(Y.sum(1))
    ids = np.concatenate([np.nonzero(Y[b])[0] for b in range(B)]).astype(np.int32)
    bt = wk.Batch(X, rp, ids)
    Wg, dXg, _ = _run(elmo, W0, bt, lr, seed, step, 256)
    Wr, dXr, _, Zr, _ = orc.step(MX, W0, X, rp, ids, lr, seed, step, want_z=True)
    assert np.array_equal(dXg, dXr)
    assert np.array_equal(Wg, Wr)
    Zg = elmo.logits(to_dev_codes(W0), batch_to_dev(bt)[0], 0, L, wfmt=elmo.ELMO_W_MXFP4).cpu().numpy()
    assert np.array_equal(Zg, Zr)


def test_mx_nan_block_propagates_as_in_the_oracle(elmo, orc):
    """A NaN scale (code 255) makes its label's logits and gradient codes NaN, every block of that
    row a NaN block (scale 255, zero codes) and every dX element NaN, as in the oracle; the other
    rows meet the weight bar."""
    wl, W0, bt = _case(40, 256, 1500)
    lr, seed, step = 0.05, 3, 1
    D = 256
    Wb = W0.copy(); Wb[700, D // 2 + 3] = 255
    Wg, dXg, _ = _run(elmo, Wb, bt, lr, seed, step, 512)
    Wr, dXr, _, _, Gr = orc.step(MX, Wb, bt.X, bt.row_ptr, bt.ids, lr, seed, step, want_g=True)
    cg, sg = mx_split(Wg)
    cr, sr = mx_split(Wr)
    assert np.array_equal(sg == 255, sr == 255) and (sg[700] == 255).all() and (cg[700] == 0).all()
    assert np.isnan(dXg).all() and np.isnan(dXr).all()
    keep = np.arange(W0.shape[0]) != 700
    _, Gg = _gpu_forward(elmo, Wb, bt, W0.shape[0])
    _, T = orc.update_from_g(MX, Wb, bt.X, Gr, lr, seed, step, want_t=True)
    R = orc.r16(seed, step, 0, W0.shape[0] * D).reshape(W0.shape[0], D)
    assert_weights_free_running_mx(orc, Wg[keep], Wr[keep], T[keep], R[keep], bt.X, Gg[:, keep], Gr[:, keep], lr,
                                   label=" (rows without NaN)")


def test_mx_feature_sizes_rejected(elmo):
    """MXFP4 needs D % 256 == 0 (8-byte aligned rows): other sizes are refused before any work."""
    assert elmo.step_workspace_bytes(32, 192, 1000, 512, elmo.ELMO_W_MXFP4, 10) == 0
    W = torch.zeros((100, 192 * 17 // 32), dtype=torch.uint8, device="cuda")
    X = torch.zeros((4, 192), dtype=torch.int16, device="cuda")
    rp = torch.zeros(5, dtype=torch.int32, device="cuda")
    ids = torch.zeros(0, dtype=torch.int32, device="cuda")
    with pytest.raises(elmo.ElmoError):
        elmo.step(W, X, rp, ids, 0.1, 0, 0, 128, wfmt=elmo.ELMO_W_MXFP4)


def test_mx_nan_feature_propagates_as_in_the_oracle(elmo, orc):
    """A NaN feature makes every logit of its sample NaN, so every label's dW and every block's t
    hold a NaN: every block becomes a NaN block (scale 255, zero codes), as in the oracle; its
    sample's dX row is NaN and the other rows stay finite and close."""
    wl, W0, bt = _case(40, 256, 1500)
    lr, seed, step = 0.05, 3, 1
    Xb = bt.X.copy(); Xb[5, 17] = 0x7FC0
    btn = wk.Batch(Xb, bt.row_ptr, bt.ids)
    Wg, dXg, _ = _run(elmo, W0, btn, lr, seed, step, 512)
    Wr, dXr, _, _, _ = orc.step(MX, W0, Xb, bt.row_ptr, bt.ids, lr, seed, step)
    cg, sg = mx_split(Wg)
    cr, sr = mx_split(Wr)
    assert (sg == 255).all() and (sr == 255).all() and (cg == 0).all()
    assert np.isnan(dXg[5]).all() and np.isnan(dXr[5]).all()
    rows = np.arange(40) != 5
    assert_close(dXg[rows], dXr[rows], RTOL[MX])


def test_mx_sample_permutation_general(elmo, orc):
    """Permuting the samples of a general MXFP4 batch: the permuted step meets the block weight bar
    against the oracle's step on the permuted batch, its dX rows are the unpermuted run's rows
    permuted (to the FP32 summation order), and the two runs' blocks are >= 99.9% equal."""
    wl, W0, bt = _case(100, 256, 2500, lam=6.0)
    perm = np.random.default_rng(21).permutation(100)
    rows = [bt.ids[bt.row_ptr[p]:bt.row_ptr[p + 1]] for p in perm]
    rp = np.zeros(101, np.int32); rp[1:] = np.cumsum([len(r) for r in rows])
    btp = wk.Batch(bt.X[perm], rp, np.concatenate(rows).astype(np.int32))
    lr, seed, step = 0.05, 6, 2
    Wa, dXa, _ = _run(elmo, W0, bt, lr, seed, step, 1024)
    Wp, dXp, _ = _run(elmo, W0, btp, lr, seed, step, 1024)
    check_step(elmo, orc, W0, btp, lr, seed, step, Wp, dXp)
    assert_close(dXp, dXa[perm], 1e-5)
    eq, nan = mx_weight_report(Wp, Wa)
    print(f"  permuted vs unpermuted blocks: equal {eq:.6f}", flush=True)
    assert eq >= 0.999 and nan == 0
