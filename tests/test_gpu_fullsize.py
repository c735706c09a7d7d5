"""Parity at the full workload sizes, in the launch configuration the benchmark times (its chunk
size and workspace), on sampled outputs the oracle computes one by one: logits of sampled labels
(chunk boundaries, the ragged end and the most frequent labels among them), the updated weight rows
of those labels against the oracle's own step (free-running, every unequal element classified), dX
rows (sums over all L labels with the pre-update weights), and the top-k of 64 held-out queries
ranked by the oracle over all labels."""
import numpy as np
import pytest
import torch

import workloads as wk
from tests._helpers import (RTOL, assert_close, assert_grad_codes_match, assert_weights_free_running,
                            assert_weights_free_running_mx, batch_to_dev, check_topk_rows, mx_weight_report,
                            weight_report)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def elmo():
    import precision_label_chunk_amd as m
    m.lib()
    return m


def _host_codes(t):
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def _sample_labels(wl, n_random=24):
    c, L = wl.chunk, wl.L
    fixed = [0, 1, 2, 127, 128, c - 1, c, c + 1, 2 * c - 1, L // 2, L - 129, L - 2, L - 1]
    g = np.random.default_rng(1234)
    js = np.unique(np.concatenate([np.array([j for j in fixed if 0 <= j < L]), g.integers(0, L, n_random)]))
    return js.astype(np.int64)


@pytest.mark.parametrize("name", ["bf16_131k", "bf16_670k", "e4m3_3m", "bf16_8p6m", "mxfp4_3m"])
def test_full_size_step_sampled(elmo, orc, name):
    wl = wk.WORKLOADS[name]
    dev = torch.device("cuda:0")
    print(f"  {wl.name}: B={wl.B} D={wl.D} L={wl.L} chunk={wl.chunk}", flush=True)
    W = wk.make_w_device(wl.L, wl.D, wl.wfmt, seed=wl.seed, device=dev)
    W0 = _host_codes(W)                                   # pre-update weights for the oracle
    bt = wk.make_batch(wl, step=0)
    X, rp, ids = batch_to_dev(bt)
    js = _sample_labels(wl)
    B = wl.B

    # logits and gradient codes of the sampled labels from the step's forward kernel
    Zg = np.empty((B, js.size), np.float32)
    Gg = np.empty((B, js.size), np.uint16)
    for i, j in enumerate(js):
        z, gcol = elmo.forward(W, X, rp, ids, int(j), int(j) + 1, wfmt=wl.wfmt)
        Zg[:, i] = z.cpu().numpy()[:, 0]
        Gg[:, i] = gcol.cpu().numpy().view(np.uint16)[:, 0]
    Zr = orc.logits(wl.wfmt, W0, bt.X, js)
    ez = assert_close(Zg, Zr, RTOL[wl.wfmt])

    dX, _ = elmo.step(W, X, rp, ids, wl.lr, wl.seed, 0, wl.chunk, wfmt=wl.wfmt)
    torch.cuda.synchronize()
    Wg = _host_codes(W[torch.from_numpy(js).to(dev)])
    assert elmo.step_flags(elmo.last_workspace) == 0

    # weights of the sampled rows against the oracle's own step (its gradient codes, its t values)
    Wf, Gr, Tf = orc.update_rows(wl.wfmt, W0, bt.X, bt.row_ptr, bt.ids, wl.lr, wl.seed, 0, js, want_detail=True)
    flips = assert_grad_codes_match(Gg, Gr)
    R = np.stack([orc.r16(wl.seed, 0, int(j) * wl.D, wl.D) for j in js])
    if wl.wfmt == wk.W_MXFP4:
        c = assert_weights_free_running_mx(orc, Wg, Wf, Tf, R, bt.X, Gg, Gr, wl.lr, label=f" ({js.size} rows)")
    else:
        c = assert_weights_free_running(orc, Wg, Wf, Tf, R, wl.wfmt, bt.X, Gg, Gr, wl.lr, label=f" ({js.size} rows)")
    eq = c["equal"] / c["n"]
    # diagnostic: the oracle's weight half on the device's own gradient codes (the update kernel alone)
    Wtf = orc.update_rows_from_g(wl.wfmt, W0, bt.X, Gg, wl.lr, wl.seed, 0, js)
    eq_tf = mx_weight_report(Wg, Wtf)[0] if wl.wfmt == wk.W_MXFP4 else weight_report(Wg, Wtf, wl.wfmt)[0]
    assert eq_tf >= 0.999, f"weights given the device's gradient codes only {eq_tf:.6f} equal"

    # dX rows: sums over every label
    bs = np.array([0, B - 1], np.int32)
    dXr = orc.dx_rows(wl.wfmt, W0, bt.X, bt.row_ptr, bt.ids, bs)
    edx = assert_close(dX.cpu().numpy()[bs], dXr, RTOL[wl.wfmt])
    print(f"  Z rel {ez:.2e}  G flips {flips:.2e}  W equal {eq:.6f} (given device G {eq_tf:.6f})  dX rel {edx:.2e}",
          flush=True)


@pytest.mark.parametrize("name", ["e4m3_3m", "bf16_8p6m", "mxfp4_3m"])
@pytest.mark.timeout(900)
def test_full_size_topk_sampled_queries(elmo, orc, name):
    """Top-k over all labels of the full weight matrix for N = 1024 held-out queries in one call; 64 of
    them (spread over the query blocks) are ranked by the oracle over all labels, with the device's
    and the oracle's logits of those rows over all labels giving each row's measured error."""
    wl = wk.WORKLOADS[name]
    k = wl.topk or 5
    dev = torch.device("cuda:0")
    W = wk.make_w_device(wl.L, wl.D, wl.wfmt, seed=wl.seed, device=dev)
    N = 1024
    Xe = wk.make_eval_x(wl, N)
    print(f"  {wl.name}: top-{k} of N={N}", flush=True)
    Xd = torch.from_numpy(Xe.view(np.int16)).to(dev)
    idx, score = elmo.topk(W, Xd, k, wfmt=wl.wfmt)
    idx = idx.cpu().numpy(); score = score.cpu().numpy()
    qs = np.unique(np.concatenate([[0, 1, 127, 128, 511, 512, N - 2, N - 1],
                                   np.random.default_rng(77).choice(N, 56, replace=False)]))[:64]
    Zg = elmo.logits(W, Xd[torch.from_numpy(qs).to(dev)], 0, wl.L, wfmt=wl.wfmt).cpu().numpy()
    W0 = _host_codes(W)
    del W
    torch.cuda.empty_cache()
    print(f"  oracle logits of {qs.size} queries over {wl.L} labels", flush=True)
    Zr = orc.logits_dense(wl.wfmt, W0, Xe[qs])
    oi, osc = orc.rank_scores(Zr, k)
    check_topk_rows(idx[qs], score[qs], oi, osc, Zg, Zr, label=f" {wl.name}")


@pytest.mark.parametrize("name", ["bf16_8p6m_b32", "e4m3_3m_b32"])
def test_full_size_single_pass_sampled(elmo, orc, name):
    """The single-pass step at full size (8.6M BF16 / 3M E4M3 labels, B = 32) in the benchmark's
    launch configuration: the sampled rows' gradient codes (from its diagnostic copy) and updated
    weights against the oracle's own step, and dX rows over all labels."""
    wl = wk.WORKLOADS[name]
    dev = torch.device("cuda:0")
    print(f"  {wl.name}: single pass, B={wl.B} D={wl.D} L={wl.L} chunk={wl.chunk}", flush=True)
    W = wk.make_w_device(wl.L, wl.D, wl.wfmt, seed=wl.seed, device=dev)
    W0 = _host_codes(W)
    bt = wk.make_batch(wl, step=0)
    X, rp, ids = batch_to_dev(bt)
    js = _sample_labels(wl)
    g = torch.zeros((wl.B, wl.L), dtype=torch.int16, device=dev)
    dX, _ = elmo.step(W, X, rp, ids, wl.lr, wl.seed, 0, wl.chunk, wfmt=wl.wfmt, single_pass=True, g_out=g)
    torch.cuda.synchronize()
    jd = torch.from_numpy(js).to(dev)
    Wg = _host_codes(W[jd])
    Gg = g[:, jd].cpu().numpy().view(np.uint16)
    del g
    assert elmo.step_flags(elmo.last_workspace) == 0
    Wf, Gr, Tf = orc.update_rows(wl.wfmt, W0, bt.X, bt.row_ptr, bt.ids, wl.lr, wl.seed, 0, js, want_detail=True)
    flips = assert_grad_codes_match(Gg, Gr)
    R = np.stack([orc.r16(wl.seed, 0, int(j) * wl.D, wl.D) for j in js])
    c = assert_weights_free_running(orc, Wg, Wf, Tf, R, wl.wfmt, bt.X, Gg, Gr, wl.lr, label=f" ({js.size} rows)")
    Wtf = orc.update_rows_from_g(wl.wfmt, W0, bt.X, Gg, wl.lr, wl.seed, 0, js)
    eq_tf = weight_report(Wg, Wtf, wl.wfmt)[0]
    assert eq_tf >= 0.999, f"weights given the device's gradient codes only {eq_tf:.6f} equal"
    bs = np.array([0, 17, wl.B - 1], np.int32)
    dXr = orc.dx_rows(wl.wfmt, W0, bt.X, bt.row_ptr, bt.ids, bs)
    edx = assert_close(dX.cpu().numpy()[bs], dXr, RTOL[wl.wfmt])
    print(f"  G flips {flips:.2e}  W equal {c['equal'] / c['n']:.6f} (given device G {eq_tf:.6f})  dX rel {edx:.2e}",
          flush=True)
