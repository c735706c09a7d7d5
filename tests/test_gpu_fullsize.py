"""Parity at the full workload sizes, in the launch configuration the benchmark times (its chunk
size and workspace), on sampled outputs the oracle computes one by one: logits of sampled labels
(chunk boundaries, the ragged end and the most frequent labels among them), the updated weight rows
of those labels (given the device's gradient codes, and free-running), dX rows (sums over all L
labels with the pre-update weights), and the top-k of sampled queries."""
import numpy as np
import pytest
import torch

import workloads as wk
from tests._helpers import (RTOL, assert_close, assert_grad_codes_match, assert_weights_match, batch_to_dev,
                            update_error_bound, weight_report)

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


@pytest.mark.parametrize("name", ["bf16_131k", "bf16_670k", "e4m3_3m", "bf16_8p6m"])
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
        z, gcol = elmo.forward(W, X, rp, ids, int(j), int(j) + 1)
        Zg[:, i] = z.cpu().numpy()[:, 0]
        Gg[:, i] = gcol.cpu().numpy().view(np.uint16)[:, 0]
    Zr = orc.logits(wl.wfmt, W0, bt.X, js)
    ez = assert_close(Zg, Zr, RTOL[wl.wfmt])

    dX, _ = elmo.step(W, X, rp, ids, wl.lr, wl.seed, 0, wl.chunk)
    torch.cuda.synchronize()
    Wg = _host_codes(W[torch.from_numpy(js).to(dev)])
    assert elmo.step_flags(elmo.last_workspace) == 0

    # weights of the sampled rows, given the device's gradient codes, then free-running
    Wt = orc.update_rows_from_g(wl.wfmt, W0, bt.X, Gg, wl.lr, wl.seed, 0, js)
    eq = assert_weights_match(Wg, Wt, wl.wfmt, abs_bound=update_error_bound(Gg, bt.X, wl.lr, B))
    Wf = orc.update_rows(wl.wfmt, W0, bt.X, bt.row_ptr, bt.ids, wl.lr, wl.seed, 0, js)
    eq_free = weight_report(Wg, Wf, wl.wfmt)[0]
    assert eq_free >= 0.999, f"free-running weights only {eq_free:.6f} equal"

    # dX rows: sums over every label
    bs = np.array([0, B - 1], np.int32)
    dXr = orc.dx_rows(wl.wfmt, W0, bt.X, bt.row_ptr, bt.ids, bs)
    edx = assert_close(dX.cpu().numpy()[bs], dXr, RTOL[wl.wfmt])
    print(f"  Z rel {ez:.2e}  W equal {eq:.6f} (free {eq_free:.6f})  dX rel {edx:.2e}", flush=True)


@pytest.mark.parametrize("name", ["e4m3_3m", "bf16_8p6m"])
def test_full_size_topk_sampled_queries(elmo, orc, name):
    """Top-k over all labels of the full weight matrix for N held-out queries; two queries are
    ranked by the oracle over all labels. Indices must be identical except where the oracle's
    neighbouring scores are closer than the logit tolerance (then the device's label must score
    within that tolerance of the oracle's at that rank)."""
    wl = wk.WORKLOADS[name]
    k = wl.topk or 5
    dev = torch.device("cuda:0")
    W = wk.make_w_device(wl.L, wl.D, wl.wfmt, seed=wl.seed, device=dev)
    N = 1024
    Xe = wk.make_eval_x(wl, N)
    print(f"  {wl.name}: top-{k} of N={N}", flush=True)
    idx, score = elmo.topk(W, torch.from_numpy(Xe.view(np.int16)).to(dev), k)
    idx = idx.cpu().numpy(); score = score.cpu().numpy()
    W0 = _host_codes(W)
    qs = np.array([0, N - 1])
    oi, osc = orc.topk(wl.wfmt, W0, Xe[qs], k)
    tol = RTOL[wl.wfmt] * 1e-2 * max(float(np.abs(osc).max()), 1e-30)
    for r, q in enumerate(qs):
        assert np.all(np.abs(score[q] - osc[r]) <= tol), (score[q], osc[r])
        for p in range(k):
            if idx[q, p] != oi[r, p]:
                zg = orc.logits(wl.wfmt, W0, Xe[q:q + 1], np.array([idx[q, p]], np.int64))[0, 0]
                assert abs(zg - osc[r, p]) <= tol, f"query {q} rank {p}: label {idx[q, p]} vs {oi[r, p]}"
