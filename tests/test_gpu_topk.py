"""Top-k scoring parity against the CPU oracle. Indices must match exactly wherever the oracle's
ranking is decided by more than the measured FP32 logit error (twice the row's largest difference
between the device's and the oracle's logits); exact ties (duplicated weight rows) must go to the
smaller label bit for bit; returned scores are the device's logits of the returned labels, in
(score desc, label asc) order."""
import numpy as np
import pytest
import torch

import workloads as wk
from tests._helpers import check_topk_rows, to_dev_codes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def elmo():
    import precision_label_chunk_amd as m
    m.lib()
    return m


def _xdev(X):
    return torch.from_numpy(np.ascontiguousarray(X).view(np.int16)).cuda()


def _check(elmo, orc, wfmt, W0, Wd, X, idx_g, sc_g, k, label=""):
    """Rows of the device's top-k against the oracle's ranking of the same queries, with the
    device's and the oracle's logits over all labels giving each row's measured error."""
    idx_r, sc_r = orc.topk(wfmt, W0, X, k)
    Zr = orc.logits(wfmt, W0, X, np.arange(W0.shape[0]))
    Zg = np.concatenate([elmo.logits(Wd, _xdev(X[r:r + 256]), 0, W0.shape[0], wfmt=wfmt).cpu().numpy()
                         for r in range(0, X.shape[0], 256)])      # (the forward takes up to 256 rows)
    return check_topk_rows(idx_g, sc_g, idx_r, sc_r, Zg, Zr, label=label)


@pytest.mark.parametrize("N,D,L,k,wfmt", [(13, 64, 500, 5, wk.W_BF16), (300, 128, 5000, 5, wk.W_E4M3),
                                          (129, 768, 3000, 1, wk.W_BF16), (64, 192, 2000, 32, wk.W_BF16),
                                          (257, 256, 4099, 8, wk.W_E4M3), (4, 64, 40, 32, wk.W_E4M3),
                                          (70, 128, 3000, 64, wk.W_BF16), (130, 256, 2000, 64, wk.W_E4M3),
                                          (3, 64, 64, 64, wk.W_BF16), (300, 256, 5000, 5, wk.W_MXFP4),
                                          (129, 768, 3000, 32, wk.W_MXFP4), (70, 512, 2000, 64, wk.W_MXFP4),
                                          (1, 256, 130, 8, wk.W_MXFP4), (257, 768, 4099, 8, wk.W_E4M3),
                                          (1, 768, 130, 1, wk.W_E4M3), (600, 768, 20000, 5, wk.W_E4M3),
                                          (13, 768, 40, 8, wk.W_E4M3),
                                          # BF16 at D = 768: the scores of 600 queries against logits from
                                          # both BF16 forwards (256-row blocks tiled, the last 88 rows
                                          # stationary), bit for bit
                                          (257, 768, 4099, 8, wk.W_BF16), (1, 768, 130, 1, wk.W_BF16),
                                          (600, 768, 20000, 5, wk.W_BF16), (13, 768, 40, 8, wk.W_BF16),
                                          # D = 768, k <= 8 in MXFP4: the stationary-query scan
                                          (300, 768, 5000, 5, wk.W_E4M3), (257, 768, 4099, 8, wk.W_MXFP4),
                                          (1, 768, 130, 1, wk.W_MXFP4), (600, 768, 20000, 5, wk.W_MXFP4),
                                          (13, 768, 40, 8, wk.W_MXFP4)])
def test_topk_matches_oracle(elmo, orc, N, D, L, k, wfmt):
    wl = wk.scaled(wk.WORKLOADS["bf16_131k"], B=N, D=D, L=L, wfmt=wfmt)
    W0 = wk.make_weights(wl)
    X = wk.make_eval_x(wl, N)
    print(f"  topk N={N} D={D} L={L} k={k} wfmt={wfmt}", flush=True)
    Wd = to_dev_codes(W0)
    idx, sc = elmo.topk(Wd, _xdev(X), k, wfmt=wfmt)
    torch.cuda.synchronize()
    _check(elmo, orc, wfmt, W0, Wd, X, idx.cpu().numpy(), sc.cpu().numpy(), k)


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_topk_exact_ties_go_to_smaller_label(elmo, orc, wfmt):
    """Dyadic inputs with few bits make every logit exact; duplicated rows then tie exactly."""
    g = np.random.default_rng(3)
    N, D, L, k = 40, 128, 2000, 6
    xs = g.choice([-1.0, 0.0, 1.0], (N, D)) * 0.25
    ws = g.choice([-1.0, 0.0, 1.0], (L, D)) * 0.125
    for a, b in [(7, 100), (7, 1999), (3, 250), (1500, 20), (900, 901)]:
        ws[b] = ws[a]
    X = wk.to_bf16_codes(xs)
    W0 = wk.to_bf16_codes(ws) if wfmt == wk.W_BF16 else wk.to_e4m3_codes(ws)
    idx, sc = elmo.topk(to_dev_codes(W0), _xdev(X), k)
    idx_r, sc_r = orc.topk(wfmt, W0, X, k)
    assert np.array_equal(idx.cpu().numpy(), idx_r)
    assert np.array_equal(sc.cpu().numpy(), sc_r)


def test_topk_k1_is_argmax(elmo, orc):
    g = np.random.default_rng(4)
    xs = g.choice([-1.0, 1.0], (50, 64)) * 0.5
    ws = g.choice([-1.0, 0.0, 1.0], (1000, 64)) * 0.25
    X = wk.to_bf16_codes(xs); W0 = wk.to_bf16_codes(ws)
    idx, _ = elmo.topk(to_dev_codes(W0), _xdev(X), 1)
    S = xs @ ws.T
    assert np.array_equal(idx.cpu().numpy()[:, 0], np.argmax(S, axis=1))


def test_topk_nan_scores_rank_last(elmo, orc):
    wl = wk.scaled(wk.WORKLOADS["bf16_131k"], B=4, D=64, L=300, wfmt=wk.W_BF16)
    W0 = wk.make_weights(wl).copy()
    W0[:, 0] = 0x7FC0
    W0[10] = wk.to_bf16_codes(np.full(64, 0.01)); W0[200] = wk.to_bf16_codes(np.full(64, -0.01))
    X = wk.make_eval_x(wl, 4)
    idx, sc = elmo.topk(to_dev_codes(W0), _xdev(X), 4)
    idx_r, sc_r = orc.topk(wk.W_BF16, W0, X, 4)
    assert np.array_equal(idx.cpu().numpy(), idx_r)


@pytest.mark.parametrize("wfmt,D", [(wk.W_BF16, 64), (wk.W_E4M3, 64), (wk.W_MXFP4, 256), (wk.W_E4M3, 768),
                                    (wk.W_MXFP4, 768), (wk.W_BF16, 768)])
def test_topk_many_tiles_per_range(elmo, orc, wfmt, D):
    """4096 queries over 60k labels: each work-group scans some 30 label tiles, so the lists fill
    and later tiles take the bounded-candidate path (lists of up to 8). Its top-8 must equal, bit for
    bit, the first 8 of the top-32, and the top-32 the first 32 of the top-64 (lists of 32 and 64
    always take the full score-tile path; at D = 768 in MXFP4 the top-8 comes from the
    stationary-query scan, so this also checks the two scans against each other); sampled queries
    must match the oracle. Duplicated weight rows across tiles force exact ties."""
    N, L = 4096, 60000
    wl = wk.scaled(wk.WORKLOADS["bf16_131k"], B=N, D=D, L=L, wfmt=wfmt)
    W0 = wk.make_weights(wl).copy()
    for a, b in [(5, 40000), (12345, 129), (59999, 0), (777, 778)]:
        W0[b] = W0[a]
    X = wk.make_eval_x(wl, N)
    Wd, Xd = to_dev_codes(W0), _xdev(X)
    print(f"  topk N={N} D={D} L={L} wfmt={wfmt}", flush=True)
    i8, s8 = elmo.topk(Wd, Xd, 8, wfmt=wfmt)
    i32, s32 = elmo.topk(Wd, Xd, 32, wfmt=wfmt)
    i8, s8, i32, s32 = i8.cpu().numpy(), s8.cpu().numpy(), i32.cpu().numpy(), s32.cpu().numpy()
    assert np.array_equal(i32[:, :8], i8)
    assert np.array_equal(s32[:, :8].view(np.uint32), s8.view(np.uint32))
    qs = np.unique(np.concatenate([[0, 1, 127, 128, 2047, 4094, 4095], np.random.default_rng(9).integers(0, N, 25)]))
    _check(elmo, orc, wfmt, W0, Wd, X[qs], i8[qs], s8[qs], 8)
    i64, s64 = elmo.topk(Wd, Xd, 64, wfmt=wfmt)
    i64, s64 = i64.cpu().numpy(), s64.cpu().numpy()
    assert np.array_equal(i64[:, :32], i32)
    assert np.array_equal(s64[:, :32].view(np.uint32), s32.view(np.uint32))
