"""The seeded input generators, pinned to the recipe they implement (CPU only).

The workloads stand in for the label spaces named on the ELMO summary page ("Experimental setup"):
their sizes are fixed here, and the distributions are checked against closed forms and against
library routines that compute the same quantity another way:
  * the finite Zipf law's head probability against the generalised harmonic number (digamma for
    s = 1, Riemann minus Hurwitz zeta for s > 1, from scipy), and its rank frequencies against the
    law by a chi-square test;
  * label rows: distinct, sorted, in range, 1 + Poisson(lam) positives (uniform 1..8 for the tiny
    case);
  * features: unit-norm rows (N(0, 1)/sqrt(D) for the tiny case), up to the BF16 cast;
  * the streams are deterministic per (workload, purpose, step) and differ between them.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
from scipy import special, stats

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import workloads as wk  # noqa: E402


def _bf16_to_f64(codes):
    return (codes.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("name,B,D,L,chunk,wfmt", [
    ("tiny", 32, 64, 4096, 1024, wk.W_BF16),
    ("bf16_131k", 256, 768, 131072, 32768, wk.W_BF16),
    ("bf16_670k", 256, 768, 670000, 65536, wk.W_BF16),
    ("e4m3_3m", 256, 768, 3000000, 131072, wk.W_E4M3),
    ("bf16_8p6m", 128, 768, 8600000, 262144, wk.W_BF16),
])
def test_workload_sizes(name, B, D, L, chunk, wfmt):
    w = wk.WORKLOADS[name]
    assert (w.B, w.D, w.L, w.chunk, w.wfmt) == (B, D, L, chunk, wfmt)
    if name == "bf16_8p6m":
        assert (w.topk, w.n_eval) == (5, 4096)


@pytest.mark.parametrize("name,share", [("bf16_131k", 0.13), ("bf16_670k", 0.07), ("e4m3_3m", 0.065),
                                        ("bf16_8p6m", 0.19)])
def test_zipf_head_probability_is_one_over_generalised_harmonic(name, share):
    w = wk.WORKLOADS[name]
    z = wk.zipf_for(w)
    if w.zipf_s == 1.0:
        h = special.digamma(w.L + 1) + np.euler_gamma              # H_L
    else:
        h = special.zeta(w.zipf_s) - special.zeta(w.zipf_s, w.L + 1)  # sum_{r <= L} r^-s
    assert z.cdf[0] == pytest.approx(1.0 / h, rel=1e-9)
    assert z.cdf[-1] == 1.0
    assert abs(z.cdf[0] - share) < 0.006                           # the head label's share


@pytest.mark.parametrize("L,s", [(40, 1.0), (60, 1.3)])
def test_zipf_rank_frequencies_follow_the_law(L, s):
    z = wk.ZipfSampler(L, s)
    g = np.random.default_rng(11)
    n = 400_000
    r = z.draw(g, n)
    assert r.min() >= 0 and r.max() < L
    p = np.arange(1, L + 1, dtype=np.float64) ** -s
    p /= p.sum()
    obs = np.bincount(r, minlength=L)
    chi2 = ((obs - n * p) ** 2 / (n * p)).sum()
    assert stats.chi2.sf(chi2, L - 1) > 1e-4


def test_zipf_label_rows():
    g = np.random.default_rng(3)
    L, lam, B = 100_000, 5.0, 4000
    rp, ids = wk.make_labels(B, L, "zipf", g, lam=lam, zipf=wk.ZipfSampler(L, 1.0))
    assert rp.dtype == np.int32 and ids.dtype == np.int32 and rp[0] == 0 and rp[-1] == ids.size
    cnt = np.diff(rp)
    assert cnt.min() >= 1
    for b in range(B):
        row = ids[rp[b]:rp[b + 1]]
        assert np.all(np.diff(row) > 0) and row[0] >= 0 and row[-1] < L
    # 1 + Poisson(lam): mean 1 + lam, variance lam
    assert abs(cnt.mean() - (1 + lam)) < 5 * np.sqrt(lam / B)
    assert abs(cnt.var() / lam - 1) < 0.1
    # the head label (id 0) appears in about the share the law gives a row of that many draws
    assert (ids == 0).sum() > 0.2 * B


def test_zipf_rows_are_capped_at_the_label_count():
    g = np.random.default_rng(4)
    rp, ids = wk.make_labels(50, 6, "zipf", g, lam=20.0, zipf=wk.ZipfSampler(6, 1.0))
    cnt = np.diff(rp)
    assert cnt.max() <= 6 and (cnt == 6).mean() > 0.9


def test_uniform_label_rows():
    g = np.random.default_rng(5)
    rp, ids = wk.make_labels(8000, 4096, "uniform", g, max_pos=8)
    cnt = np.diff(rp)
    assert cnt.min() == 1 and cnt.max() == 8
    assert np.abs(np.bincount(cnt, minlength=9)[1:] / 8000 - 1 / 8).max() < 0.02
    for b in range(0, 8000, 97):
        row = ids[rp[b]:rp[b + 1]]
        assert np.all(np.diff(row) > 0) and row[0] >= 0 and row[-1] < 4096


def test_features():
    g = np.random.default_rng(6)
    x = _bf16_to_f64(wk.make_x(300, 768, "rownorm", g))
    assert np.abs(np.linalg.norm(x, axis=1) - 1).max() < 2 ** -8
    x = _bf16_to_f64(wk.make_x(300, 64, "gauss_sqrtD", g))
    assert abs(x.var() * 64 - 1) < 0.03 and abs(x.mean()) < 0.01
    with pytest.raises(ValueError):
        wk.make_x(2, 64, "other", g)


@pytest.mark.parametrize("wfmt", [wk.W_BF16, wk.W_E4M3])
def test_weights(wfmt):
    w = wk.make_w(2000, 64, wfmt, np.random.default_rng(7))
    if wfmt == wk.W_BF16:
        v = _bf16_to_f64(w)
        assert abs(v.std() / 0.02 - 1) < 0.01
    else:
        assert w.dtype == np.uint8 and not np.any((w & 0x7F) == 0x7F)    # no NaN codes
        sub = ((w >> 3) & 0xF) == 0
        assert sub.mean() > 0.5                                          # over half subnormal


def test_streams_are_deterministic_and_distinct():
    w = wk.scaled(wk.WORKLOADS["bf16_131k"], L=5000, B=16)
    a, b = wk.make_batch(w, 0), wk.make_batch(w, 0)
    assert np.array_equal(a.X, b.X) and np.array_equal(a.row_ptr, b.row_ptr) and np.array_equal(a.ids, b.ids)
    c = wk.make_batch(w, 1)
    assert not np.array_equal(a.X, c.X)
    other = wk.scaled(wk.WORKLOADS["bf16_670k"], L=5000, B=16)
    assert not np.array_equal(a.X, wk.make_batch(other, 0).X)
    assert not np.array_equal(wk.make_eval_x(w, 16), a.X)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
