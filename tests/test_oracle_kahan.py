"""Pins of the oracle's Kahan-compensated BF16 update (encoder parameters; ELMO summary,
Approach: the encoder is trained with Kahan summation, no FP32 master weights): a sequence worked
by hand from the definition, the compensation property (Kahan keeps the sum that plain BF16 SGD
loses), exact cases where the compensation stays zero, and sign symmetry."""
import os

import numpy as np

import oracle as orc

HERE = os.path.dirname(os.path.abspath(__file__))


def _bf16(x):
    return orc.bf16_rne(np.asarray(x, np.float32))


def _val(codes):
    return orc.bf16_value(np.asarray(codes, np.uint16))


def test_hand_worked_sequence():
    rows = [ln.split() for ln in open(os.path.join(HERE, "golden", "kahan_bf16_steps.txt"))
            if ln.strip() and not ln.startswith("#")]
    w = np.array([0x3F80], np.uint16); c = np.array([0], np.uint16)
    for k, (step, wc, cc) in enumerate(rows, start=1):
        assert int(step) == k
        w, c = orc.kahan_update(w, c, np.array([-1.0], np.float32), 2.0 ** -10)
        assert (int(w[0]), int(c[0])) == (int(wc, 16), int(cc, 16)), (k, hex(w[0]), hex(c[0]))
        assert float(_val(w)[0]) - float(_val(c)[0]) == 1.0 + k * 2.0 ** -10


def test_compensation_keeps_what_plain_bf16_loses():
    """Increments of 0.2-0.45 of a BF16 spacing: plain BF16 SGD never moves, while the parameter
    stays within two spacings of the exact binary64 sum. The pair w - c is the sum up to the
    rounding of c to BF16: |c| stays below about half a spacing of w (2^-8 in [1, 2)), so each step
    adds at most half a BF16 unit of c, 2^-16, to the error of w - c."""
    g = np.random.default_rng(11)
    n, steps = 512, 600
    w0 = g.uniform(1.0, 2.0, n)
    w = _bf16(w0); c = np.zeros(n, np.uint16)
    spacing = 2.0 ** -7                                   # BF16 spacing in [1, 2)
    lr = np.float32(2.0 ** -12)
    exact = _val(w).astype(np.float64)
    plain = w.copy()
    for _ in range(steps):
        d = g.uniform(0.2, 0.45, n) * spacing
        grad = (-(d / float(lr))).astype(np.float32)    # -lr * grad = d up to binary32 rounding
        dd = (-lr * grad).astype(np.float32).astype(np.float64)
        exact += dd
        w, c = orc.kahan_update(w, c, grad, lr)
        plain = _bf16(_val(plain).astype(np.float32) + dd.astype(np.float32))
    err_kahan = np.abs(_val(w) - _val(c) - exact)
    err_w = np.abs(_val(w) - exact)
    moved = np.abs(_val(plain) - _val(_bf16(w0)))
    assert np.all(moved == 0.0)                           # plain BF16 SGD stalls
    assert exact.max() - exact.min() > 0 and np.all(exact - _val(_bf16(w0)) > 0.5)
    assert np.all(err_w <= spacing * 2)                   # the parameter follows the true sum
    assert np.all(err_kahan <= steps * 2.0 ** -16)        # bound from the rounding of c
    err_plain = np.abs(_val(plain) - exact)
    assert err_kahan.mean() < 1e-3 * err_plain.mean()


def test_exact_increments_leave_compensation_zero():
    """w integers, d integers: every w + y is representable, so c stays 0 and w is the plain sum."""
    w = _bf16(np.arange(-50, 50, dtype=np.float32)); c = np.zeros(100, np.uint16)
    for s in range(5):
        grad = np.full(100, -(s + 1), np.float32)
        w, c = orc.kahan_update(w, c, grad, 1.0)
    assert np.all(c == 0)
    assert np.array_equal(_val(w), np.arange(-50, 50) + 15.0)


def test_sign_symmetry():
    g = np.random.default_rng(5)
    n = 4096
    w = _bf16(g.normal(0, 0.05, n).astype(np.float32)); c = _bf16(g.normal(0, 1e-4, n).astype(np.float32))
    grad = g.normal(0, 1.0, n).astype(np.float32)
    w1, c1 = orc.kahan_update(w, c, grad, 1e-3)
    w2, c2 = orc.kahan_update(w ^ 0x8000, c ^ 0x8000, -grad, 1e-3)
    nz = (_val(w1) != 0) & (_val(c1) != 0)
    assert np.array_equal((w2 ^ 0x8000)[nz], w1[nz]) and np.array_equal((c2 ^ 0x8000)[nz], c1[nz])
