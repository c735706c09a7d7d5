"""Pins of the oracle's MX-scaled FP4 weights (OCP Microscaling: 32 E2M1 elements share one E8M0
scale; the summary page's Limitations name FP4 weights as the recipe gap that needs micro-tensor
scaling). The element and scale codecs against their closed forms over every code; the stochastic
rounding to E2M1 exhaustively over the 16-bit draw; the block exponent's closed form and edge cases;
block quantisation invariants; and a whole MXFP4 step with exact arithmetic predicted without the
oracle."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as wk

W_MX = wk.W_MXFP4
MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def test_e2m1_every_code(orc):
    # s ee m, exponent bias 1, exponent 0 subnormal: (-1)^s m / 2; else (-1)^s 2^(e - 1) (1 + m / 2)
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = m / 2 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        assert orc.e2m1_value(np.uint8(c)) == (-v if s else v), c
    assert sorted({abs(float(orc.e2m1_value(np.uint8(c)))) for c in range(16)}) == [float(m) for m in MAGS]


def test_e8m0_every_code(orc):
    v = orc.e8m0_value(np.arange(256, dtype=np.uint8))
    assert np.isnan(v[255])
    assert np.array_equal(v[:255], 2.0 ** (np.arange(255) - 127))


@pytest.mark.parametrize("v", [0.1, 0.5, 0.6, 1.2, 1.75, 2.5, 3.3, 4.0001, 5.9, -0.3, -2.2, -5.0])
def test_sr_e2m1_exhaustive_over_the_draw(orc, v):
    """Counting the draws r in [0, 2^16) that round |v| up must give exactly q = floor(frac * 2^16)."""
    a = Fraction(abs(v))
    lo = max(m for m in MAGS if m <= a)
    hi = MAGS[MAGS.index(lo) + 1]
    q = int((a - lo) / (hi - lo) * 65536)
    codes = orc.sr_e2m1(np.full(65536, v), np.arange(65536, dtype=np.uint32))
    vals = orc.e2m1_value(codes)
    sign = -1 if v < 0 else 1
    ups = int((vals == sign * float(hi)).sum())
    assert ups == q and int((vals == sign * float(lo)).sum()) == 65536 - q
    # the draws that round up are the top q of them (r >= 2^16 - q)
    assert np.all(vals[65536 - q:] == sign * float(hi))


def test_sr_e2m1_identities_and_saturation(orc):
    r = np.random.default_rng(0).integers(0, 65536, 200, dtype=np.uint32)
    for c in range(16):
        v = float(orc.e2m1_value(np.uint8(c)))
        assert np.all(orc.e2m1_value(orc.sr_e2m1(np.full(200, v), r)) == v)    # representable: itself
    for v in (6.0, 6.5, 7.99, 1e30, np.inf):
        assert np.all(orc.sr_e2m1(np.full(200, v), r) == 7)
        assert np.all(orc.sr_e2m1(np.full(200, -v), r) == 15)
    assert orc.sr_e2m1(np.array([-0.0]), np.array([65535], np.uint32))[0] == 8      # -0 keeps its sign


def test_sr_e2m1_is_unbiased(orc):
    g = np.random.default_rng(1)
    r = g.integers(0, 65536, 10 ** 6, dtype=np.uint32)
    for v in (0.3, 1.1, 2.7, 4.4, -3.6):
        m = orc.e2m1_value(orc.sr_e2m1(np.full(r.size, v), r)).mean()
        assert abs(m - v) <= 1e-3 * abs(v)


def test_block_exponent(orc):
    # X = floor(log2 amax) - 2: amax / 2^X lands in [4, 8)
    for amax, x in [(6.0, 0), (4.0, 0), (3.99, -1), (8.0, 1), (7.99, 0), (0.02, -8), (1.0, -2),
                    (3.0e38, 125), (1e-40, -127), (0.0, -127)]:
        assert orc.mx_block_exponent(np.float32(amax)) == x, amax
    assert orc.mx_block_exponent(np.float32(np.inf)) == 127
    assert orc.mx_block_exponent(np.float32(np.nan)) == 128
    g = np.random.default_rng(2)
    for a in g.uniform(1e-6, 1e6, 500).astype(np.float32):
        x = orc.mx_block_exponent(a)
        assert 4 <= float(a) / 2.0 ** x < 8


def test_quantize_block(orc):
    g = np.random.default_rng(3)
    r = g.integers(0, 65536, 32, dtype=np.uint32)
    # exactly representable blocks come back unchanged whatever the draws
    codes = g.integers(0, 16, 32).astype(np.uint8); codes[5] = 7       # one magnitude 6: amax = 6 * 2^x
    for x in (-9, 0, 3):
        t = (orc.e2m1_value(codes) * 2.0 ** x).astype(np.float32)
        c, sc = orc.mx_quantize_block(t, r)
        assert sc == x + 127
        assert np.array_equal(orc.e2m1_value(c), orc.e2m1_value(codes))
    # a power-of-two rescaling moves only the scale
    t = g.normal(0, 0.02, 32).astype(np.float32)
    c0, s0 = orc.mx_quantize_block(t, r)
    c1, s1 = orc.mx_quantize_block(t * np.float32(2.0 ** 5), r)
    assert np.array_equal(c0, c1) and s1 == s0 + 5
    # the decoded block is within one grid spacing of t, and its largest magnitude in [4, 8) saturates
    v = orc.e2m1_value(c0) * 2.0 ** (s0 - 127)
    assert np.all(np.abs(v - t) <= 2.0 * 2.0 ** (s0 - 127))
    # a NaN makes the whole block NaN (scale 255); an all-zero block keeps its signed zeros
    tn = t.copy(); tn[7] = np.nan
    assert orc.mx_quantize_block(tn, r)[1] == 255
    cz, sz = orc.mx_quantize_block(np.where(np.arange(32) % 2, -0.0, 0.0).astype(np.float32), r)
    assert sz == 0 and np.array_equal(cz, np.where(np.arange(32) % 2, 8, 0))


def test_mxfp4_layout_and_contractions(orc):
    """Row layout (codes two per byte, low nibble first, then one scale per 32) against a direct
    decode, and the logits / dX of the step against numpy's binary64 matmul of the decoded operands."""
    wl = wk.scaled(wk.WORKLOADS["mxfp4_3m"], B=7, D=128, L=90, lam=3.0)
    W = wk.make_weights(wl)
    bt = wk.make_batch(wl)
    L, D = orc.dims(W_MX, W)
    assert (L, D) == (90, 128) and W.shape == (90, 68)
    vals = orc.mx_decode(W)
    for j, k in [(0, 0), (0, 1), (5, 77), (89, 127), (40, 64)]:
        byte = int(W[j, k // 2]); code = (byte >> 4) if k & 1 else (byte & 15)
        assert vals[j, k] == float(orc.e2m1_value(np.uint8(code))) * 2.0 ** (int(W[j, D // 2 + k // 32]) - 127)
    Wn, dX, _, Z, G = orc.step(W_MX, W, bt.X, bt.row_ptr, bt.ids, wl.lr, 1, 0, want_z=True, want_g=True)
    x = torch.from_numpy(bt.X.view(np.int16)).view(torch.bfloat16).double().numpy()
    xt = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()   # E4M3 forward operand
    assert np.array_equal(Z, (xt @ vals.T).astype(np.float32))
    g = torch.from_numpy(G.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.allclose(dX, g @ vals, rtol=1e-6, atol=1e-9)
    assert Wn.shape == W.shape


def test_saturated_dyadic_mxfp4_step_is_predicted(orc):
    """X, W dyadic with a dominant first feature: |z| >= 116, G in {0, +-1}, every sum exact, so t is
    exact and each block's scale and codes follow from the rule by exact rational arithmetic and the
    element draws (the oracle's generator, pinned against rocRAND elsewhere)."""
    g = np.random.default_rng(11)
    B, D, L = 8, 64, 40
    lr, seed, step = 2.0 ** -6, 5, 3
    xs = g.choice([-1.0, 1.0], (B, D)) * 0.125
    xs[:, 0] = g.choice([-128.0, 128.0], B)
    codes = g.integers(0, 16, (L, D)).astype(np.uint8)
    codes[:, 0] = g.choice([4, 12], L)                 # +-2 in feature 0 (scale 2^-1: +-1)
    W = np.empty((L, D // 2 + D // 32), np.uint8)
    W[:, :D // 2] = codes[:, 0::2] | (codes[:, 1::2] << 4)
    W[:, D // 2:] = 126                                # scale 2^-1
    ws = orc.mx_decode(W)
    X = wk.to_bf16_codes(xs)
    Y = g.random((B, L)) < 0.2
    rp = np.zeros(B + 1, np.int32); rp[1:] = np.cumsum(Y.sum(1))
    ids = np.concatenate([np.nonzero(Y[b])[0] for b in range(B)]).astype(np.int32)
    Wn, dX, _, Z, _ = orc.step(W_MX, W, X, rp, ids, lr, seed, step, want_z=True)
    xt = torch.from_numpy(xs.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
    z = xt @ ws.T
    assert np.all(np.abs(z) >= 116) and np.array_equal(Z, z.astype(np.float32))
    gexp = (z > 0).astype(np.float64) - Y
    t = ws - lr * (gexp.T @ xs)                        # exact dyadic values
    R = orc.r16(seed, step, 0, L * D).reshape(L, D)
    for j in range(L):
        for b in range(D // 32):
            blk = [Fraction(float(v)) for v in t[j, 32 * b:32 * b + 32]]
            amax = max(abs(v) for v in blk)
            x = int(np.floor(np.log2(float(amax)))) - 2 if amax else -127
            assert int(Wn[j, D // 2 + b]) == x + 127
            for k in range(32):
                a = abs(blk[k]) / Fraction(2) ** x
                if a >= 6:
                    mag = 6
                else:
                    lo = max(m for m in MAGS if m <= a)
                    if lo == a:
                        mag = lo
                    else:
                        hi = MAGS[MAGS.index(lo) + 1]
                        q = int((a - lo) / (hi - lo) * 65536)
                        mag = hi if q + int(R[j, 32 * b + k]) >= 65536 else lo
                kk = 32 * b + k
                byte = int(Wn[j, kk // 2]); code = (byte >> 4) if kk & 1 else (byte & 15)
                got = float(orc.e2m1_value(np.uint8(code)))
                assert abs(got) == float(mag) and (got == 0 or (got < 0) == (blk[k] < 0)), (j, kk)
