"""Pins of the oracle's stochastic rounding (SR) of the classifier update.

The pages say the classifier is updated with stochastic rounding in pure BF16/FP8 (ELMO summary
page, "Approach"; arXiv abstract) but give no mechanism. The reading: round the magnitude up with
probability equal to its fractional position between the two neighbouring format values, decided
by a 16-bit uniform integer. Pinned here by exhaustive enumeration over all 2^16 random values
(exact counts computed with rational arithmetic from the torch-decoded format tables) and by the
unbiasedness requirement (mean of 10^6 draws within 1e-3 relative of the input).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

R_ALL = np.arange(65536, dtype=np.uint32)


def _bf16_table():
    v = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).to(torch.float64).numpy()
    return v  # all finite non-negative BF16 magnitudes, ascending


def _e4m3_table():
    return torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _expected_up_count(t, table):
    a = Fraction(abs(float(t)))
    i = int(np.searchsorted(table, float(a), side="right")) - 1
    lo, hi = Fraction(float(table[i])), Fraction(float(table[i + 1]))
    q = int((a - lo) / (hi - lo) * 65536)  # floor of a non-negative rational
    return q, float(lo), float(hi)


def _bf16_val(codes):
    return torch.from_numpy(codes.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def _e4m3_val(codes):
    return torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


BF16_TS = [0.1, -0.1, 1.0 + 2**-9, 3.14159, -2.71828e-3, 1e-30, 6.1e-39, 1e30, 0.02 - 7.3e-6,
           np.float32(1 + 2**-7 - 2**-23), np.float32(2**-126 * 1.3)]
E4M3_TS = [0.1, -0.1, 0.0137, 1.0 + 2**-5, 300.0, 440.0, -447.9, 2.0**-9 * 0.3, 2.0**-7 * 1.1,
           0.0197, -0.004, 2.0**-6 * 0.99]


@pytest.mark.parametrize("t", BF16_TS)
def test_sr_bf16_exhaustive_over_r(orc, t):
    t = np.float32(t)
    q, lo, hi = _expected_up_count(t, _bf16_table())
    out = _bf16_val(orc.sr_bf16(np.full(65536, t, np.float32), R_ALL))
    sgn = -1.0 if t < 0 else 1.0
    up = out == sgn * hi
    assert np.all(up | (out == sgn * lo))
    assert up.sum() == q
    # monotone threshold: exactly the largest q values of r round up
    assert np.all(up == (R_ALL >= 65536 - q))


@pytest.mark.parametrize("t", E4M3_TS)
def test_sr_e4m3_exhaustive_over_r(orc, t):
    t = np.float32(t)
    q, lo, hi = _expected_up_count(t, _e4m3_table())
    out = _e4m3_val(orc.sr_e4m3(np.full(65536, t, np.float32), R_ALL))
    sgn = -1.0 if t < 0 else 1.0
    up = out == sgn * hi
    assert np.all(up | (out == sgn * lo))
    assert up.sum() == q
    assert np.all(up == (R_ALL >= 65536 - q))


def test_sr_of_representable_values_is_identity(orc):
    bf = _bf16_table()[::97].astype(np.float32)
    for t in np.concatenate([bf, -bf]):
        out = orc.sr_bf16(np.full(4096, t, np.float32), R_ALL[::16])
        assert np.all(_bf16_val(out) == t)
    e4 = _e4m3_table().astype(np.float32)
    for t in np.concatenate([e4, -e4]):
        out = orc.sr_e4m3(np.full(4096, t, np.float32), R_ALL[::16])
        assert np.all(_e4m3_val(out) == t)


def test_sr_e4m3_saturates(orc):
    t = np.array([448.0, 449.0, 1e4, np.inf, -500.0, -np.inf], np.float32)
    out = orc.sr_e4m3(t, np.full(t.shape, 65535, np.uint32))
    assert list(out) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert orc.sr_e4m3(np.array([np.nan], np.float32), np.array([0], np.uint32))[0] in (0x7F, 0xFF)


def test_sr_sign_symmetry(orc):
    g = np.random.default_rng(3)
    t = (g.standard_normal(20000) * 0.05).astype(np.float32)
    r = g.integers(0, 65536, t.size).astype(np.uint32)
    assert np.array_equal(orc.sr_bf16(-t, r), orc.sr_bf16(t, r) ^ 0x8000)
    assert np.array_equal(orc.sr_e4m3(-t, r), orc.sr_e4m3(t, r) ^ 0x80)


@pytest.mark.parametrize("fmt,t", [("bf16", 0.0123457), ("bf16", -1.2345), ("bf16", 3.3e-3),
                                   ("e4m3", 0.0197), ("e4m3", -0.11), ("e4m3", 2.0**-6 * 1.37),
                                   ("e4m3", 37.3)])
def test_sr_unbiased_over_1e6_draws(orc, fmt, t):
    """Mean of 10^6 stochastic roundings (random bits from the oracle's counter-based RNG) within
    1e-3 relative of the input."""
    n = 10**6
    r = orc.r16(seed=12345, step=7, idx0=0, n=n)
    tt = np.full(n, t, np.float32)
    vals = _bf16_val(orc.sr_bf16(tt, r)) if fmt == "bf16" else _e4m3_val(orc.sr_e4m3(tt, r))
    mean = vals.mean(dtype=np.float64)
    assert abs(mean - float(np.float32(t))) <= 1e-3 * abs(float(np.float32(t)))


def test_sr_unbiased_e4m3_subnormal_within_4_sigma(orc):
    # a relative 1e-3 bound is statistically out of reach where the E4M3 spacing (2^-9) dwarfs t
    n = 10**6
    t = np.float32(1e-4)
    r = orc.r16(seed=99, step=0, idx0=0, n=n)
    vals = _e4m3_val(orc.sr_e4m3(np.full(n, t, np.float32), r))
    p = float(t) / 2.0**-9
    sigma = 2.0**-9 * np.sqrt(p * (1 - p) / n)
    assert abs(vals.mean() - float(t)) <= 4 * sigma
