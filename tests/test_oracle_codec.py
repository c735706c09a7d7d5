"""Pins of the oracle's BF16 and OCP-E4M3 codecs against PyTorch's casts and the format tables.

The pages name the formats ("pure BF16 or FP8", "E4M3 native range suffices": ELMO summary page,
"Approach" and "Surprising findings"); the OCP E4M3FN reading (max 448, no infinity) is checked
against torch.float8_e4m3fn, an independent implementation.
"""
import numpy as np
import pytest
import torch


def _torch_bf16_to_f64(codes):
    return torch.from_numpy(codes.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def _torch_e4m3_to_f64(codes):
    return torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _same(a, b):
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    return bool(np.all((a == b) | both_nan) and np.all((np.signbit(a) == np.signbit(b)) | both_nan))


def test_bf16_decode_every_code(orc):
    codes = np.arange(65536, dtype=np.uint16)
    assert _same(orc.bf16_value(codes), _torch_bf16_to_f64(codes))


def test_bf16_rne_matches_torch_random_and_midpoints(orc):
    g = np.random.default_rng(1)
    # random binary32 bit patterns over the whole range, plus a normal-ish sample
    x = np.concatenate([g.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
                        g.standard_normal(100000).astype(np.float32) * 10.0 ** g.integers(-40, 38, 100000)])
    x = x[np.isfinite(x)].astype(np.float32)
    # exact midpoints between neighbouring BF16 values (ties) and one binary32 ulp either side
    base = g.integers(0, 0x7F7F, 50000, dtype=np.uint32)
    mid = ((base << 16) | 0x8000).view(np.float32)
    lo = ((base << 16) | 0x7FFF).view(np.float32)
    hi = ((base << 16) | 0x8001).view(np.float32)
    x = np.concatenate([x, mid, lo, hi, -mid, -lo, -hi])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.bf16_rne(x)
    assert np.array_equal(got, ref)


def test_bf16_rne_ties_go_to_even(orc):
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even is 1.0; 1 + 3*2^-8 goes up to 1.015625
    assert orc.bf16_value(orc.bf16_rne(np.float32(1 + 2**-8)))[()] == 1.0
    assert orc.bf16_value(orc.bf16_rne(np.float32(1 + 3 * 2**-8)))[()] == 1.015625
    # overflow past the largest BF16 rounds to infinity, as IEEE 754
    big = np.float32(np.finfo(np.float32).max)
    assert orc.bf16_rne(big)[()] == 0x7F80
    # NaN stays NaN with its sign
    n = orc.bf16_rne(np.array([np.nan, -np.nan], np.float32))
    assert np.all(np.isnan(orc.bf16_value(n)))


def test_e4m3_decode_every_code(orc):
    codes = np.arange(256, dtype=np.uint8)
    assert _same(orc.e4m3_value(codes), _torch_e4m3_to_f64(codes))


def test_e4m3_format_table(orc):
    v = orc.e4m3_value(np.arange(256, dtype=np.uint8))
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x01] == 2.0**-9 and v[0x08] == 2.0**-6 and v[0x38] == 1.0
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)       # codes ascend with value
    assert torch.finfo(torch.float8_e4m3fn).max == 448.0


def test_e4m3_roundtrip_every_code(orc):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(orc.e4m3_rne_sat(orc.e4m3_value(codes)), codes)


def test_e4m3_rne_matches_torch_below_464(orc):
    g = np.random.default_rng(2)
    v = orc.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = (v[:-1] + v[1:]) / 2                 # exact ties between neighbours
    eps = np.diff(v) * 1e-3
    x = np.concatenate([g.uniform(-463.9, 463.9, 100000),
                        g.standard_normal(100000) * 10.0 ** g.uniform(-4, 2, 100000),
                        mids, -mids, mids + eps, mids - eps, -(mids + eps), v, -v])
    x = x[np.abs(x) < 464]
    ref = torch.from_numpy(x.astype(np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.e4m3_rne_sat(x)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("x,code", [(448.0, 0x7E), (450.0, 0x7E), (464.0, 0x7E), (500.0, 0x7E),
                                    (1e30, 0x7E), (np.inf, 0x7E), (-np.inf, 0xFE), (-1e9, 0xFE),
                                    (-0.0, 0x80), (0.0, 0x00), (2.0**-10, 0x00), (3 * 2.0**-11, 0x01)])
def test_e4m3_saturates_and_keeps_sign(orc, x, code):
    assert orc.e4m3_rne_sat(np.array([x]))[0] == code


def test_e4m3_nan(orc):
    assert orc.e4m3_rne_sat(np.array([np.nan]))[0] in (0x7F, 0xFF)
