"""Device codec, stochastic rounding, RNG and gradient rule vs the CPU oracle, element by element
(bit-exact for every integer/code decision; the gradient code within the sigmoid's FP32 error)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def elmo():
    import precision_label_chunk_amd as m
    m.lib()
    return m


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _f32_sample(n, seed):
    g = np.random.default_rng(seed)
    bits = g.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    normal = (g.standard_normal(n) * 10.0 ** g.uniform(-12, 6, n)).astype(np.float32)
    x = np.concatenate([bits, normal, normal * 1e-30])
    return x[np.isfinite(x)].astype(np.float32)


def test_bf16_rne_bit_exact(elmo, orc):
    x = _f32_sample(300000, 1)
    base = np.random.default_rng(2).integers(0, 0x7F7F, 50000, dtype=np.uint32)
    x = np.concatenate([x, ((base << 16) | 0x8000).view(np.float32), ((base << 16) | 0x7FFF).view(np.float32),
                        np.array([np.inf, -np.inf, np.nan], np.float32)])
    got = elmo.numerics_probe(0, _dev(x)).cpu().numpy().view(np.uint16)
    ref = orc.bf16_rne(x)
    fin = np.isfinite(x)
    assert np.array_equal(got[fin], ref[fin])
    assert np.all(((got[~fin] & 0x7F80) == 0x7F80))


def test_e4m3_encode_bit_exact(elmo, orc):
    g = np.random.default_rng(3)
    v = orc.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = (v[:-1] + v[1:]) / 2
    x = np.concatenate([g.uniform(-600, 600, 100000), g.standard_normal(200000) * 10.0 ** g.uniform(-5, 2, 200000),
                        mids, -mids, v, -v, [448.0, 464.0, 1e30, -1e30, np.inf, -np.inf, 0.0, -0.0]])
    x32 = x.astype(np.float32)
    got = elmo.numerics_probe(1, _dev(x32)).cpu().numpy()
    ref = orc.e4m3_rne_sat(x32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_decode_every_code(elmo, orc):
    c = np.arange(256, dtype=np.uint8)
    got = elmo.numerics_probe(2, _dev(c)).cpu().numpy().astype(np.float64)
    ref = orc.e4m3_value(c)
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.all((got == ref) | both_nan) and np.isnan(got).sum() == 2


def test_e4m3_to_bf16_pairs_every_code(elmo, orc):
    """The paired decode the backward kernel stages its weight tiles with: every code in every byte."""
    c = np.arange(256, dtype=np.uint32)
    words = np.concatenate([c, c << 8, c << 16, c << 24, c | (c[::-1] << 8) | (c << 16) | (c[::-1] << 24)])
    got = elmo.numerics_probe(7, _dev(words.astype(np.uint32).view(np.int32))).cpu().numpy().view(np.uint32)
    codes = np.stack([(words >> (8 * k)) & 0xFF for k in range(4)], axis=1).astype(np.uint8)
    val = orc.e4m3_value(codes.ravel()).astype(np.float32)
    ref16 = torch.from_numpy(val).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).reshape(-1, 4)
    g16 = np.stack([got[0::2] & 0xFFFF, got[0::2] >> 16, got[1::2] & 0xFFFF, got[1::2] >> 16], axis=1)
    nan = np.isnan(val.reshape(-1, 4))
    assert np.array_equal(g16[~nan], ref16[~nan].astype(np.uint32))
    assert np.all((g16[nan] & 0x7FFF) > 0x7F80)


@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
def test_stochastic_rounding_bit_exact(elmo, orc, fmt):
    g = np.random.default_rng(4)
    n = 400000
    t = np.concatenate([(g.standard_normal(n) * 0.05), g.standard_normal(n // 4) * 10.0 ** g.uniform(-9, 2.7, n // 4),
                        [447.9, 448.0, 500.0, -1e9, 1e-45, -1e-40, 0.0, -0.0, 2.0**-6, 2.0**-9 * 0.5],
                        [np.inf, -np.inf, np.nan, -np.nan, 3e38, -3e38]]).astype(np.float32)
    r = g.integers(0, 65536, t.size).astype(np.uint32)
    r[:1000] = 0; r[1000:2000] = 65535
    op = 3 if fmt == "bf16" else 4
    got = elmo.numerics_probe(op, _dev(t), _dev(r)).cpu().numpy()
    if fmt == "bf16":
        got = got.view(np.uint16); ref = orc.sr_bf16(t, r)
        nan_g = (got & 0x7FFF) > 0x7F80; nan_r = (ref & 0x7FFF) > 0x7F80
    else:
        ref = orc.sr_e4m3(t, r)
        nan_g = (got & 0x7F) == 0x7F; nan_r = (ref & 0x7F) == 0x7F
    # a NaN input gives a NaN code (its sign and payload are not specified); everything else is exact
    assert np.array_equal(nan_g, nan_r) and nan_r.sum() == 2
    assert np.array_equal(got[~nan_r], ref[~nan_r])


@pytest.mark.parametrize("seed,step,idx0", [(0, 0, 0), (12345, 7, 3), (2**63 + 5, 2**40 + 1, 6_600_000_000 - 77)])
def test_rng_bit_exact(elmo, orc, seed, step, idx0):
    n = 100003
    got = elmo.numerics_probe(5, n=n, seed=seed, step=step, idx0=idx0).cpu().numpy().view(np.uint32)
    ref = orc.r16(seed, step, idx0, n)
    assert np.array_equal(got, ref)


def test_gradient_code_within_fp32_sigmoid_error(elmo, orc):
    g = np.random.default_rng(5)
    z = np.concatenate([g.standard_normal(100000) * 2, g.uniform(-60, 60, 50000), [0.0, 100.0, -100.0]]).astype(np.float32)
    y = (g.random(z.size) < 0.3).astype(np.uint32)
    got = elmo.numerics_probe(6, _dev(z), _dev(y)).cpu().numpy().view(np.uint16)
    ref = np.array([orc.grad_code(float(a), int(b)) for a, b in zip(z, y)], np.uint16)
    sg = np.where(got & 0x8000, -(got.astype(np.int64) & 0x7FFF), got.astype(np.int64) & 0x7FFF)
    sr = np.where(ref & 0x8000, -(ref.astype(np.int64) & 0x7FFF), ref.astype(np.int64) & 0x7FFF)
    d = np.abs(sg - sr)
    assert d.max() <= 1
    assert (d != 0).mean() <= 1e-3


@pytest.mark.parametrize("op,zmax,bound", [(8, 2.0, 4.0), (9, 80.0, 3.0)])
def test_gradient_forms_within_stated_ulps(elmo, op, zmax, bound):
    """The forward's two fast gradient forms in binary32 against sigmoid(z) - y in binary64
    (the cancellation-free -sigmoid(-z) for y = 1), in units of the binary32 spacing at the exact
    value: the small-argument form over |z| <= 2, the split-exponent form over |z| <= 80."""
    from scipy.special import expit
    g = np.random.default_rng(9)
    z = np.concatenate([g.uniform(-zmax, zmax, 200000), g.standard_normal(50000) * min(zmax, 2.0) / 2,
                        [0.0, zmax, -zmax, 1e-30, -1e-30]]).astype(np.float32)
    z = np.clip(z, -zmax, zmax)
    y = (g.random(z.size) < 0.5).astype(np.uint32)
    got = elmo.numerics_probe(op, _dev(z), _dev(y)).cpu().numpy().astype(np.float64)
    zd = z.astype(np.float64)
    ref = np.where(y == 1, -expit(-zd), expit(zd))
    ulps = np.abs(got - ref) / np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    print(f"op {op}: max {ulps.max():.3f} ulp, mean {ulps.mean():.3f}")
    assert np.all(np.isfinite(got)) and ulps.max() <= bound
