"""Device numerics of the MX-scaled FP4 weights against the oracle, bit for bit: the stochastic
rounding to E2M1 (the hardware's scaled conversion, with the rule it follows pinned over every
range and scale), the block quantisation (shared exponent and elements), the E2M1 -> BF16 decode
with a block scale, and the scaled FP4 MFMA's operand layout."""
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


def test_sr_e2m1_bit_exact(elmo, orc):
    g = np.random.default_rng(1)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    v = np.concatenate([g.uniform(-8, 8, 40000), g.normal(0, 1, 20000), np.tile(grid, 100), -np.tile(grid, 100),
                        np.array([6.0, 7.999, 1e30, -1e30, np.inf, -np.inf, 1e-40, -1e-40, 0.0, -0.0, 5.9999995])]
                       ).astype(np.float32)
    r = g.integers(0, 65536, v.size, dtype=np.uint32)
    r[:200] = 0; r[200:400] = 65535
    got = elmo.numerics_probe(10, _dev(v), _dev(r)).cpu().numpy()
    ref = orc.sr_e2m1(v.astype(np.float64), r)
    assert np.array_equal(got, ref), np.nonzero(got != ref)[0][:10]


def _hw_convert(elmo, v0, v1, rnd, scale):
    n = v0.size
    a = np.empty(2 * n, np.float32); a[0::2] = v0; a[1::2] = v1
    b = np.empty(2 * n, np.uint32); b[0::2] = rnd
    b[1::2] = np.full(n, np.float32(scale), np.float32).view(np.uint32)
    return elmo.numerics_probe(14, _dev(a), _dev(b.view(np.int32))).cpu().numpy().view(np.uint32) & 0xFF


@pytest.mark.parametrize("X", [-127, -126, -60, -3, 0, 7, 126, 127])
def test_hw_sr_fp4_conversion_rule(elmo, orc, X):
    """The first value of the scaled FP4 conversion's pair, divided by the scale 2^X and rounded with
    the draw in bits 31..16 of the random operand (bits 15..0 zero), is the oracle's SR(t / 2^X) for
    every value range, signed zeros, subnormal inputs and infinities; the second value takes the
    operand shifted left by one bit (so two independent draws cannot share one conversion)."""
    g = np.random.default_rng(200 + X)
    a = np.concatenate([g.uniform(-8, 8, 60000), g.uniform(-1, 1, 20000), g.uniform(-2.0**-10, 2.0**-10, 5000),
                        np.tile(orc.e2m1_value(np.arange(16, dtype=np.uint8)), 50)])
    t = np.ldexp(a, X).astype(np.float32)
    t = np.concatenate([t, np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, -1e-40, np.inf, -np.inf], np.float32)])
    r16 = g.integers(0, 65536, t.size, dtype=np.uint32)
    got = _hw_convert(elmo, t, np.zeros_like(t), r16 << 16, np.ldexp(1.0, X))
    exact = np.ldexp(t.astype(np.float64), -X)
    assert np.array_equal(got & 15, orc.sr_e2m1(exact, r16))
    assert np.all(got >> 4 == 0)                                        # +0 in the second slot
    # the second slot: the same random operand shifted left by one bit
    rnd = g.integers(0, 2 ** 32, t.size, dtype=np.uint64).astype(np.uint32) & np.uint32(0xFFFF8000)
    got2 = _hw_convert(elmo, np.zeros_like(t), t, rnd, np.ldexp(1.0, X))
    assert np.array_equal(got2 >> 4, orc.sr_e2m1(exact, (rnd << 1) >> 16))


def test_mx_block_quantize_bit_exact(elmo, orc):
    g = np.random.default_rng(2)
    nb = 3000
    t = (g.normal(0, 0.02, (nb, 32)) * (2.0 ** g.integers(-30, 30, (nb, 1)))).astype(np.float32)
    t[0] = 0.0; t[1, ::2] = -0.0; t[1, 1::2] = 0.0
    t[2] = 1e-42; t[3, 5] = np.nan; t[4, 7] = np.inf; t[5] = 3.0e38; t[6, :] = 6.0; t[7, 0] = 7.99
    r = g.integers(0, 65536, (nb, 32), dtype=np.uint32)
    got = elmo.numerics_probe(11, _dev(t.ravel()), _dev(r.ravel()), n=nb).cpu().numpy().reshape(nb, 33)
    for i in range(nb):
        codes, sc = orc.mx_quantize_block(t[i], r[i])
        assert got[i, 32] == sc, (i, got[i, 32], sc)
        if sc != 255:
            assert np.array_equal(got[i, :32], codes), i


def test_fp4_decode_bit_exact(elmo, orc):
    g = np.random.default_rng(3)
    words = np.arange(0, 2 ** 32, 2 ** 32 // 4096, dtype=np.uint64).astype(np.uint32)
    words = np.concatenate([words, g.integers(0, 2 ** 32, 4096, dtype=np.uint64).astype(np.uint32)])
    scales = np.tile(np.array([127, 120, 100, 135, 1, 126, 119, 121], np.uint32), words.size // 8)
    got = elmo.numerics_probe(12, _dev(words), _dev(scales)).cpu().numpy().view(np.uint32).reshape(-1, 4)
    bf = np.stack([got & 0xFFFF, got >> 16], axis=-1).reshape(words.size, 8).astype(np.uint16)
    gv = torch.from_numpy(bf.view(np.int16)).view(torch.bfloat16).double().numpy()
    nib = np.stack([(words >> (4 * e)) & 15 for e in range(8)], axis=1).astype(np.uint8)
    ref = orc.e2m1_value(nib) * orc.e8m0_value(scales.astype(np.uint8))[:, None]
    assert np.array_equal(gv, ref)


def test_scaled_fp4_mfma_layout(elmo, orc):
    """A = E4M3 codes with few significant bits and B = E2M1 codes, block scales 2^-3 .. 2^3: every
    product and partial sum is exact in FP32, so C must equal the binary64 product exactly."""
    g = np.random.default_rng(4)
    a_vals = np.array([0.0, 0.5, 1.0, 1.5, 2.0, -0.5, -1.0, -2.0, 3.0, -3.0])
    A = orc.e4m3_rne_sat(g.choice(a_vals, (32, 64)))
    Bc = g.integers(0, 16, (32, 64)).astype(np.uint8)
    Bp = (Bc[:, 0::2] | (Bc[:, 1::2] << 4)).astype(np.uint8)
    sA = g.integers(124, 131, (32, 2)).astype(np.uint8)
    sB = g.integers(124, 131, (32, 2)).astype(np.uint8)
    blob = np.concatenate([A.ravel(), Bp.ravel(), sA.ravel(), sB.ravel()]).astype(np.uint8)
    C = elmo.numerics_probe(13, _dev(blob), n=1).cpu().numpy().reshape(32, 32)
    av = orc.e4m3_value(A) * np.repeat(orc.e8m0_value(sA), 32, axis=1)
    bv = orc.e2m1_value(Bc) * np.repeat(orc.e8m0_value(sB), 32, axis=1)
    assert np.array_equal(C.astype(np.float64), av @ bv.T)
