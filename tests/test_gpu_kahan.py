"""Parity of the Kahan-compensated BF16 update (encoder parameters) with the oracle: BF16 codes of
w and c must be bit-identical after every step (the device evaluates the same binary32 operations
in the same order and rounds the two stores to nearest-even). Ragged sizes exercise the vector
body and the scalar tail, offset views the scalar path, and the encoder-sized case the launch the
benchmark times."""
import numpy as np
import pytest
import torch

import oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def elmo():
    import precision_label_chunk_amd as m
    m.lib()
    return m


def _inputs(n, seed, gscale=1.0):
    g = np.random.default_rng(seed)
    w = orc.bf16_rne(g.normal(0, 0.02, n).astype(np.float32))
    c = np.zeros(n, np.uint16)
    grads = [(g.normal(0, gscale, n) * g.choice([1.0, 1e-3, 1e2], n)).astype(np.float32) for _ in range(4)]
    return w, c, grads


def _dev16(a):
    return torch.from_numpy(a.view(np.int16)).cuda()


@pytest.mark.parametrize("n", [1, 7, 8, 9, 1000, 4099, (1 << 20) + 3])
@pytest.mark.parametrize("lr", [1e-3, 0.37])
def test_kahan_update_matches_oracle(elmo, n, lr):
    w, c, grads = _inputs(n, seed=n % 97)
    wd, cd = _dev16(w.copy()), _dev16(c.copy())
    print(f"  kahan n={n} lr={lr}", flush=True)
    for s, gr in enumerate(grads):
        elmo.kahan_update(wd, cd, torch.from_numpy(gr).cuda(), lr)
        w, c = orc.kahan_update(w, c, gr, lr)
        assert np.array_equal(wd.cpu().numpy().view(np.uint16), w), s
        assert np.array_equal(cd.cpu().numpy().view(np.uint16), c), s
    assert np.any(c != 0)


def test_kahan_update_unaligned_views_and_special_values(elmo):
    n = 5000
    w, c, grads = _inputs(n + 1, seed=3)
    w[:8] = np.array([0x0000, 0x8000, 0x7F7F, 0xFF7F, 0x0001, 0x8001, 0x3F80, 0xBF80], np.uint16)
    c[:8] = np.array([0x0000, 0x8000, 0x0000, 0x0000, 0x8001, 0x0001, 0xBA80, 0x3A80], np.uint16)
    g = grads[0]
    g[:8] = np.array([0.0, -0.0, -1e30, 1e30, 0.0, 0.0, -1.0, 1.0], np.float32)
    wd, cd, gd = _dev16(w.copy()), _dev16(c.copy()), torch.from_numpy(g).cuda()
    elmo.kahan_update(wd[1:], cd[1:], gd[1:], 2.0 ** -10)      # offset by one element: scalar path
    elmo.kahan_update(wd, cd, gd, 2.0 ** -10)                  # then the whole array
    w1, c1 = orc.kahan_update(w[1:], c[1:], g[1:], 2.0 ** -10)
    w2, c2 = orc.kahan_update(np.concatenate([w[:1], w1]), np.concatenate([c[:1], c1]), g, 2.0 ** -10)
    assert np.array_equal(wd.cpu().numpy().view(np.uint16), w2)
    assert np.array_equal(cd.cpu().numpy().view(np.uint16), c2)


def test_kahan_update_empty_is_a_no_op(elmo):
    wd = torch.zeros(0, dtype=torch.int16, device="cuda")
    elmo.kahan_update(wd, wd.clone(), torch.zeros(0, dtype=torch.float32, device="cuda"), 0.1)


def test_kahan_update_encoder_size(elmo):
    """110M parameters (a 768-wide, 12-layer encoder), the size the benchmark times; all compared."""
    n = 110_000_000
    g = np.random.default_rng(21)
    w = orc.bf16_rne(g.normal(0, 0.02, n).astype(np.float32))
    c = orc.bf16_rne(g.normal(0, 1e-5, n).astype(np.float32))
    gr = g.normal(0, 1.0, n).astype(np.float32)
    print(f"  kahan n={n}", flush=True)
    wd, cd = _dev16(w), _dev16(c)
    elmo.kahan_update(wd, cd, torch.from_numpy(gr).cuda(), 1e-3)
    wr, cr = orc.kahan_update(w, c, gr, 1e-3)
    assert np.array_equal(wd.cpu().numpy().view(np.uint16), wr)
    assert np.array_equal(cd.cpu().numpy().view(np.uint16), cr)
