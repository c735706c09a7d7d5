"""The allocation-free step (elmo_xmc_step_noalloc: the library's static scratch instead of a
caller-supplied workspace) against the workspace step on the same inputs: identical weights, dX and
loss, on two calls in a row where the second is smaller (the scratch keeps the first call's
contents), and a clear error for a step larger than the scratch."""
import numpy as np
import pytest
import torch

import workloads as wk
from tests._helpers import batch_to_dev, from_dev_codes, to_dev_codes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def elmo():
    import precision_label_chunk_amd as m
    m.lib()
    return m


def _both(elmo, B, D, L, chunk, wfmt, seed):
    base = "mxfp4_3m" if wfmt == wk.W_MXFP4 else "bf16_131k"
    wl = wk.scaled(wk.WORKLOADS[base], B=B, D=D, L=L, wfmt=wfmt, lam=5.0, seed=seed)
    W0, bt = wk.make_weights(wl), wk.make_batch(wl)
    X, rp, ids = batch_to_dev(bt)
    print(f"  noalloc vs workspace step: B={B} D={D} L={L} chunk={chunk} wfmt={wfmt}", flush=True)
    Wa = to_dev_codes(W0)
    dXa, la = elmo.step(Wa, X, rp, ids, 0.05, 9, 4, chunk, want_loss=True, wfmt=wfmt)
    Wb = to_dev_codes(W0)
    dXb = torch.empty((B, D), dtype=torch.float32, device="cuda")
    lb = torch.empty((1,), dtype=torch.float32, device="cuda")
    elmo.step_noalloc(Wb, X, rp, ids, 0.05, 9, 4, chunk, dXb, lb, wfmt=wfmt)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_codes(Wa), from_dev_codes(Wb))
    assert np.array_equal(dXa.cpu().numpy(), dXb.cpu().numpy())
    assert la.item() == lb.item()
    assert not np.array_equal(from_dev_codes(Wb), W0)


@pytest.mark.parametrize("wfmt", [wk.W_E4M3, wk.W_BF16, wk.W_MXFP4])
def test_noalloc_step_equals_workspace_step_twice(elmo, wfmt):
    _both(elmo, 256, 768, 20000, 8192, wfmt, seed=1)       # the larger call first
    # then a smaller one over the same scratch (MXFP4 rows need D % 256 == 0)
    _both(elmo, 37, 256 if wfmt == wk.W_MXFP4 else 128, 3000, 1024, wfmt, seed=2)


def test_noalloc_rejects_steps_beyond_the_scratch(elmo):
    W = torch.zeros((2_000_000, 1024), dtype=torch.uint8, device="cuda")
    X = torch.zeros((256, 1024), dtype=torch.int16, device="cuda")
    rp = torch.zeros((257,), dtype=torch.int32, device="cuda")
    ids = torch.zeros((0,), dtype=torch.int32, device="cuda")
    dX = torch.empty((256, 1024), dtype=torch.float32, device="cuda")
    with pytest.raises(elmo.ElmoError) as e:
        elmo.step_noalloc(W, X, rp, ids, 0.05, 0, 0, 1_000_000, dX)
    assert e.value.status == -7
