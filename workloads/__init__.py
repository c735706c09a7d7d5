"""Seeded synthetic inputs for the XMC classifier-head step and top-k pass.

This module only draws inputs; it holds none of the method's arithmetic. Both the HIP path's tests
and the CPU oracle consume what it produces. The initial quantisation of synthetic weights and
features to BF16 / FP8-E4M3 uses PyTorch's own casts (a library routine), not either codec under
test.

Workloads stand in for the label spaces the ELMO pages train on (LF-AmazonTitles-131K,
(Amazon|AmazonTitles)-670K, Amazon-3M and LF-Paper2Keywords-8.6M, named in the summary page's
"Experimental setup" and "Key results"); no dataset item is reproduced, only sizes and shapes:
  * X: N(0, 1) rows normalised to unit L2 norm (tiny case: N(0, 1)/sqrt(D)), cast to BF16;
  * W: N(0, 0.02^2), cast to BF16 or E4M3; MX-scaled FP4 weights are drawn in code space: E8M0
    scales 2^-8 .. 2^-6 and E2M1 elements whose magnitudes follow |N(0, 0.02^2)| / 2^-7 binned to the
    nearest E2M1 magnitude (signs uniform), which gives values of the same size;
  * labels: per sample 1 + Poisson(lam) positives with ids drawn from a finite Zipf(s) law over
    ranks 1..L (id = rank - 1), without replacement within a sample (tiny case: 1..8 positives,
    uniform ids without replacement).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

W_BF16 = 0
W_E4M3 = 1
W_MXFP4 = 2


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    D: int
    L: int
    chunk: int
    wfmt: int
    lr: float
    steps: int
    x_kind: str                  # "rownorm" or "gauss_sqrtD"
    label_kind: str              # "zipf" or "uniform"
    lam: float = 0.0             # Poisson mean of extra positives (zipf)
    zipf_s: float = 1.0
    max_pos: int = 8             # uniform: 1..max_pos positives
    topk: int = 0
    n_eval: int = 0
    seed: int = 0
    tag: int = 0                 # stream separator between workloads

    @property
    def wdtype(self):
        return np.uint16 if self.wfmt == W_BF16 else np.uint8

    @property
    def wbytes(self):
        """storage bytes per weight (MXFP4: half a byte plus a scale byte per 32)"""
        return 2 if self.wfmt == W_BF16 else (17 / 32 if self.wfmt == W_MXFP4 else 1)


WORKLOADS = {
    "tiny": Workload("xmc-bf16-L4096-D64-B32", 32, 64, 4096, 1024, W_BF16, 0.05, 1,
                     "gauss_sqrtD", "uniform", max_pos=8, tag=0),
    "bf16_131k": Workload("xmc-bf16-L131072-D768-B256", 256, 768, 131072, 32768, W_BF16, 0.05, 10,
                          "rownorm", "zipf", lam=4.0, zipf_s=1.1, tag=1),
    "bf16_670k": Workload("xmc-bf16-L670000-D768-B256", 256, 768, 670000, 65536, W_BF16, 0.05, 10,
                          "rownorm", "zipf", lam=5.0, zipf_s=1.0, tag=2),
    "e4m3_3m": Workload("xmc-e4m3-L3000000-D768-B256", 256, 768, 3000000, 131072, W_E4M3, 0.1, 10,
                        "rownorm", "zipf", lam=35.0, zipf_s=1.0, tag=3),
    "bf16_8p6m": Workload("xmc-bf16-L8600000-D768-B128", 128, 768, 8600000, 262144, W_BF16, 0.05, 5,
                          "rownorm", "zipf", lam=9.0, zipf_s=1.2, topk=5, n_eval=4096, tag=4),
    # the FP4 weights the pages leave open (with micro-tensor scaling), at the 3M-label head's shape
    "mxfp4_3m": Workload("xmc-mxfp4-L3000000-D768-B256", 256, 768, 3000000, 131072, W_MXFP4, 0.1, 10,
                         "rownorm", "zipf", lam=35.0, zipf_s=1.0, tag=5),
    "mxfp4_131k": Workload("xmc-mxfp4-L131072-D768-B256", 256, 768, 131072, 32768, W_MXFP4, 0.1, 10,
                           "rownorm", "zipf", lam=35.0, zipf_s=1.0, tag=6),
    # the 8.6M- and 3M-label heads at a batch of 32 samples, where the single-pass step applies
    "bf16_8p6m_b32": Workload("xmc-bf16-L8600000-D768-B32", 32, 768, 8600000, 262144, W_BF16, 0.05, 5,
                              "rownorm", "zipf", lam=9.0, zipf_s=1.2, tag=7),
    "e4m3_3m_b32": Workload("xmc-e4m3-L3000000-D768-B32", 32, 768, 3000000, 131072, W_E4M3, 0.1, 10,
                            "rownorm", "zipf", lam=35.0, zipf_s=1.0, tag=8),
    # one GPU's share of each head when its labels are split into eight contiguous ranges (the same
    # batch; positives drawn by the same recipe over the shard's own labels)
    "e4m3_375k": Workload("xmc-e4m3-L375000-D768-B256", 256, 768, 375000, 131072, W_E4M3, 0.1, 10,
                          "rownorm", "zipf", lam=35.0, zipf_s=1.0, tag=9),
    "bf16_1075k": Workload("xmc-bf16-L1075000-D768-B128", 128, 768, 1075000, 262144, W_BF16, 0.05, 5,
                           "rownorm", "zipf", lam=9.0, zipf_s=1.2, tag=10),
}


def mx_row_bytes(D: int) -> int:
    return D // 2 + D // 32


def _mx_magnitude_probs() -> np.ndarray:
    """P(nearest E2M1 magnitude) of |N(0, (0.02 / 2^-7)^2)| (bin edges halfway between magnitudes)."""
    import math
    sd = 0.02 / 2.0 ** -7
    edges = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    cdf = [math.erf(e / (sd * math.sqrt(2.0))) for e in edges] + [1.0]
    p = np.diff(np.array([0.0] + cdf))
    return p / p.sum()


def make_w_mx(L: int, D: int, g: np.random.Generator) -> np.ndarray:
    """MX-scaled FP4 rows [L][D/2 + D/32] drawn in code space (see the module docstring)."""
    mag = g.choice(8, size=(L, D), p=_mx_magnitude_probs()).astype(np.uint8)
    codes = mag | (g.integers(0, 2, (L, D), dtype=np.uint8) << 3)
    out = np.empty((L, mx_row_bytes(D)), np.uint8)
    out[:, :D // 2] = codes[:, 0::2] | (codes[:, 1::2] << 4)
    out[:, D // 2:] = g.integers(119, 122, (L, D // 32), dtype=np.uint8)
    return out

_PURPOSE = {"x": 0, "w": 1, "labels": 2, "eval_x": 3}


def rng(wl: Workload, purpose: str, step: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([wl.seed, wl.tag, _PURPOSE[purpose], step]))


def to_bf16_codes(x: np.ndarray) -> np.ndarray:
    """float array -> BF16 codes (uint16) via torch's round-to-nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float array (|x| < 448) -> OCP E4M3 codes (uint8) via torch's float8_e4m3fn cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def make_x(B: int, D: int, kind: str, g: np.random.Generator) -> np.ndarray:
    x = g.standard_normal((B, D))
    if kind == "rownorm":
        x /= np.linalg.norm(x, axis=1, keepdims=True)
    elif kind == "gauss_sqrtD":
        x /= np.sqrt(D)
    else:
        raise ValueError(kind)
    return to_bf16_codes(x)


def make_w(L: int, D: int, wfmt: int, g: np.random.Generator, block: int = 1 << 16) -> np.ndarray:
    if wfmt == W_MXFP4:
        return make_w_mx(L, D, g)
    out = np.empty((L, D), np.uint16 if wfmt == W_BF16 else np.uint8)
    for r0 in range(0, L, block):
        r1 = min(L, r0 + block)
        w = (g.standard_normal((r1 - r0, D)) * 0.02).astype(np.float32)
        out[r0:r1] = to_bf16_codes(w) if wfmt == W_BF16 else to_e4m3_codes(w)
    return out


def make_w_device(L: int, D: int, wfmt: int, seed: int, device, block: int = 1 << 18):
    """Same distribution drawn on a torch device (for sizes where host generation is slow).
    Returns a uint16/uint8 tensor [L, D] of codes."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    if wfmt == W_MXFP4:
        out = torch.empty((L, mx_row_bytes(D)), dtype=torch.uint8, device=device)
        probs = torch.from_numpy(_mx_magnitude_probs()).to(device=device, dtype=torch.float32)
        cum = torch.cumsum(probs, 0)
        cum[-1] = 1.0
        for r0 in range(0, L, block):
            r1 = min(L, r0 + block)
            u = torch.rand((r1 - r0, D), generator=gen, device=device)
            mag = torch.searchsorted(cum, u.contiguous()).clamp_(max=7).to(torch.uint8)
            sign = (torch.rand((r1 - r0, D), generator=gen, device=device) < 0.5).to(torch.uint8) << 3
            codes = mag | sign
            out[r0:r1, :D // 2] = codes[:, 0::2] | (codes[:, 1::2] << 4)
            out[r0:r1, D // 2:] = torch.randint(119, 122, (r1 - r0, D // 32), generator=gen, device=device,
                                                dtype=torch.uint8)
        return out
    dt = torch.int16 if wfmt == W_BF16 else torch.uint8
    out = torch.empty((L, D), dtype=dt, device=device)
    for r0 in range(0, L, block):
        r1 = min(L, r0 + block)
        w = torch.randn((r1 - r0, D), generator=gen, device=device, dtype=torch.float32) * 0.02
        if wfmt == W_BF16:
            out[r0:r1] = w.to(torch.bfloat16).view(torch.int16)
        else:
            out[r0:r1] = w.to(torch.float8_e4m3fn).view(torch.uint8)
    return out


class ZipfSampler:
    """Finite Zipf law over ranks 1..L, p(r) proportional to r^-s, by inverse CDF."""

    def __init__(self, L: int, s: float):
        w = np.arange(1, L + 1, dtype=np.float64) ** (-s)
        self.cdf = np.cumsum(w)
        self.cdf /= self.cdf[-1]
        self.L = L

    def draw(self, g: np.random.Generator, n: int) -> np.ndarray:
        return np.minimum(np.searchsorted(self.cdf, g.random(n), side="right"), self.L - 1)


def make_labels(B: int, L: int, kind: str, g: np.random.Generator, lam: float = 0.0,
                zipf: ZipfSampler | None = None, max_pos: int = 8):
    """CSR labels (row_ptr int32 [B+1], ids int32 [nnz]), distinct ids within a row."""
    rows = []
    for _ in range(B):
        if kind == "uniform":
            n = int(g.integers(1, max_pos + 1))
            rows.append(np.sort(g.choice(L, size=min(n, L), replace=False)))
        elif kind == "zipf":
            n = min(L, 1 + int(g.poisson(lam)))
            chosen: set[int] = set()
            while len(chosen) < n:
                for v in zipf.draw(g, n - len(chosen)):
                    chosen.add(int(v))
            rows.append(np.array(sorted(chosen), dtype=np.int64))
        else:
            raise ValueError(kind)
    row_ptr = np.zeros(B + 1, np.int32)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    ids = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)
    return row_ptr, ids


@dataclass
class Batch:
    X: np.ndarray            # uint16 [B, D] BF16 codes
    row_ptr: np.ndarray      # int32 [B+1]
    ids: np.ndarray          # int32 [nnz]


_ZIPF_CACHE: dict = {}


def zipf_for(wl: Workload) -> ZipfSampler | None:
    if wl.label_kind != "zipf":
        return None
    key = (wl.L, wl.zipf_s)
    if key not in _ZIPF_CACHE:
        _ZIPF_CACHE[key] = ZipfSampler(wl.L, wl.zipf_s)
    return _ZIPF_CACHE[key]


def make_batch(wl: Workload, step: int = 0, B: int | None = None) -> Batch:
    B = wl.B if B is None else B
    X = make_x(B, wl.D, wl.x_kind, rng(wl, "x", step))
    rp, ids = make_labels(B, wl.L, wl.label_kind, rng(wl, "labels", step), lam=wl.lam,
                          zipf=zipf_for(wl), max_pos=wl.max_pos)
    return Batch(X, rp, ids)


def make_eval_x(wl: Workload, n: int | None = None) -> np.ndarray:
    n = wl.n_eval if n is None else n
    return make_x(n, wl.D, wl.x_kind, rng(wl, "eval_x"))


def make_weights(wl: Workload, L: int | None = None) -> np.ndarray:
    return make_w(wl.L if L is None else L, wl.D, wl.wfmt, rng(wl, "w"))


def scaled(wl: Workload, **kw) -> Workload:
    """A copy of a workload with some sizes changed (for parity tests at reduced L or B)."""
    d = dict(wl.__dict__)
    d.update(kw)
    return Workload(**d)
