"""Pins of the oracle's counter-based RNG (Philox4x32-10, Salmon et al., SC'11).

The pages do not state the RNG behind stochastic rounding; the reading is a counter-based generator
keyed on (seed, step, element index). Known answers come from running rocRAND's Philox4x32-10
engine (a library routine shipped with ROCm as a source header), compiled here for the host with
g++; it is executed, not copied.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

HELPER = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
int main() {
  unsigned long long seed, sub, off;
  while (scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    rocrand_device::philox4x32_10_engine e(seed, sub, off);
    uint4 v = e.next4();
    printf("%u %u %u %u\n", v.x, v.y, v.z, v.w);
  }
  return 0;
}
"""

TRIPLES = [(0, 0, 0), (1, 0, 0), (0, 1, 0), (0, 0, 1), (0xFFFFFFFFFFFFFFFF, 3, 5),
           (0xDEADBEEFCAFEF00D, 123456789, 987654321), (2**32 + 7, 2**33 + 1, 2**35 + 11),
           (42, 9, 2**32 - 1), (7, 2**40, 17)]


@pytest.fixture(scope="module")
def rocrand_kat():
    hdr = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    if not (os.path.exists(hdr) and shutil.which("g++")):
        pytest.skip("rocRAND header or g++ not available")
    d = tempfile.mkdtemp()
    src, exe = os.path.join(d, "kat.cpp"), os.path.join(d, "kat")
    open(src, "w").write(HELPER)
    subprocess.run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", src,
                    "-o", exe], check=True, capture_output=True)
    # rocRAND's engine(seed, subsequence, offset): key = seed, counter = (offset / 4, subsequence)
    inp = "".join(f"{s} {step} {4 * g}\n" for (s, step, g) in TRIPLES)
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    shutil.rmtree(d, ignore_errors=True)
    return [np.array(list(map(int, ln.split())), np.uint32) for ln in out.strip().splitlines()]


def _ctr_key(seed, step, g):
    ctr = np.array([g & 0xFFFFFFFF, g >> 32, step & 0xFFFFFFFF, step >> 32], np.uint32)
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32)
    return ctr, key


def test_philox_matches_rocrand(orc, rocrand_kat):
    for (s, step, g), ref in zip(TRIPLES, rocrand_kat):
        ctr, key = _ctr_key(s, step, g)
        assert np.array_equal(orc.philox4x32(ctr, key, 10), ref), (s, step, g)


def test_philox_zero_block_known_value(orc, rocrand_kat):
    # counter 0, key 0: the first word rocRAND returns is 0x6627e8d5
    assert rocrand_kat[0][0] == 0x6627E8D5
    assert orc.philox4x32(np.zeros(4, np.uint32), np.zeros(2, np.uint32), 10)[0] == 0x6627E8D5


def _block_elements(g):
    # the 8 element indices of block g, in position order p = 0..7: 8g .. 8g + 7
    return [8 * g + p for p in range(8)]


def test_r16_slices_the_block(orc, rocrand_kat):
    # element at position p of block g uses 16-bit half (p & 1) of word p >> 1 of that block
    for (s, step, g), ref in zip(TRIPLES, rocrand_kat):
        halves = [(int(ref[p // 2]) >> (16 * (p % 2))) & 0xFFFF for p in range(8)]
        for p, idx in enumerate(_block_elements(g)):
            assert int(orc.r16(s, step, idx, 1)[0]) == halves[p], (s, step, g, p)


def test_r16_array_crosses_blocks(orc, rocrand_kat):
    # 10 consecutive draws from index 8g - 1: the last position of block g - 1, all of block g (the
    # rocRAND words), the first position of block g + 1 (from the oracle's generator, pinned above)
    for (s, step, g), ref in zip(TRIPLES, rocrand_kat):
        if g == 0 or g + 1 >= 2**64:
            continue
        r = [int(v) for v in orc.r16(s, step, 8 * g - 1, 10)]
        prev = orc.philox4x32(*_ctr_key(s, step, g - 1), 10)
        nxt = orc.philox4x32(*_ctr_key(s, step, g + 1), 10)
        assert r[0] == int(prev[3]) >> 16
        assert r[1:9] == [(int(ref[p // 2]) >> (16 * (p % 2))) & 0xFFFF for p in range(8)]
        assert r[9] == int(nxt[0]) & 0xFFFF


def test_r16_blocks_partition_the_indices():
    # every index belongs to exactly one block, at one position
    seen = sorted(i for g in range(20, 24) for i in _block_elements(g))
    assert seen == list(range(160, 192))


def test_r16_statistics(orc):
    n = 1 << 20
    r = orc.r16(seed=0, step=0, idx0=0, n=n).astype(np.int64)
    # chi-square on 256 bins of the top 8 bits
    h = np.bincount(r >> 8, minlength=256)
    chi2 = ((h - n / 256) ** 2 / (n / 256)).sum()
    assert chi2 < 256 + 6 * np.sqrt(2 * 256)
    # every bit balanced
    for b in range(16):
        frac = ((r >> b) & 1).mean()
        assert abs(frac - 0.5) < 5 * 0.5 / np.sqrt(n)
    # streams at another step / seed are uncorrelated with this one
    for (seed, step) in [(0, 1), (1, 0)]:
        r2 = orc.r16(seed=seed, step=step, idx0=0, n=n).astype(np.float64)
        c = np.corrcoef(r.astype(np.float64), r2)[0, 1]
        assert abs(c) < 5 / np.sqrt(n)
    # adjacent indices uncorrelated
    c = np.corrcoef(r[:-1].astype(np.float64), r[1:].astype(np.float64))[0, 1]
    assert abs(c) < 5 / np.sqrt(n)
