"""Host replay of the single-pass kernel's launch schedule and address arithmetic (no GPU): for
chunk sizes, ragged tails and grids with more work-groups than tiles, every tile of every chunk is
taken by exactly one work-group, and every global offset and LDS address the kernel forms stays
inside its buffer. The formulas restate those of step_single.hip and the workspace layout
(step_layout) independently, so a change to either that breaks a bound shows here first."""
import pytest

TJ, MB, TJ1 = 32, 32, 128


def w_row_bytes(wf, D):
    return 2 * D if wf == 0 else D if wf == 1 else D // 2 + D // 32


def chunk_of(L, chunk, wf, D):
    Lr = (L + TJ1 - 1) // TJ1 * TJ1
    c = chunk - chunk % TJ1
    c = max(c, TJ1)
    c = min(c, Lr)
    rb = w_row_bytes(wf, D)
    cmax = ((0x7FFFFFFF // rb - TJ1) // TJ1) * TJ1
    return min(c, cmax)


def row_swz(cpr, j):
    j0, j1, j2, j3 = j & 1, (j >> 1) & 1, (j >> 2) & 1, (j >> 3) & 1
    if cpr >= 16:
        return j2 | (j0 << 1) | (j1 << 2) | ((j0 ^ j3) << 3)
    return j2 | (j3 << 1)


def replay(L, D, chunk, wf, cus):
    nfw = D // 256
    rb = w_row_bytes(wf, D)
    Cc = chunk_of(L, chunk, wf, D)
    NR1 = min((Cc + 31) // 32, cus)
    ntiles = (L + TJ1 - 1) // TJ1
    loss_slots = 4 * ntiles + 4
    nchunks = 0
    for c0 in range(0, L, Cc):
        nchunks += 1
        clen = min(L - c0, Cc)
        assert c0 % TJ1 == 0
        nt = (clen + TJ - 1) // TJ
        seen = [0] * nt
        for r in range(NR1):
            t0, t1 = nt * r // NR1, nt * (r + 1) // NR1
            assert 0 <= t0 <= t1 <= nt
            for t in range(t0, t1):
                seen[t] += 1
                # weight rows of the tile (loads and stores through a resource of clen * rb bytes:
                # offsets must fit the 32-bit offset field; those past clen * rb read zero / drop)
                assert (t * TJ + TJ - 1) * rb + rb <= 0x7FFFFFFF
                # bucket tile and its successor in the per-128-label offsets (ntiles + 1 entries)
                tb = c0 // TJ1 + (t >> 2)
                assert tb + 1 <= ntiles
            if t0 < t1:
                assert c0 // TJ + t0 < loss_slots     # the work-group's loss partial
            # the work-group's dX partial slot: r * D * MB floats, within max(NR, NR1) slots
            assert r < NR1
        assert all(s == 1 for s in seen)
    # LDS: two decoded weight tiles, the logits' partials, the G tile, label bits
    lds = 2 * TJ * D * 2 + 8 * 4 * 64 * 16 + TJ * MB * 2 + 4 * TJ * 4 + 8 * 4
    assert lds <= 160 * 1024
    return nchunks, NR1


@pytest.mark.parametrize("L,D,chunk,wf", [(1, 768, 1, 0), (1, 256, 128, 1), (70, 768, 128, 0), (300, 256, 128, 0),
                                          (1000, 512, 1000, 1), (1337, 768, 128, 1), (4096, 768, 1024, 0),
                                          (20000, 768, 20000, 0), (2500, 512, 512, 2), (8_600_000, 768, 262_144, 0),
                                          (3_000_000, 768, 131_072, 1), (3_000_000, 768, 131_072, 2)])
@pytest.mark.parametrize("cus", [256, 80, 1])
def test_schedule_and_offsets_in_bounds(L, D, chunk, wf, cus):
    replay(L, D, chunk, wf, cus)


def test_lds_addresses_of_one_tile_stay_in_their_arrays():
    """Every LDS element offset the kernel forms for a tile (forward reads, dX transposing reads of
    the weight and G tiles, dW reads of G rows, the update's old-weight reads, the staging writes)
    for every lane of every wave lies inside its array, and the swizzled chunks of a row are a
    permutation of the row's chunks."""
    for D in (256, 512, 768):
        nfw, cpr = D // 256, D // 8
        for j in range(TJ):
            assert sorted(c ^ row_swz(cpr, j) for c in range(cpr)) == list(range(cpr))
            assert sorted(c ^ row_swz(4, j) for c in range(4)) == list(range(4))
        for wave in range(8):
            for lane in range(64):
                l32, hi, q, li = lane & 31, lane >> 5, lane >> 4, lane & 15
                swL = row_swz(cpr, l32)
                for k in range(2 * nfw):                          # forward: 8 BF16 at offF
                    kk = 2 * nfw * wave + k
                    off = l32 * D + (((2 * kk + hi) ^ swL) << 3)
                    assert 0 <= off and off + 8 <= TJ * D
                gW = row_swz(4, l32)
                for kk in range(2):                               # dW B: G row l32
                    off = l32 * MB + (((2 * kk + hi) ^ gW) << 3)
                    assert off + 8 <= TJ * MB
                jX = 8 * (q >> 1) + (li >> 2)
                cB = 2 * (q & 1) + ((li & 3) >> 1)
                for row in (jX, jX + 4):
                    for kx in range(2):                           # dX B: G^T, 4 BF16 per read
                        off = (row + 16 * kx) * MB + ((cB ^ row_swz(4, row)) << 3) + 4 * (li & 1)
                        assert off % 4 == 0 and off + 4 <= TJ * MB
                for f in range(nfw):
                    fb = nfw * wave + f
                    cA = 4 * fb + 2 * (q & 1) + ((li & 3) >> 1)
                    for row in (jX, jX + 4):
                        for kx in range(2):                       # dX A: W^T
                            off = (row + 16 * kx) * D + ((cA ^ row_swz(cpr, row)) << 3) + 4 * (li & 1)
                            assert off % 4 == 0 and off + 4 <= TJ * D
                    for u in range(2):                            # update: old weights, 4 BF16
                        for c in (4 * fb + 2 * u, 4 * fb + 2 * u + 1):
                            off = l32 * D + ((c ^ swL) << 3) + 4 * hi
                            assert off + 4 <= TJ * D
                # epilogue G write: samples b0, b0 + 1 of label l32 (waves 0..7)
                b0 = 8 * (wave >> 1) + 4 * hi + 2 * (wave & 1)
                off = l32 * MB + ((((b0 >> 3) ^ gW) << 3) | (b0 & 7))
                assert off % 2 == 0 and off + 2 <= TJ * MB
