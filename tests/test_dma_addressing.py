"""CPU check of the forward's direct global->LDS tile addressing (no GPU).

The forward stages K/V tiles with global_load_lds_dwordx4: lane l of wave w
fills LDS bytes [16 (64 w + l), +16) of a tile slot and fetches from global
memory the 16-byte chunk that belongs there (fwd_bf16.hip, dma_kv and
dma_kv8). This module restates that index arithmetic in NumPy and checks,
for every tile step a row tile issues (including the re-loads past its last
needed tile) and for key counts that end anywhere inside a tile, that

* every global read lies inside the sequence's needed keys (row < kend) and
  inside one row (chunk offset + 16 <= row bytes);
* every LDS write lies inside its ring slot (the K half or V half for fp8);
* on a tile with all rows needed, the writes fill the slot exactly once and
  chunk c of row r sits in slot c ^ swz(r), the layout the operand reads
  assume.

These are the helpers the shipped persistent variable-length forward shares
with the withdrawn stream forward; the constants below are the kernel's.
"""
import numpy as np
import pytest

BN = 32


def swz_k(D, r):
    return (r & 15) if D == 128 else ((r >> 1) & 7)


def swz_v(D, r):
    return 4 * (r & 3) if D == 128 else 4 * ((r >> 1) & 1)


def swz8(D, r):
    return ((r >> 1) & 7) if D == 128 else ((r >> 2) & 3)


def nwaves(D):
    return 8 if D == 128 else 4


def dma_kv(D, kend, t, is_v):
    """Per (wave, lane): (global key row, byte offset in the row, LDS byte offset in the slot)."""
    NW, C8 = nwaves(D), D // 8
    ndma = BN * D * 2 // 1024 // NW
    assert ndma == 1
    ntiles = -(-kend // BN)
    tt = min(t, ntiles - 1)
    last = kend - 1 - tt * BN
    w = np.arange(NW)[:, None]
    lane = np.arange(64)[None, :]
    idx = 64 * w + lane
    r = idx // C8
    sw = swz_v(D, r) if is_v else swz_k(D, r)
    ch = ((idx % C8) ^ sw) * 16
    row = tt * BN + np.minimum(r, last)
    lds = 1024 * w + 16 * lane
    return row, ch, lds, r


def dma_kv8(D, kend, t):
    """fp8: waves < NW/2 fetch K, the others V, one load each per tile."""
    NW, C16 = nwaves(D), D // 16
    ntiles = -(-kend // BN)
    tt = min(t, ntiles - 1)
    last = kend - 1 - tt * BN
    w = np.arange(NW)[:, None]
    lane = np.arange(64)[None, :]
    is_v = w >= NW // 2
    wk = np.where(is_v, w - NW // 2, w)
    r = (64 * wk + lane) // C16
    c = (64 * wk + lane) % C16
    ch = np.where(is_v, c, c ^ swz8(D, r)) * 16
    row = tt * BN + np.minimum(r, last)
    lds = np.where(is_v, BN * D, 0) + 1024 * wk + 16 * lane
    return row, ch, lds, r, is_v


KENDS = [1, 2, 31, 32, 33, 63, 64, 65, 100, 128, 129, 4095, 4096]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("is_v", [False, True])
def test_bf16_tile_dma_stays_in_bounds(D, is_v):
    row_bytes = 2 * D
    for kend in KENDS:
        ntiles = -(-kend // BN)
        for t in range(ntiles + 5):  # steps past the end re-load the last tile
            row, ch, lds, r = dma_kv(D, kend, t, is_v)
            assert row.min() >= 0 and row.max() <= kend - 1, (D, kend, t)
            assert ch.min() >= 0 and ch.max() + 16 <= row_bytes
            assert (ch % 16 == 0).all()
            assert lds.min() >= 0 and lds.max() + 16 <= BN * D * 2
            full = (t < ntiles) and (kend - t * BN >= BN)
            if full:
                # every slot written once; chunk c of row r at slot c ^ swz(r)
                flat = lds.ravel() // 16
                assert np.array_equal(np.sort(flat), np.arange(BN * D * 2 // 16))
                C8 = D // 8
                sw = swz_v(D, r) if is_v else swz_k(D, r)
                slot_in_row = (lds // 16) % C8
                assert np.array_equal(slot_in_row, (ch // 16) ^ sw)
                assert np.array_equal(lds // 16 // C8, r)


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_tile_dma_stays_in_bounds(D):
    row_bytes = D
    for kend in KENDS:
        ntiles = -(-kend // BN)
        for t in range(ntiles + 5):
            row, ch, lds, r, is_v = dma_kv8(D, kend, t)
            assert row.min() >= 0 and row.max() <= kend - 1
            assert ch.min() >= 0 and ch.max() + 16 <= row_bytes
            # K half [0, BN D), V half [BN D, 2 BN D) of the slot
            assert (lds[~is_v[:, 0]] + 16 <= BN * D).all() and (lds[is_v[:, 0]] >= BN * D).all()
            assert lds.max() + 16 <= 2 * BN * D
            if t < ntiles and kend - t * BN >= BN:
                assert np.array_equal(np.sort(lds.ravel() // 16), np.arange(2 * BN * D // 16))


def test_decode_key_clamp_stays_in_range():
    # decode_bf16.hip: a tile's K and V rows are min(t0 + offset, w_hi - 1)
    # for offsets below 32, with t0 < w_hi
    for w_hi in [1, 2, 31, 32, 33, 200]:
        for t0 in range(0, w_hi):
            keys = np.minimum(t0 + np.arange(32), w_hi - 1)
            assert keys.min() >= 0 and keys.max() <= w_hi - 1
