"""Pins for the general-cache decode oracle (``oracle/cache.py``), CPU only.

Each pin checks ``decode_cache`` or one of its steps against something other
than itself: PyTorch's own float8_e4m3fn conversion and textbook E4M3 values
(fp8 decoding), a contiguous cache scattered into pages by the test (page
gather), slices of the cache fed to the already pinned ``oracle.gqa.decode``
(ragged lengths and the window), closed forms (a window of one key), scale
invariants, and the pure-Python brute force. The mutation tests plant
plausible mistakes in each step and check that some pin fails.
"""
import math

import numpy as np
import pytest
import torch

import gqa_inputs as gi
from oracle import brute
from oracle import cache as oc
from oracle import gqa as oa

TOL = 1e-12


def _close(a, b, tol=TOL):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if a.shape != b.shape:
        return False
    same_inf = np.array_equal(np.isneginf(a), np.isneginf(b))
    fa, fb = np.where(np.isfinite(a), a, 0.0), np.where(np.isfinite(b), b, 0.0)
    return same_inf and bool(np.all(np.abs(fa - fb) <= tol * (1 + np.abs(fb))))


def _run(w, **over):
    kw = dict(seqlens=w.seqlens, block_table=w.block_table, window_left=w.window_left,
              fp8=w.fp8, k_scale=w.k_scale, v_scale=w.v_scale)
    kw.update(over)
    return oc.decode_cache(w.q, w.k_cache, w.v_cache, w.scale, **kw)


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------

def pin_fp8_matches_torch():
    """All 256 codes decode as PyTorch's float8_e4m3fn -> float64 does."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oc.fp8_e4m3_decode(np.arange(256))
    nan_ok = np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    return nan_ok and np.array_equal(ref[fin], got[fin])


def pin_fp8_textbook():
    """Landmark E4M3 codes: 1.0, -1.0, the largest normal 448, the smallest
    normal 2^-6, the smallest subnormal 2^-9, -0 and the two NaN codes."""
    got = oc.fp8_e4m3_decode(np.array([0x38, 0xB8, 0x7E, 0x08, 0x01, 0x80, 0x7F, 0xFF]))
    want = [1.0, -1.0, 448.0, 2.0 ** -6, 2.0 ** -9, -0.0]
    return (list(got[:6]) == want and math.copysign(1, got[5]) < 0
            and np.isnan(got[6]) and np.isnan(got[7]))


def pin_contiguous_full_is_decode():
    """Contiguous cache, all lengths equal, no window: the plain decode."""
    w = gi.cache_decode([24] * 3, 8, 2, 64, seed=11, with_seqlens=False)
    o, l = _run(w)
    o2, l2 = oa.decode(w.q, w.k_cache, w.v_cache, w.scale)
    return _close(o, o2) and _close(l, l2)


def pin_ragged_is_slice():
    """Length L_b: the plain decode of that sequence's first L_b keys; an
    empty cache gives O = 0, LSE = -inf."""
    lens = [0, 1, 9, 33]
    w = gi.cache_decode(lens, 8, 2, 64, seed=12)
    o, l = _run(w)
    for b, L in enumerate(lens):
        o2, l2 = oa.decode(w.q[b:b + 1], w.k_cache[b:b + 1, :L], w.v_cache[b:b + 1, :L], w.scale)
        if not (_close(o[b], o2[0]) and _close(l[b], l2[0])):
            return False
    return bool(np.all(o[0] == 0) and np.all(np.isneginf(l[0])))


def _paged_matches_contiguous(lens, bs):
    """The test scatters a contiguous cache into shuffled pages of ``bs``
    keys; the paged decode must give the contiguous result exactly."""
    w = gi.cache_decode(lens, 8, 2, 64, seed=13)
    S = w.k_cache.shape[1]
    nblk = -(-S // bs)
    rng = np.random.default_rng(bs)
    perm = rng.permutation(len(lens) * nblk)
    pages_k = torch.zeros(len(perm), bs, 2, 64, dtype=w.k_cache.dtype)
    pages_v = torch.zeros_like(pages_k)
    table = torch.zeros(len(lens), nblk, dtype=torch.int32)
    for b in range(len(lens)):
        for blk in range(nblk):
            page = int(perm[b * nblk + blk])
            table[b, blk] = page
            n = min(bs, S - blk * bs)
            pages_k[page, :n] = w.k_cache[b, blk * bs:blk * bs + n]
            pages_v[page, :n] = w.v_cache[b, blk * bs:blk * bs + n]
    o, l = _run(w)
    o2, l2 = oc.decode_cache(w.q, pages_k, pages_v, w.scale, seqlens=w.seqlens,
                             block_table=table)
    return _close(o, o2, 0.0) and _close(l, l2, 0.0)


def pin_paged_is_contiguous():
    """Pages of 4 keys, 4 pages per sequence (so a page/slot mix-up still
    indexes in range and shows up as a wrong value)."""
    return _paged_matches_contiguous([3, 16, 12, 0], 4)


def pin_paged_one_page_each():
    """One shuffled 16-key page per sequence (a gather that ignores the table
    still indexes in range and reads the wrong sequence's page)."""
    return _paged_matches_contiguous([3, 16, 9, 1], 16)


def pin_window_is_slice():
    """Window W: the plain decode of the last W + 1 keys; W >= L - 1 is no
    window at all."""
    lens = [1, 5, 30, 30]
    w = gi.cache_decode(lens, 8, 2, 64, seed=14, block_size=8)
    for W in (1, 4, 29):
        o, l = _run(w, window_left=W)
        o_full, l_full = _run(w, window_left=-1)
        kc, vc = _contiguous(w)
        for b, L in enumerate(lens):
            lo = max(0, L - 1 - W)
            o2, l2 = oa.decode(w.q[b:b + 1], kc[b:b + 1, lo:L], vc[b:b + 1, lo:L], w.scale)
            if not (_close(o[b], o2[0]) and _close(l[b], l2[0])):
                return False
            if W >= L - 1 and not (_close(o[b], o_full[b]) and _close(l[b], l_full[b])):
                return False
    return True


def pin_window_zero_closed_form():
    """W = 0 leaves one key, the newest: O = v[L-1] of each head's KV head and
    LSE = scale * q . k[L-1]."""
    lens = [6, 1, 13]
    w = gi.cache_decode(lens, 8, 2, 64, seed=15)
    o, l = _run(w, window_left=0)
    q = w.q.double()
    for b, L in enumerate(lens):
        for h in range(8):
            g = h // 4
            kv = w.k_cache[b, L - 1, g].double()
            vv = w.v_cache[b, L - 1, g].double().numpy()
            if not np.allclose(o[b, h], vv, rtol=0, atol=1e-15):
                return False
            if abs(l[b, h] - w.scale * float(q[b, h] @ kv)) > 1e-12:
                return False
    return True


def pin_scale_invariants():
    """fp8: k_scale c equals k_scale 1 with the softmax scale times c;
    v_scale c multiplies O by c and leaves LSE alone."""
    w = gi.cache_decode([7, 20], 8, 2, 64, seed=16, fp8=True, block_size=8)
    o1, l1 = _run(w, k_scale=1.0, v_scale=1.0)
    o2, l2 = _run(w, k_scale=0.375, v_scale=1.0)
    o3, l3 = oc.decode_cache(w.q, w.k_cache, w.v_cache, w.scale * 0.375, seqlens=w.seqlens,
                             block_table=w.block_table, fp8=True)
    o4, l4 = _run(w, k_scale=1.0, v_scale=2.5)
    return (_close(o2, o3) and _close(l2, l3) and _close(o4, 2.5 * o1) and _close(l4, l1)
            and not _close(o1, o2))


def pin_brute_fp8_paged_window():
    """Pure-Python brute force on values decoded by PyTorch, walking the
    block table by hand."""
    lens = [5, 11, 0]
    w = gi.cache_decode(lens, 4, 2, 8, seed=17, block_size=4, fp8=True, k_scale=0.5,
                        v_scale=1.5, window_left=6)
    kd = (w.k_cache.to(torch.float64) * w.k_scale).tolist()
    vd = (w.v_cache.to(torch.float64) * w.v_scale).tolist()
    o, l = _run(w)
    q = w.q.double().tolist()
    for b, L in enumerate(lens):
        keys = [(int(w.block_table[b, j // 4]), j % 4) for j in range(max(0, L - 7), L)]
        ks = [[kd[p][s][g] for g in range(2)] for p, s in keys]
        vs = [[vd[p][s][g] for g in range(2)] for p, s in keys]
        ob, lb = brute.sequence([q[b]], ks, vs, w.scale, False)
        for h in range(4):
            if not keys:
                if not (np.all(o[b, h] == 0) and np.isneginf(l[b, h])):
                    return False
                continue
            if not (_close(o[b, h], ob[0][h], 1e-12) and abs(l[b, h] - lb[h][0]) < 1e-12):
                return False
    return True


def _contiguous(w):
    """Per-sequence contiguous copy of a paged cache (test-side gather)."""
    if w.block_table is None:
        return w.k_cache, w.v_cache
    B, nblk = w.block_table.shape
    bs = w.block_size
    k = w.k_cache[w.block_table.long()].reshape(B, nblk * bs, *w.k_cache.shape[2:])
    v = w.v_cache[w.block_table.long()].reshape(B, nblk * bs, *w.v_cache.shape[2:])
    return k, v


PINS = [pin_fp8_matches_torch, pin_fp8_textbook, pin_contiguous_full_is_decode,
        pin_ragged_is_slice, pin_paged_is_contiguous, pin_paged_one_page_each,
        pin_window_is_slice,
        pin_window_zero_closed_form, pin_scale_invariants, pin_brute_fp8_paged_window]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin_holds(pin):
    assert pin()


# ---------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail.
# ---------------------------------------------------------------------------

_good_decode = oc.fp8_e4m3_decode
_good_slots = oc.key_slots
_good_stored = oc.stored_values


def _fp8_variant(bias=7, subnormal=True, mdiv=8.0):
    def f(codes):
        c = np.asarray(codes, dtype=np.int64) & 0xFF
        sign = np.where(c >> 7, -1.0, 1.0)
        e = (c >> 3) & 0xF
        m = (c & 0x7).astype(np.float64)
        normal = (1.0 + m / mdiv) * np.exp2(e - float(bias))
        sub = (m / mdiv) * 2.0 ** (1 - bias)
        val = sign * (np.where(e == 0, sub, normal) if subnormal else normal)
        return np.where((e == 15) & (m == 7), np.nan, val)
    return f


MUTATIONS = {
    "fp8_bias_8": ("fp8_e4m3_decode", _fp8_variant(bias=8)),
    "fp8_no_subnormals": ("fp8_e4m3_decode", _fp8_variant(subnormal=False)),
    "fp8_mantissa_16": ("fp8_e4m3_decode", _fp8_variant(mdiv=16.0)),
    "page_slot_swapped": ("key_slots", lambda b, n, t, bs: (
        _good_slots(b, n, t, bs) if t is None else
        (np.asarray(t)[b, np.arange(n) % bs], np.arange(n) // bs))),
    "table_ignored": ("key_slots", lambda b, n, t, bs: (np.full(n, b), np.arange(n))),
    "window_one_short": ("visible_range", lambda L, W: (0, L) if W < 0 else (max(0, L - W), L)),
    "window_ignored": ("visible_range", lambda L, W: (0, L)),
    "window_from_front": ("visible_range", lambda L, W: (0, L) if W < 0 else (0, min(L, W + 1))),
    "scale_dropped": ("stored_values", lambda c, fp8, s: _good_stored(c, fp8, 1.0)),
    "scale_squared": ("stored_values", lambda c, fp8, s: _good_stored(c, fp8, s * s)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oc, attr, fn)
    failed = []
    for p in PINS:
        try:
            ok = p()
        except (IndexError, ValueError):  # a wrong gather may index out of range
            ok = False
        if not ok:
            failed.append(p.__name__)
    assert failed, f"mutation {name} slipped past every pin"
