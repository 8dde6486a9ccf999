"""Pins for the fp8-input forward oracle (``oracle/fp8_forward.py``), CPU only.

Each pin checks ``attention_fp8`` against something other than itself: scale
invariants that follow from the definition (q_scale and k_scale trade with the
softmax scale, O is linear in v_scale and LSE does not depend on it), and a
closed form (keys that are all equal make the softmax uniform over the
visible keys, so O is the mean of the visible values, decoded here by
PyTorch's own float8_e4m3fn conversion, and LSE = score + log(count)). The
mutation tests plant plausible mistakes and check that some pin fails.
"""
import math

import numpy as np
import pytest
import torch

import gqa_inputs as gi
from oracle import fp8_forward as of8

TOL = 1e-12


def _close(a, b, tol=TOL):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if a.shape != b.shape:
        return False
    same_inf = np.array_equal(np.isneginf(a), np.isneginf(b))
    fa, fb = np.where(np.isfinite(a), a, 0.0), np.where(np.isfinite(b), b, 0.0)
    return same_inf and bool(np.all(np.abs(fa - fb) <= tol * (1 + np.abs(fb))))


def _w(causal=True):
    return gi.fixed_fp8(2, 6, 2, 19, 23, 16, seed=41, causal=causal)


def pin_q_scale_trades_with_softmax_scale():
    """Doubling q_scale equals doubling the softmax scale."""
    w = _w()
    o1, l1 = of8.attention_fp8(w.q, w.k, w.v, w.scale, True, 2.0, 1.0, 1.0)
    o2, l2 = of8.attention_fp8(w.q, w.k, w.v, 2 * w.scale, True, 1.0, 1.0, 1.0)
    return _close(o1, o2) and _close(l1, l2)


def pin_k_scale_trades_with_softmax_scale():
    """Multiplying k_scale by 4 equals multiplying the softmax scale by 4."""
    w = _w(causal=False)
    o1, l1 = of8.attention_fp8(w.q, w.k, w.v, w.scale, False, 1.0, 4.0, 1.0)
    o2, l2 = of8.attention_fp8(w.q, w.k, w.v, 4 * w.scale, False, 1.0, 1.0, 1.0)
    return _close(o1, o2) and _close(l1, l2)


def pin_v_scale_is_linear():
    """v_scale multiplies O and leaves LSE unchanged."""
    w = _w()
    o1, l1 = of8.attention_fp8(w.q, w.k, w.v, w.scale, True, 1.0, 1.0, 0.5)
    o2, l2 = of8.attention_fp8(w.q, w.k, w.v, w.scale, True, 1.0, 1.0, 1.0)
    return _close(o1, 0.5 * o2) and _close(l1, l2) and not _close(o1, o2)


def pin_uniform_keys_closed_form():
    """Every key code = 0x38 (1.0): all visible keys score the same, so O is
    the mean of the visible values and LSE = score + log(count); causal,
    Lq = 5 < Lk = 9 (bottom-right: row i sees keys 0 .. i + 4)."""
    g = torch.Generator().manual_seed(43)
    q = torch.randn(1, 5, 2, 8, generator=g).to(torch.float8_e4m3fn)
    k = torch.full((1, 9, 1, 8), 0x38, dtype=torch.uint8).view(torch.float8_e4m3fn)
    v = torch.randn(1, 9, 1, 8, generator=g).to(torch.float8_e4m3fn)
    qs, ks, vs, scale = 0.5, 0.25, 2.0, 0.35
    o, lse = of8.attention_fp8(q, k, v, scale, True, qs, ks, vs)
    qf = q.to(torch.float64).numpy()
    vf = v.to(torch.float64).numpy()[0, :, 0, :] * vs
    s32 = float(np.float32(scale))
    ok = True
    for i in range(5):
        n = i + 5
        for h in range(2):
            score = s32 * qs * ks * float(qf[0, i, h].sum())
            ok &= _close(o[0, i, h], vf[:n].mean(axis=0), 1e-12)
            ok &= _close(lse[0, h, i], score + math.log(n), 1e-12)
    return ok


def pin_varlen_is_per_sequence():
    """A variable-length batch equals its sequences run one at a time."""
    w = gi.varlen_fp8([7, 0, 12], [9, 4, 12], 4, 2, 16, seed=44, causal=True,
                      q_scale=0.5, k_scale=2.0, v_scale=0.25)
    cq, ck = w.cu_seqlens_q.tolist(), w.cu_seqlens_k.tolist()
    qs, ks, vs = w.fp8_scales
    o, l = of8.attention_fp8(w.q, w.k, w.v, w.scale, True, qs, ks, vs, cq, ck)
    ok = True
    for b in range(3):
        if cq[b + 1] == cq[b]:
            continue
        ob, lb = of8.attention_fp8(w.q[None, cq[b]:cq[b + 1]], w.k[None, ck[b]:ck[b + 1]],
                                   w.v[None, ck[b]:ck[b + 1]], w.scale, True, qs, ks, vs)
        ok &= _close(o[cq[b]:cq[b + 1]], ob[0]) and _close(l[cq[b]:cq[b + 1]], lb[0].T)
    return ok


PINS = [pin_q_scale_trades_with_softmax_scale, pin_k_scale_trades_with_softmax_scale,
        pin_v_scale_is_linear, pin_uniform_keys_closed_form, pin_varlen_is_per_sequence]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin_holds(pin):
    assert pin()


def test_rows_agree_with_full():
    """attention_rows_fp8 equals attention_fp8 at the chosen rows."""
    w = gi.fixed_fp8(2, 4, 2, 11, 13, 16, seed=45, causal=True, q_scale=0.5, k_scale=0.5,
                     v_scale=2.0)
    qs, ks, vs = w.fp8_scales
    o, l = of8.attention_fp8(w.q, w.k, w.v, w.scale, True, qs, ks, vs)
    rows = [(0, 0, 0), (1, 10, 3), (0, 5, 2)]
    ro, rl = of8.attention_rows_fp8(w.q, w.k, w.v, w.scale, True, qs, ks, vs, rows)
    for t, (b, i, h) in enumerate(rows):
        assert _close(ro[t], o[b, i, h]) and _close(rl[t], l[b, h, i])


# ---------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail.
# ---------------------------------------------------------------------------

_good = of8.dequantised

MUTATIONS = {
    "q_scale_dropped": lambda q, k, v, qs, ks, vs: _good(q, k, v, 1.0, ks, vs),
    "k_scale_dropped": lambda q, k, v, qs, ks, vs: _good(q, k, v, qs, 1.0, vs),
    "v_scale_dropped": lambda q, k, v, qs, ks, vs: _good(q, k, v, qs, ks, 1.0),
    "k_scale_on_v": lambda q, k, v, qs, ks, vs: _good(q, k, v, qs, vs, ks),
    "scales_squared": lambda q, k, v, qs, ks, vs: _good(q, k, v, qs * qs, ks * ks, vs * vs),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    monkeypatch.setattr(of8, "dequantised", MUTATIONS[name])
    failed = [p.__name__ for p in PINS if not p()]
    assert failed, f"mutation {name} slipped past every pin"
