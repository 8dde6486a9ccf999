"""Pins for the fp64 gradient oracle (``oracle/backward.py``), CPU only.

The gradients are checked against things other than their own formulas:
central finite differences of the (separately pinned) forward oracle,
PyTorch's float64 autograd through its own scaled_dot_product_attention with
grouped heads, the GQA = MHA identity with K/V gradients summed over each
group (the FlashAttention-2 page's statement for grouped heads), and
invariants of the softmax (a shift of V changes no gradient; every row of dS
sums to zero, so dK sums to zero over the keys). Planted mistakes in each step
must fail at least one pin.
"""
import numpy as np
import pytest
import torch

import gqa_inputs as gi
from oracle import backward as ob
from oracle import gqa as oa


def _fd_grads(w, do, h=1e-6):
    """Central differences of sum(O * do) w.r.t. every element of q, k, v."""
    q, k, v = (oa.as_f64(x).copy() for x in (w.q, w.k, w.v))
    cq = w.cu_seqlens_q.tolist() if w.varlen else None
    ck = w.cu_seqlens_k.tolist() if w.varlen else None

    def loss(q_, k_, v_):
        o, _ = oa.attention(q_, k_, v_, w.scale, w.causal, cq, ck)
        return float((o * do).sum())

    grads = []
    for idx, x in enumerate((q, k, v)):
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            old = x[mi]
            x[mi] = old + h
            up = loss(q, k, v)
            x[mi] = old - h
            dn = loss(q, k, v)
            x[mi] = old
            g[mi] = (up - dn) / (2 * h)
        grads.append(g)
    return grads


def _do_like(w, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(w.q.shape, generator=g, dtype=torch.float64).numpy()


def _grads(w, do):
    cq = w.cu_seqlens_q.tolist() if w.varlen else None
    ck = w.cu_seqlens_k.tolist() if w.varlen else None
    return ob.attention_grad(w.q, w.k, w.v, do, w.scale, w.causal, cq, ck)


def _close(a, b, tol):
    return bool(np.max(np.abs(np.asarray(a) - np.asarray(b))) <= tol)


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------

def pin_finite_differences_fixed():
    """Causal with Lq < Lk (bottom-right) and Lq > Lk (rows with no key), G = 2."""
    for sq, sk in ((3, 5), (4, 2)):
        w = gi.fixed(1, 4, 2, sq, sk, 4, seed=21 + sq, dtype=torch.float32, causal=True,
                     scale=0.7)
        do = _do_like(w, 1)
        got = _grads(w, do)
        ref = _fd_grads(w, do)
        if not all(_close(a, b, 1e-6) for a, b in zip(got, ref)):
            return False
    return True


def pin_finite_differences_varlen():
    """Two packed sequences (one empty of queries), not causal, G = 3."""
    w = gi.varlen([2, 0, 3], [3, 2, 1], 3, 1, 4, seed=23, dtype=torch.float32, scale=0.5)
    do = _do_like(w, 2)
    got = _grads(w, do)
    ref = _fd_grads(w, do)
    return all(_close(a, b, 1e-6) for a, b in zip(got, ref))


def pin_torch_sdpa_autograd():
    """PyTorch float64 SDPA (enable_gqa) backward, causal and not, Lq = Lk."""
    import torch.nn.functional as F
    for causal in (False, True):
        w = gi.fixed(2, 6, 2, 7, 7, 8, seed=24, dtype=torch.float32, causal=causal, scale=0.3)
        do = _do_like(w, 3)
        got = _grads(w, do)
        t = lambda x: x.to(torch.float64).transpose(1, 2).contiguous().requires_grad_(True)
        q, k, v = t(w.q), t(w.k), t(w.v)
        o = F.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=float(np.float32(w.scale)),
                                           enable_gqa=True)
        o.backward(torch.from_numpy(do).transpose(1, 2))
        ref = [x.grad.transpose(1, 2).numpy() for x in (q, k, v)]
        if not all(_close(a, b, 1e-10) for a, b in zip(got, ref)):
            return False
    return True


def pin_gqa_equals_mha_summed():
    """GQA gradients = MHA gradients on repeat-interleaved K/V, with the K/V
    gradients of each group's copies summed."""
    w = gi.fixed(1, 8, 2, 6, 9, 4, seed=25, dtype=torch.float32, causal=True)
    do = _do_like(w, 4)
    dq, dk, dv = _grads(w, do)
    rep = lambda x: x.repeat_interleave(4, dim=2)
    dq2, dk2, dv2 = ob.attention_grad(w.q, rep(w.k), rep(w.v), do, w.scale, True)
    fold = lambda x: x.reshape(x.shape[0], x.shape[1], 2, 4, x.shape[3]).sum(axis=3)
    return _close(dq, dq2, 1e-12) and _close(dk, fold(dk2), 1e-12) and _close(dv, fold(dv2), 1e-12)


def pin_v_shift_invariance():
    """Adding a constant row to every V row changes no gradient."""
    w = gi.fixed(1, 4, 2, 5, 6, 4, seed=26, dtype=torch.float32, causal=False)
    do = _do_like(w, 5)
    a = _grads(w, do)
    shift = torch.tensor([0.5, -1.0, 2.0, 0.25], dtype=torch.float64)  # exact in fp64
    w2 = gi.Workload("s", w.q, w.k, w.v.double() + shift, w.causal, w.scale)
    b = _grads(w2, do)
    return all(_close(x, y, 1e-12) for x, y in zip(a, b))


def pin_dk_sums_to_zero():
    """Each row of dS sums to zero, so dK summed over the keys vanishes."""
    for causal in (False, True):
        w = gi.fixed(2, 6, 3, 7, 5, 4, seed=27, dtype=torch.float32, causal=causal)
        _, dk, _ = _grads(w, _do_like(w, 6))
        if not _close(dk.sum(axis=1), 0.0, 1e-12):
            return False
        if not np.abs(dk).max() > 1e-3:
            return False
    return True


def pin_zero_output_gradient():
    w = gi.fixed(1, 4, 1, 3, 4, 4, seed=28, dtype=torch.float32, causal=True)
    return all(np.all(x == 0) for x in _grads(w, np.zeros(w.q.shape)))


def pin_unseen_rows_have_zero_dq():
    """Causal Lq > Lk: the first Lq - Lk rows see no key and get dq = 0."""
    w = gi.fixed(1, 2, 1, 6, 3, 4, seed=29, dtype=torch.float32, causal=True)
    dq, _, _ = _grads(w, _do_like(w, 7))
    return bool(np.all(dq[0, :3] == 0) and np.abs(dq[0, 3:]).max() > 1e-3)


PINS = [pin_finite_differences_fixed, pin_finite_differences_varlen, pin_torch_sdpa_autograd,
        pin_gqa_equals_mha_summed, pin_v_shift_invariance, pin_dk_sums_to_zero,
        pin_zero_output_gradient, pin_unseen_rows_have_zero_dq]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin_holds(pin):
    assert pin()


# ---------------------------------------------------------------------------
# Planted mistakes
# ---------------------------------------------------------------------------

def _bad_head_grad(kind):
    def f(q, k, v, do, scale, vis):
        n, d = q.shape
        _, _, p = oa.head_rows(q, k, v, scale, vis, return_probs=True)
        dv = p.T @ do
        dp = do @ v.T
        ds = ob.softmax_backward(p, dp)
        dq = scale * (ds @ k)
        dk = scale * (ds.T @ q)
        if kind == "dq_uses_v":
            dq = scale * (ds @ v)
        elif kind == "dk_no_scale":
            dk = ds.T @ q
        elif kind == "dv_from_ds":
            dv = ds.T @ do
        return dq, dk, dv
    return f


def _group_first(per_head, hkv):
    hq = per_head.shape[1]
    g = hq // hkv
    return per_head[:, ::g].copy()


def _group_mod(per_head, hkv):
    out = np.zeros((per_head.shape[0], hkv, per_head.shape[2]))
    for h in range(per_head.shape[1]):
        out[:, h % hkv] += per_head[:, h]
    return out


MUTATIONS = {
    "no_rowsum_term": ("softmax_backward", lambda p, dp: p * dp),
    "rowsum_sign": ("softmax_backward",
                    lambda p, dp: p * (dp + (p * dp).sum(axis=1, keepdims=True))),
    "group_first_head_only": ("group_sum", _group_first),
    "group_map_mod": ("group_sum", _group_mod),
    "dq_uses_v": ("head_grad", _bad_head_grad("dq_uses_v")),
    "dk_no_scale": ("head_grad", _bad_head_grad("dk_no_scale")),
    "dv_from_ds": ("head_grad", _bad_head_grad("dv_from_ds")),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(ob, attr, fn)
    failed = []
    for p in PINS:
        try:
            ok = p()
        except (IndexError, ValueError):
            ok = False
        if not ok:
            failed.append(p.__name__)
    assert failed, f"mutation {name} slipped past every pin"


def test_sampled_gradients_match_full():
    """The row/key-sampled evaluator agrees with the full oracle."""
    for causal in (False, True):
        w = gi.fixed(2, 6, 2, 9, 7, 4, seed=31, dtype=torch.float32, causal=causal)
        do = _do_like(w, 8)
        dq, dk, dv = _grads(w, do)
        rows = [(0, 0, 0), (1, 8, 5), (0, 4, 3), (1, 1, 2)]
        keys = [(0, 0, 0), (1, 6, 1), (0, 3, 1)]
        sq, sk, sv = ob.attention_grad_sampled(w.q, w.k, w.v, do, w.scale, causal, rows, keys)
        assert _close(sq, [dq[b, i, h] for b, i, h in rows], 1e-12)
        assert _close(sk, [dk[b, j, g] for b, j, g in keys], 1e-12)
        assert _close(sv, [dv[b, j, g] for b, j, g in keys], 1e-12)
