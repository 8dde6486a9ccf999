"""Pins for the fp64 oracle, run on the CPU (no GPU marker).

The oracle is checked against things other than itself: a pure-Python brute
force, PyTorch's float64 CPU scaled_dot_product_attention, closed forms,
invariants the pages state, and the figures the glossary page prints. The
mutation tests at the bottom plant plausible mistakes in the oracle and check
that at least one pin catches each.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import gqa_inputs
import oracle
from oracle import gqa as oa
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _to_lists(x):
    return oa.as_f64(x).tolist()


def _brute_fixed(w):
    q, k, v = _to_lists(w.q), _to_lists(w.k), _to_lists(w.v)
    scale = float(np.float32(w.scale))
    outs, lses = [], []
    for b in range(len(q)):
        o, l = brute.sequence(q[b], k[b], v[b], scale, w.causal)
        outs.append(o)
        lses.append(l)
    return np.array(outs, dtype=np.float64), np.array(lses, dtype=np.float64)


def _brute_varlen(w):
    q, k, v = _to_lists(w.q), _to_lists(w.k), _to_lists(w.v)
    scale = float(np.float32(w.scale))
    cq, ck = w.cu_seqlens_q.tolist(), w.cu_seqlens_k.tolist()
    hq, d = w.q.shape[1], w.q.shape[2]
    out = np.zeros((w.q.shape[0], hq, d))
    lse = np.full((w.q.shape[0], hq), -np.inf)
    for b in range(len(cq) - 1):
        o, l = brute.sequence(q[cq[b]:cq[b + 1]], k[ck[b]:ck[b + 1]],
                              v[ck[b]:ck[b + 1]], scale, w.causal)
        if cq[b + 1] > cq[b]:
            out[cq[b]:cq[b + 1]] = np.array(o)
            lse[cq[b]:cq[b + 1]] = np.array(l).T
    return out, lse


def _close(a, b, tol):
    a, b = np.asarray(a), np.asarray(b)
    if a.shape != b.shape:
        return False
    fin = np.isfinite(b)
    if not np.array_equal(np.isfinite(a), fin):
        return False
    if not np.array_equal(a[~fin], b[~fin]):
        return False
    return bool(np.all(np.abs(a[fin] - b[fin]) <= tol))


# ---------------------------------------------------------------------------
# Pins. Each returns True when it holds for the oracle as currently loaded.
# ---------------------------------------------------------------------------

TINY_FIXED = [
    # B, Hq, Hkv, Sq, Sk, d, causal
    (1, 1, 1, 1, 1, 1, False), (2, 2, 1, 3, 5, 2, True), (1, 4, 2, 5, 3, 4, True),
    (2, 4, 4, 2, 2, 2, False), (1, 4, 1, 5, 5, 4, True), (2, 2, 2, 3, 2, 1, True),
    (1, 4, 2, 3, 5, 4, False), (2, 4, 1, 2, 3, 2, False), (1, 2, 1, 5, 2, 4, True),
    (1, 6, 2, 3, 3, 2, True),
]


def pin_brute_fixed():
    for i, (B, hq, hkv, sq, sk, d, causal) in enumerate(TINY_FIXED):
        w = gqa_inputs.fixed(B, hq, hkv, sq, sk, d, seed=100 + i, dtype=torch.float32,
                             causal=causal, scale=0.7)
        o, l = oracle.attention(w.q, w.k, w.v, w.scale, w.causal)
        bo, bl = _brute_fixed(w)
        if not (_close(o, bo, 1e-12) and _close(l, bl, 1e-12)):
            return False
    return True


TINY_VARLEN = [
    # lengths_q, lengths_k, Hq, Hkv, d, causal
    ([2, 0, 3], [2, 0, 3], 4, 2, 2, True),
    ([3, 1], [5, 2], 2, 1, 4, True),
    ([1, 2, 3], [3, 0, 1], 4, 4, 2, False),
    ([5, 2], [2, 5], 4, 1, 2, True),
]


def pin_brute_varlen():
    for i, (lq, lk, hq, hkv, d, causal) in enumerate(TINY_VARLEN):
        w = gqa_inputs.varlen(lq, lk, hq, hkv, d, seed=200 + i, dtype=torch.float32,
                              causal=causal, scale=0.9)
        o, l = oracle.attention(w.q, w.k, w.v, w.scale, w.causal,
                                w.cu_seqlens_q.tolist(), w.cu_seqlens_k.tolist())
        bo, bl = _brute_varlen(w)
        if not (_close(o, bo, 1e-12) and _close(l, bl, 1e-12)):
            return False
    return True


def pin_sdpa_float64():
    """PyTorch float64 CPU SDPA with enable_gqa on the glossary snippet's draws."""
    w = gqa_inputs.tiny_causal_gqa_fp32()
    o, l = oracle.attention(w.q, w.k, w.v, w.scale, True)
    q = w.q.transpose(1, 2).double()
    k = w.k.transpose(1, 2).double()
    v = w.v.transpose(1, 2).double()
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, is_causal=True, enable_gqa=True, scale=float(np.float32(w.scale)))
    ref = ref.transpose(1, 2).numpy()
    s = float(np.float32(w.scale)) * torch.matmul(
        q, k.repeat_interleave(4, dim=1).transpose(-1, -2))
    mask = torch.ones(16, 16, dtype=torch.bool).tril()
    lref = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1).numpy()
    return _close(o, ref, 1e-12) and _close(l, lref, 1e-12)


def pin_sdpa_noncausal_rect():
    """Same library cross-check without a mask and with Sq != Sk."""
    w = gqa_inputs.fixed(2, 6, 3, 7, 11, 8, seed=7, dtype=torch.float32, scale=0.3)
    o, l = oracle.attention(w.q, w.k, w.v, w.scale, False)
    q, k, v = (x.transpose(1, 2).double() for x in (w.q, w.k, w.v))
    sc = float(np.float32(w.scale))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, enable_gqa=True, scale=sc).transpose(1, 2).numpy()
    s = sc * torch.matmul(q, k.repeat_interleave(2, dim=1).transpose(-1, -2))
    lref = torch.logsumexp(s, dim=-1).numpy()
    return _close(o, ref, 1e-12) and _close(l, lref, 1e-12)


def pin_causal_row0():
    """Lq = Lk causal: row 0 sees only key 0, so O = V[0] and LSE = s q0.k0."""
    w = gqa_inputs.fixed(2, 4, 2, 9, 9, 16, seed=11, dtype=torch.float32, causal=True)
    o, l = oracle.attention(w.q, w.k, w.v, w.scale, True)
    q, k, v = (oa.as_f64(x) for x in (w.q, w.k, w.v))
    sc = float(np.float32(w.scale))
    for b in range(2):
        for h in range(4):
            g = h // 2
            if np.max(np.abs(o[b, 0, h] - v[b, 0, g])) > 1e-12:
                return False
            if abs(l[b, h, 0] - sc * float(np.dot(q[b, 0, h], k[b, 0, g]))) > 1e-12:
                return False
    return True


def pin_zero_query():
    """q = 0: uniform weights over the visible keys, O = their mean, LSE = log(count)."""
    w = gqa_inputs.fixed(1, 4, 2, 6, 8, 4, seed=12, dtype=torch.float32, causal=True)
    q = torch.zeros_like(w.q)
    o, l = oracle.attention(q, w.k, w.v, w.scale, True)
    v = oa.as_f64(w.v)
    for i in range(6):
        cnt = i + 1 + (8 - 6)
        for h in range(4):
            if np.max(np.abs(o[0, i, h] - v[0, :cnt, h // 2].mean(axis=0))) > 1e-12:
                return False
            if abs(l[0, h, i] - math.log(cnt)) > 1e-12:
                return False
    return True


def pin_single_key():
    """Sk = 1: O = v0 and LSE = s q.k0 for every row."""
    w = gqa_inputs.fixed(2, 4, 1, 3, 1, 8, seed=13, dtype=torch.float32)
    o, l = oracle.attention(w.q, w.k, w.v, w.scale, False)
    q, k, v = (oa.as_f64(x) for x in (w.q, w.k, w.v))
    sc = float(np.float32(w.scale))
    exp_o = np.broadcast_to(v[:, :, :1, :], o.shape)
    exp_l = sc * np.einsum("bihd,bd->bhi", q, k[:, 0, 0, :])
    return _close(o, exp_o, 1e-12) and _close(l, exp_l, 1e-12)


def pin_constant_v():
    """V = c everywhere gives O = c (convex combination)."""
    w = gqa_inputs.fixed(1, 4, 2, 5, 7, 4, seed=14, dtype=torch.float32, causal=True)
    v = torch.full_like(w.v, 1.75)
    o, _ = oracle.attention(w.q, w.k, v, w.scale, True)
    return bool(np.max(np.abs(o - 1.75)) <= 1e-12)


def pin_probs_rows_sum_to_one():
    """Row softmax: every P row sums to 1 and 0 <= P <= 1; masked entries are 0."""
    rng = np.random.default_rng(15)
    q, k, v = rng.standard_normal((6, 8)), rng.standard_normal((9, 8)), rng.standard_normal((9, 3))
    vis = oa.visible(6, 9, True)
    _, _, p = oa.head_rows(q, k, v, 0.5, vis, return_probs=True)
    return (np.max(np.abs(p.sum(axis=1) - 1)) <= 1e-12 and p.min() >= 0 and p.max() <= 1
            and np.all(p[~vis] == 0))


def pin_key_permutation():
    """Non-causal: permuting keys together with values changes nothing."""
    w = gqa_inputs.fixed(1, 4, 2, 5, 11, 8, seed=16, dtype=torch.float32)
    o, l = oracle.attention(w.q, w.k, w.v, w.scale, False)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(11))
    o2, l2 = oracle.attention(w.q, w.k[:, perm], w.v[:, perm], w.scale, False)
    return _close(o, o2, 1e-12) and _close(l, l2, 1e-12)


def pin_gqa_equals_expanded_mha():
    """Glossary snippet: GQA equals MHA on repeat-interleaved K/V (to 1e-6 on
    fp32 inputs; the oracle gives equality to rounding)."""
    w = gqa_inputs.tiny_causal_gqa_fp32()
    o, l = oracle.attention(w.q, w.k, w.v, w.scale, True)
    kx = w.k.repeat_interleave(4, dim=2)
    vx = w.v.repeat_interleave(4, dim=2)
    o2, l2 = oracle.attention(w.q, kx, vx, w.scale, True)
    # the MHA form has Hkv = Hq and so reads its own head in every query head
    b = _brute_fixed(gqa_inputs.Workload("x", w.q, kx, vx, True, w.scale))
    return _close(o, o2, 1e-12) and _close(l, l2, 1e-12) and _close(o2, b[0], 1e-12)


def pin_split_merge():
    """Merging per-split results through their LSEs equals the unsplit result."""
    w = gqa_inputs.decode(3, 8, 2, 37, 16, seed=17, dtype=torch.float32)
    o, l = oracle.decode(w.q, w.k, w.v, w.scale)
    for ns in (1, 2, 3, 4, 8, 64):
        po, pl = oracle.decode_partials(w.q, w.k, w.v, w.scale, ns, align=8)
        mo, ml = oracle.merge_partials(po, pl)
        if not (_close(mo, o, 1e-12) and _close(ml, l, 1e-12)):
            return False
    return True


def pin_varlen_is_per_sequence():
    """A packed batch equals each sequence run on its own."""
    w = gqa_inputs.varlen([3, 4, 1], [5, 4, 2], 4, 2, 8, seed=18, dtype=torch.float32,
                          causal=True)
    cq, ck = w.cu_seqlens_q.tolist(), w.cu_seqlens_k.tolist()
    o, l = oracle.attention(w.q, w.k, w.v, w.scale, True, cq, ck)
    for b in range(3):
        ob, lb = oracle.attention(w.q[None, cq[b]:cq[b + 1]], w.k[None, ck[b]:ck[b + 1]],
                                  w.v[None, ck[b]:ck[b + 1]], w.scale, True)
        if not (_close(o[cq[b]:cq[b + 1]], ob[0], 0) and _close(l[cq[b]:cq[b + 1]], lb[0].T, 0)):
            return False
    return True


def pin_fully_masked_rows():
    """Causal with Lq > Lk: the first Lq - Lk rows see no key: O = 0, LSE = -inf."""
    w = gqa_inputs.fixed(1, 2, 1, 6, 3, 4, seed=19, dtype=torch.float32, causal=True)
    o, l = oracle.attention(w.q, w.k, w.v, w.scale, True)
    return (np.all(o[0, :3] == 0) and np.all(np.isneginf(l[0, :, :3]))
            and np.all(np.isfinite(l[0, :, 3:])))


def pin_rows_subset():
    """attention_rows agrees with the full oracle at the sampled rows."""
    w = gqa_inputs.fixed(2, 4, 2, 9, 13, 8, seed=20, dtype=torch.float32, causal=True)
    o, l = oracle.attention(w.q, w.k, w.v, w.scale, True)
    rows = [(0, 0, 0), (1, 8, 3), (0, 4, 1), (1, 2, 2)]
    ro, rl = oracle.attention_rows(w.q, w.k, w.v, w.scale, True, rows)
    want_o = np.array([o[b, i, h] for b, i, h in rows])
    want_l = np.array([l[b, h, i] for b, i, h in rows])
    wv = gqa_inputs.varlen([3, 6], [3, 6], 4, 2, 8, seed=21, dtype=torch.float32, causal=True)
    cq = wv.cu_seqlens_q.tolist()
    vo, vl = oracle.attention(wv.q, wv.k, wv.v, wv.scale, True, cq, cq)
    vrows = [(0, 2, 1), (1, 0, 3), (1, 5, 0)]
    so, sl = oracle.attention_rows(wv.q, wv.k, wv.v, wv.scale, True, vrows, cq, cq)
    want_vo = np.array([vo[cq[b] + i, h] for b, i, h in vrows])
    want_vl = np.array([vl[cq[b] + i, h] for b, i, h in vrows])
    return (_close(ro, want_o, 1e-13) and _close(rl, want_l, 1e-13)
            and _close(so, want_vo, 1e-13) and _close(sl, want_vl, 1e-13))


PINS = [pin_brute_fixed, pin_brute_varlen, pin_sdpa_float64, pin_sdpa_noncausal_rect,
        pin_causal_row0, pin_zero_query, pin_single_key, pin_constant_v,
        pin_probs_rows_sum_to_one, pin_key_permutation, pin_gqa_equals_expanded_mha,
        pin_split_merge, pin_varlen_is_per_sequence, pin_fully_masked_rows,
        pin_rows_subset]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin_holds(pin):
    assert pin()


# ---------------------------------------------------------------------------
# Printed figures from the pages.
# ---------------------------------------------------------------------------

def test_golden_glossary_snippet():
    """The snippet prints shape (1, 8, 16, 64), 'True' for allclose(atol=1e-6)
    against repeat-interleaved heads, and 256 / 1024 cached values per token."""
    gold = json.load(open(os.path.join(GOLDEN, "kv_cache.json")))["snippet"]
    w = gqa_inputs.tiny_causal_gqa_fp32()
    assert list(w.q.transpose(1, 2).shape) == gold["q_shape_bhsd"]
    assert list(w.k.transpose(1, 2).shape) == gold["kv_shape_bhsd"]
    o, _ = oracle.attention(w.q, w.k, w.v, w.scale, True)
    assert list(o.transpose(0, 2, 1, 3).shape) == gold["printed_output_shape"]
    kx, vx = w.k.repeat_interleave(4, dim=2), w.v.repeat_interleave(4, dim=2)
    o2, _ = oracle.attention(w.q, kx, vx, w.scale, True)
    same = bool(np.allclose(o, o2, atol=gold["allclose_atol"], rtol=0))
    assert same == gold["printed_same_as_copied_heads"]
    d, hkv, hq = w.k.shape[-1], w.k.shape[2], w.q.shape[2]
    assert oracle.kv_cache_elements(1, 1, d, hkv) == gold["printed_cached_values_per_token_per_layer_gqa"]
    assert oracle.kv_cache_elements(1, 1, d, hq) == gold["printed_cached_values_per_token_per_layer_mha"]


def test_golden_llama_kv_cache():
    gold = json.load(open(os.path.join(GOLDEN, "kv_cache.json")))["llama31_8b"]
    per_tok = oracle.kv_cache_bytes(1, 1, gold["head_dim"], gold["kv_heads"], gold["layers"],
                                    gold["bytes_per_value"])
    assert per_tok == gold["printed_bytes_per_token"] == 128 * 1024
    full = oracle.kv_cache_bytes(1, gold["max_context_tokens"], gold["head_dim"],
                                 gold["kv_heads"], gold["layers"], gold["bytes_per_value"])
    assert full == gold["printed_bytes_at_max_context"] == 16 * 2 ** 30
    mha_tok = oracle.kv_cache_bytes(1, 1, gold["head_dim"], gold["query_heads"], gold["layers"])
    assert mha_tok == gold["printed_mha_bytes_per_token"]
    mha_full = oracle.kv_cache_bytes(1, gold["max_context_tokens"], gold["head_dim"],
                                     gold["query_heads"], gold["layers"])
    assert mha_full == gold["printed_mha_bytes_at_max_context"]


def test_golden_guide_saving():
    gold = json.load(open(os.path.join(GOLDEN, "kv_cache.json")))["guide_4to1"]
    gqa = oracle.kv_cache_elements(1, 1, 128, gold["kv_heads"])
    mha = oracle.kv_cache_elements(1, 1, 128, gold["query_heads"])
    assert 1 - gqa / mha == pytest.approx(gold["printed_saving_vs_mha"])


def test_flop_count_brute():
    """Algorithmic flops: 4 d per visible pair per query head; causal Lq = Lk
    gives L(L+1)/2 pairs."""
    assert oracle.attention_flops(16, 16, 8, 64, True) == 4 * 64 * 8 * 136
    assert oracle.attention_flops(5, 7, 2, 4, False) == 4 * 4 * 2 * 35
    vis = oa.visible(5, 9, True)
    assert oracle.attention_flops(5, 9, 3, 8, True) == 4 * 8 * 3 * int(vis.sum())


# ---------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail.
# ---------------------------------------------------------------------------

def _bad_head_rows(kind):
    orig = oa.head_rows

    def f(q, k, v, scale, vis, return_probs=False):
        if kind == "no_scale":
            return orig(q, k, v, 1.0, vis, return_probs)
        if kind == "squared_scale":
            return orig(q, k, v, scale * scale, vis, return_probs)
        if kind == "k_for_v":
            return orig(q, k, k[:, :v.shape[1]] if k.shape[1] >= v.shape[1] else v * 0, scale,
                        vis, return_probs)
        res = orig(q, k, v, scale, vis, return_probs)
        o, l = res[0], res[1]
        if kind == "lse_log2":
            l = l / math.log(2.0)
        elif kind == "lse_no_max":
            s = np.where(vis, scale * (q @ k.T), -np.inf) if len(k) else np.zeros((len(q), 0))
            m = s.max(axis=1) if s.shape[1] else np.full(len(q), -np.inf)
            l = np.where(np.isfinite(m), l - m, l)
        elif kind == "unnormalised":
            s = np.where(vis, scale * (q @ k.T), -np.inf) if len(k) else np.zeros((len(q), 0))
            if s.shape[1]:
                e = np.exp(s - s.max(axis=1, keepdims=True))
                e = np.nan_to_num(e)
                o = e @ v
        elif kind == "mask_zero":
            s = np.where(vis, scale * (q @ k.T), 0.0) if len(k) else np.zeros((len(q), 0))
            if s.shape[1]:
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                o = (e / e.sum(axis=1, keepdims=True)) @ v
                l = (m[:, 0] + np.log(e.sum(axis=1)))
        return (o, l) + tuple(res[2:])
    return f


MUTATIONS = {
    "head_map_mod": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "diagonal_masked": ("visible", lambda lq, lk, causal: (
        np.ones((lq, lk), bool) if not causal else
        np.arange(lk)[None, :] < np.arange(lq)[:, None] + (lk - lq))),
    "top_left_causal": ("visible", lambda lq, lk, causal: (
        np.ones((lq, lk), bool) if not causal else
        np.arange(lk)[None, :] <= np.arange(lq)[:, None])),
    "causal_ignored": ("visible", lambda lq, lk, causal: np.ones((lq, lk), bool)),
    "no_scale": ("head_rows", _bad_head_rows("no_scale")),
    "squared_scale": ("head_rows", _bad_head_rows("squared_scale")),
    "k_for_v": ("head_rows", _bad_head_rows("k_for_v")),
    "lse_log2": ("head_rows", _bad_head_rows("lse_log2")),
    "lse_no_max": ("head_rows", _bad_head_rows("lse_no_max")),
    "unnormalised": ("head_rows", _bad_head_rows("unnormalised")),
    "mask_zero": ("head_rows", _bad_head_rows("mask_zero")),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oa, attr, fn)
    failed = [p.__name__ for p in PINS if not p()]
    assert failed, f"mutation {name} slipped past every pin"
