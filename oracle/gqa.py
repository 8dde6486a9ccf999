"""fp64 CPU oracle for exact grouped-query attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, links or runs
this module: only the tests, the smoke check and the bench's CPU-baseline leg
do. It shares no code with the HIP kernels.

What it computes is the plain definition, written out with S and P
materialised and K/V expanded per query head:

* FlashAttention-2 summary (azimuth.plus), paragraph recalling standard
  attention: S = Q Kᵀ, a row-wise softmax gives P, and O = P V. The same page
  states that tiling with a running max and running sum reaches this result
  with no approximation, so the tiled GPU method must equal this definition up
  to rounding.
* Ultralytics glossary "Grouped Query Attention (GQA)", section "How GQA
  works": each query head computes unchanged exact scaled dot-product
  attention against the K/V head of its group; the snippet builds the
  equivalent MHA with ``repeat_interleave`` along the head axis, so query head
  h uses KV head floor(h / G) with G = Hq / Hkv.
* FlashAttention-2 summary, paragraph on causal masking: entries above the
  diagonal of S are set to -inf (the diagonal itself stays visible).
* FlashAttention-2 summary, paragraph on deferred normalisation: the stored
  per-row statistic is L = m + log(l), the log of the row's sum of
  exponentials of the scaled scores (natural log).

Readings where the pages are silent:

* the scale multiplies Q Kᵀ before the softmax and the LSE is taken over the
  scaled scores;
* causal alignment when Lq != Lk is bottom-right: key j is visible to query i
  iff j <= i + (Lk - Lq);
* a row with no visible key has O = 0 and LSE = -inf (the empty-sum limit);
* a variable-length batch is the concatenation of independent sequences whose
  rows and keys are given by prefix offsets ``cu_seqlens``.

All inputs are upcast to float64 exactly (bf16 and fp32 both embed exactly).
Row blocks are chunked only to bound memory; softmax is per row so chunking is
exact.

Parity pins for every function here live in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

_ROW_CHUNK_BYTES = 64 << 20  # cap on one materialised S/P block


def as_f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (bf16/fp16/fp32/fp64) or array to fp64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """KV head used by query head h: floor(h / G), G = Hq / Hkv.

    Glossary page, "How GQA works": the equivalent MHA repeats each KV head
    G times consecutively along the head axis (repeat_interleave).
    """
    return h // (hq // hkv)


def expand_kv(kv: np.ndarray, hq: int) -> np.ndarray:
    """[L, Hkv, d] -> [L, Hq, d]: copy each KV head to its G query heads."""
    hkv = kv.shape[1]
    index = [kv_head_of(h, hq, hkv) for h in range(hq)]
    return kv[:, index, :]


def visible(lq: int, lk: int, causal: bool) -> np.ndarray:
    """Boolean [lq, lk]: may query row i attend to key j?

    Causal: FlashAttention-2 summary, causal-masking paragraph (above the
    diagonal is masked, the diagonal is kept); bottom-right aligned.
    """
    if not causal:
        return np.ones((lq, lk), dtype=bool)
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    return j <= i + (lk - lq)


def head_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              vis: np.ndarray, return_probs: bool = False):
    """Exact softmax attention of some query rows against one head's keys.

    q [n, d], k [Lk, d], v [Lk, d] (fp64), vis [n, Lk] bool.
    Returns O [n, d] and LSE [n] (and P [n, Lk] when asked).

    Standard attention as recalled on the FlashAttention-2 page: scaled scores
    S = scale * q kᵀ, masked entries -inf, P = row softmax of S, O = P v,
    LSE = log(sum_j exp(S_ij)). The row max is subtracted before exp only to
    stay in fp64 range; it cancels exactly in P and is added back in LSE.
    """
    n, d = q.shape
    lk = k.shape[0]
    out = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full((n,), -np.inf, dtype=np.float64)
    probs = np.zeros((n, lk), dtype=np.float64) if return_probs else None
    if n == 0 or lk == 0:
        return (out, lse, probs) if return_probs else (out, lse)
    s = scale * (q @ k.T)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    live = np.isfinite(m)
    e = np.zeros_like(s)
    e[live] = np.exp(s[live] - m[live, None])
    den = e.sum(axis=1)
    p = np.zeros_like(s)
    p[live] = e[live] / den[live, None]
    out[live] = p[live] @ v
    lse[live] = m[live] + np.log(den[live])
    if return_probs:
        probs[:] = p
        return out, lse, probs
    return out, lse


def _sequence(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              causal: bool) -> Tuple[np.ndarray, np.ndarray]:
    """One sequence: q [Lq, Hq, d], k/v [Lk, Hkv, d] -> O [Lq, Hq, d], LSE [Hq, Lq]."""
    lq, hq, d = q.shape
    lk = k.shape[0]
    kx = expand_kv(k, hq)
    vx = expand_kv(v, hq)
    vis = visible(lq, lk, causal)
    out = np.zeros((lq, hq, v.shape[2]), dtype=np.float64)
    lse = np.full((hq, lq), -np.inf, dtype=np.float64)
    step = max(1, _ROW_CHUNK_BYTES // (8 * max(lk, 1)))
    for h in range(hq):
        for r0 in range(0, lq, step):
            r1 = min(lq, r0 + step)
            o, l = head_rows(q[r0:r1, h, :], kx[:, h, :], vx[:, h, :], scale,
                             vis[r0:r1])
            out[r0:r1, h, :] = o
            lse[h, r0:r1] = l
    return out, lse


def attention(q, k, v, scale: float, causal: bool,
              cu_seqlens_q: Optional[Sequence[int]] = None,
              cu_seqlens_k: Optional[Sequence[int]] = None):
    """Exact GQA attention forward in fp64.

    Fixed length: q [B, Sq, Hq, d], k/v [B, Sk, Hkv, d] ->
        O [B, Sq, Hq, d], LSE [B, Hq, Sq].
    Variable length (both offset arrays given): q [Tq, Hq, d], k/v [Tk, Hkv, d]
        -> O [Tq, Hq, d], LSE [Tq, Hq]; sequence b owns rows
        cu_q[b]:cu_q[b+1] and keys cu_k[b]:cu_k[b+1].
    ``scale`` is used as the fp32 value a kernel receives.
    """
    scale = float(np.float32(scale))
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    if q.shape[-2] % k.shape[-2] != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if cu_seqlens_q is None:
        B, sq, hq, _ = q.shape
        out = np.zeros(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
        lse = np.full((B, hq, sq), -np.inf, dtype=np.float64)
        for b in range(B):
            out[b], lse[b] = _sequence(q[b], k[b], v[b], scale, causal)
        return out, lse
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    hq = q.shape[1]
    out = np.zeros(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    lse = np.full((q.shape[0], hq), -np.inf, dtype=np.float64)
    for b in range(len(cq) - 1):
        o, l = _sequence(q[cq[b]:cq[b + 1]], k[ck[b]:ck[b + 1]],
                         v[ck[b]:ck[b + 1]], scale, causal)
        out[cq[b]:cq[b + 1]] = o
        lse[cq[b]:cq[b + 1]] = l.T
    return out, lse


def decode(q, k_cache, v_cache, scale: float):
    """One new token per sequence attending to its whole cache (no mask).

    Glossary page, KV-cache section: each new token reads the cache in full.
    q [B, Hq, d], caches [B, Sk, Hkv, d] -> O [B, Hq, d], LSE [B, Hq].
    """
    q = as_f64(q)
    out, lse = attention(q[:, None], k_cache, v_cache, scale, False)
    return out[:, 0], lse[:, :, 0]


def attention_rows(q, k, v, scale: float, causal: bool, rows,
                   cu_seqlens_q=None, cu_seqlens_k=None):
    """The same definition evaluated only at chosen (sequence, row, head) triples.

    Used for parity at full workload sizes, where materialising every row is
    too slow. ``rows`` is an iterable of (b, i, h) with i the row inside
    sequence b. Returns O [n, d] and LSE [n].
    """
    scale = float(np.float32(scale))
    rows = list(rows)
    out = np.zeros((len(rows), v.shape[-1]), dtype=np.float64)
    lse = np.full((len(rows),), -np.inf, dtype=np.float64)
    hq = q.shape[-2]
    hkv = k.shape[-2]
    cache = {}

    def kv_rows(b, kvh):
        key = (b, kvh)
        if key not in cache:
            if cu_seqlens_q is None:
                cache[key] = (as_f64(k[b, :, kvh]), as_f64(v[b, :, kvh]))
            else:
                k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
                cache[key] = (as_f64(k[k0:k1, kvh]), as_f64(v[k0:k1, kvh]))
        return cache[key]

    for t, (b, i, h) in enumerate(rows):
        kh, vh = kv_rows(b, kv_head_of(h, hq, hkv))
        if cu_seqlens_q is None:
            qrow = as_f64(q[b, i, h])[None, :]
            lq = q.shape[1]
        else:
            q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
            qrow = as_f64(q[q0 + i, h])[None, :]
            lq = q1 - q0
        vis = visible(lq, kh.shape[0], causal)[i:i + 1]
        o, l = head_rows(qrow, kh, vh, scale, vis)
        out[t], lse[t] = o[0], l[0]
    return out, lse


def split_ranges(sk: int, num_splits: int, align: int = 1):
    """Contiguous key ranges for split-KV: chunk = ceil(Sk / ns) rounded up to
    a multiple of ``align``; trailing splits may be empty.

    The gitcode GQA guide names the ``num_splits`` knob (parameter table and
    code sample) but prints no partition; contiguous equal chunks are the
    plainest reading. The result does not depend on the partition beyond
    rounding.
    """
    chunk = -(-sk // num_splits)
    chunk = -(-chunk // align) * align
    return [(min(sk, s * chunk), min(sk, (s + 1) * chunk)) for s in range(num_splits)]


def decode_partials(q, k_cache, v_cache, scale: float, num_splits: int,
                    align: int = 1):
    """Per-split (O_s, LSE_s) of decode: the definition over each key range.

    Returns O [ns, B, Hq, d] (each normalised over its own keys; zeros for an
    empty split) and LSE [ns, B, Hq] (-inf for an empty split).
    """
    sk = k_cache.shape[1]
    os_, ls_ = [], []
    for a, b in split_ranges(sk, num_splits, align):
        o, l = decode(q, k_cache[:, a:b], v_cache[:, a:b], scale)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_), np.stack(ls_)


def merge_partials(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge split results through their LSEs (split axis first).

    Not printed on the pages; it follows from the LSE definition on the
    FlashAttention-2 page: log-sum-exp over a partition of the keys is
    L = M + log sum_s exp(L_s - M) with M = max_s L_s, and each split's
    normalised output is weighted by exp(L_s - L). Empty splits (L_s = -inf)
    get weight 0.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    live = np.isfinite(m)
    w = np.zeros_like(lse_parts)
    w[:, live] = np.exp(lse_parts[:, live] - m[live])
    tot = w.sum(axis=0)
    lse = np.full(m.shape, -np.inf)
    lse[live] = m[live] + np.log(tot[live])
    out = np.zeros(o_parts.shape[1:])
    out[live] = (w[:, live, None] * o_parts[:, live]).sum(axis=0) / tot[live, None]
    return out, lse


def attention_flops(lq: int, lk: int, hq: int, d: int, causal: bool) -> int:
    """Algorithmic flops of one sequence: 4 d per visible (query, key) pair and
    query head (two products, one multiply-add = 2 flops)."""
    if not causal:
        pairs = lq * lk
    else:
        pairs = sum(max(0, min(lk, i + 1 + lk - lq)) for i in range(lq))
    return 4 * d * hq * pairs
