"""fp64 CPU oracle for the gradient of exact grouped-query attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, links or runs
this module: only the tests, the smoke check and the bench's CPU-baseline leg
do. It shares no code with the HIP kernels.

FlashAttention-2 summary (azimuth.plus), paragraph on the backward pass: the
gradients are computed from the same inputs plus the stored row statistic,
and for grouped heads the key and value gradients are summed over the query
heads that share them. The page prints no formulas; the ones here are the
chain rule through the definition used by ``oracle.gqa`` (standard attention
as recalled on the same page), written out with every matrix materialised:

    S = scale q kᵀ (masked entries -inf),  P = row softmax of S,  O = P v
    dv = Pᵀ dO
    dP = dO vᵀ
    dS = P ∘ (dP - rowsum(P ∘ dP))          (the softmax Jacobian applied to dP)
    dq = scale dS k,   dk = scale dSᵀ q

for each query head against the K/V head of its group (Ultralytics glossary
"Grouped Query Attention (GQA)", section "How GQA works": head h uses K/V head
floor(h / G)); dk and dv of a K/V head are the sums over its G query heads.
Masked entries and rows with no visible key have P = 0 and contribute nothing.

Parity pins live in ``tests/test_oracle_grad.py``.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import gqa as _gqa


def softmax_backward(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """dS = P ∘ (dP - rowsum(P ∘ dP)): the Jacobian of a row softmax applied
    to the output gradient dP (rows of P that are all zero give zero)."""
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def head_grad(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
              vis: np.ndarray):
    """One query head against one K/V head (all fp64).

    q, do [n, d]; k, v [Lk, d]; vis [n, Lk] bool. Returns dq [n, d],
    dk [Lk, d], dv [Lk, d].
    """
    n, d = q.shape
    lk = k.shape[0]
    if n == 0 or lk == 0:
        return np.zeros((n, d)), np.zeros((lk, d)), np.zeros((lk, v.shape[1]))
    _, _, p = _gqa.head_rows(q, k, v, scale, vis, return_probs=True)
    dv = p.T @ do
    dp = do @ v.T
    ds = softmax_backward(p, dp)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def group_sum(per_head: np.ndarray, hkv: int) -> np.ndarray:
    """[L, Hq, d] per-query-head K/V gradients -> [L, Hkv, d]: K/V head g gets
    the sum over the query heads h with floor(h / G) = g."""
    hq = per_head.shape[1]
    out = np.zeros((per_head.shape[0], hkv, per_head.shape[2]))
    for h in range(hq):
        out[:, _gqa.kv_head_of(h, hq, hkv)] += per_head[:, h]
    return out


def _sequence_grad(q, k, v, do, scale: float, causal: bool):
    """One sequence: q, do [Lq, Hq, d]; k, v [Lk, Hkv, d] -> dq, dk, dv."""
    lq, hq, d = q.shape
    lk, hkv = k.shape[0], k.shape[1]
    vis = _gqa.visible(lq, lk, causal)
    dq = np.zeros(q.shape)
    dk_h = np.zeros((lk, hq, d))
    dv_h = np.zeros((lk, hq, v.shape[2]))
    for h in range(hq):
        g = _gqa.kv_head_of(h, hq, hkv)
        dq[:, h], dk_h[:, h], dv_h[:, h] = head_grad(q[:, h], k[:, g], v[:, g], do[:, h],
                                                      scale, vis)
    return dq, group_sum(dk_h, hkv), group_sum(dv_h, hkv)


def attention_grad(q, k, v, do, scale: float, causal: bool,
                   cu_seqlens_q: Optional[Sequence[int]] = None,
                   cu_seqlens_k: Optional[Sequence[int]] = None):
    """Gradients of exact GQA attention w.r.t. q, k, v for output gradient do.

    Layouts as ``oracle.gqa.attention`` (fixed [B, S, H, d] or packed
    variable length [T, H, d] with offsets); ``scale`` is used as the fp32
    value a kernel receives. Returns (dq, dk, dv) in fp64.
    """
    scale = float(np.float32(scale))
    q, k, v, do = (_gqa.as_f64(x) for x in (q, k, v, do))
    if cu_seqlens_q is None:
        dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
        for b in range(q.shape[0]):
            dq[b], dk[b], dv[b] = _sequence_grad(q[b], k[b], v[b], do[b], scale, causal)
        return dq, dk, dv
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(len(cq) - 1):
        qs, ks = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        dq[qs], dk[ks], dv[ks] = _sequence_grad(q[qs], k[ks], v[ks], do[qs], scale, causal)
    return dq, dk, dv


def attention_grad_sampled(q, k, v, do, scale: float, causal: bool, rows, keys):
    """The same gradients evaluated only at chosen rows (dq) and keys (dk, dv),
    for full-size workloads where materialising every P is too costly.

    Fixed length only. rows: (b, pos, head) triples -> dq [n, d]; keys:
    (b, key, kv_head) triples -> dk, dv [m, d]. Every row's LSE and
    D = rowsum(dO * O) come from the plain forward definition
    (``oracle.gqa.attention``); then, per the chain rule above,
        dq_i = scale sum_j P_ij (dP_ij - D_i) k_j
        dk_j = scale sum over rows i and query heads h of group(j) of
               P_ij (dP_ij - D_i) q_i,    dv_j = sum of P_ij dO_i.
    """
    scale = float(np.float32(scale))
    q, k, v, do = (_gqa.as_f64(x) for x in (q, k, v, do))
    o, lse = _gqa.attention(q, k, v, scale, causal)        # [B, Sq, Hq, d], [B, Hq, Sq]
    dsum = (do * o).sum(axis=-1)                             # [B, Sq, Hq]
    B, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    G = hq // hkv
    dq = np.zeros((len(rows), d))
    for n, (b, i, h) in enumerate(rows):
        g = _gqa.kv_head_of(h, hq, hkv)
        vis = _gqa.visible(sq, sk, causal)[i]
        s_row = scale * (k[b, :, g] @ q[b, i, h])
        p = np.where(vis, np.exp(s_row - lse[b, h, i]), 0.0) if np.isfinite(lse[b, h, i]) \
            else np.zeros(sk)
        dp = v[b, :, g] @ do[b, i, h]
        dq[n] = scale * ((p * (dp - dsum[b, i, h])) @ k[b, :, g])
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), v.shape[-1]))
    vis_all = _gqa.visible(sq, sk, causal)
    for n, (b, j, g) in enumerate(keys):
        for h in range(g * G, (g + 1) * G):
            s_col = scale * (q[b, :, h] @ k[b, j, g])
            l = lse[b, h]
            live = vis_all[:, j] & np.isfinite(l)
            p = np.zeros(sq)
            p[live] = np.exp(s_col[live] - l[live])
            dp = do[b, :, h] @ v[b, j, g]
            ds = p * (dp - dsum[b, :, h])
            dk[n] += scale * (ds @ q[b, :, h])
            dv[n] += p @ do[b, :, h]
    return dq, dk, dv


def attention_grad_flops(lq: int, lk: int, hq: int, d: int, causal: bool) -> int:
    """Algorithmic flops of the backward of one sequence: five products per
    visible (query, key) pair and query head (S, dP, dV, dQ, dK), each a
    multiply-add over d: 10 d per pair."""
    return 10 * d * hq * _pairs(lq, lk, causal)


def _pairs(lq: int, lk: int, causal: bool) -> int:
    if not causal:
        return lq * lk
    return sum(max(0, min(lk, i + 1 + lk - lq)) for i in range(lq))
