"""Scalar brute-force attention in pure Python.

TEST INFRASTRUCTURE ONLY (see ``oracle/gqa.py``). A second, independent
statement of the same definition, used to pin the NumPy oracle on tiny shapes:
no NumPy, no K/V expansion, no matrix routines. Each query head h reads KV
head h // G directly (Ultralytics glossary "Grouped Query Attention (GQA)",
section "How GQA works"); causal visibility is j <= i + (Lk - Lq)
(FlashAttention-2 summary, causal-masking paragraph, diagonal kept); the
softmax, output and log-sum-exp follow the standard attention recalled on the
FlashAttention-2 page, with math.fsum for every sum.

Inputs are nested Python lists (or anything indexable) of floats.
"""
from __future__ import annotations

import math


def attend_row(qv, keys, values, scale):
    """One query vector against a list of visible (key, value) vectors.

    Returns (output vector, log-sum-exp). No keys -> zeros and -inf.
    """
    if not keys:
        return [0.0] * (len(values[0]) if values else len(qv)), -math.inf
    scores = [scale * math.fsum(a * b for a, b in zip(qv, kv)) for kv in keys]
    top = max(scores)
    weights = [math.exp(s - top) for s in scores]
    total = math.fsum(weights)
    dv = len(values[0])
    out = [math.fsum(w * val[t] for w, val in zip(weights, values)) / total
           for t in range(dv)]
    return out, top + math.log(total)


def sequence(q, k, v, scale, causal):
    """q[i][h][t], k[j][g][t], v[j][g][t] for one sequence.

    Returns O[i][h][t] and LSE[h][i].
    """
    lq, lk = len(q), len(k)
    hq = len(q[0]) if lq else 0
    hkv = len(k[0]) if lk else 1
    group = hq // hkv if hkv else 1
    out = [[None] * hq for _ in range(lq)]
    lse = [[None] * lq for _ in range(hq)]
    for h in range(hq):
        g = h // group
        for i in range(lq):
            vis = [j for j in range(lk) if (not causal) or j <= i + (lk - lq)]
            o, l = attend_row(q[i][h], [k[j][g] for j in vis],
                              [v[j][g] for j in vis], scale)
            if not vis:
                o = [0.0] * len(q[i][h])
            out[i][h] = o
            lse[h][i] = l
    return out, lse
