"""The pooled oracle driver equals the serial oracle bit for bit.

``oracle.pool.attention_pooled`` only schedules ``oracle.gqa.head_rows`` over
(sequence, head, row block) units in worker processes; the results must be
identical to ``oracle.gqa.attention`` (softmax is per row, so cutting the rows
changes nothing). Row blocks are forced small here so that every case spans
several blocks, including a ragged last one.
"""
import numpy as np
import pytest

import gqa_inputs
import oracle
from oracle import pool


@pytest.fixture(autouse=True)
def small_blocks(monkeypatch):
    # 8 KiB blocks: 16 rows of 64 keys per unit
    monkeypatch.setattr(pool, "_ROW_BLOCK_BYTES", 8 << 10)


def _same(a, b):
    assert a.shape == b.shape
    assert np.array_equal(a, b), float(np.nanmax(np.abs(a - b)))


@pytest.mark.parametrize("causal", [False, True])
def test_fixed_gqa_equals_serial(causal):
    w = gqa_inputs.fixed(2, 8, 2, 70, 64, 64, seed=31, causal=causal)
    ro, rl = oracle.attention(w.q, w.k, w.v, w.scale, causal)
    po, pl = pool.attention_pooled(w.q, w.k, w.v, w.scale, causal, workers=3)
    _same(po, ro)
    _same(pl, rl)


def test_varlen_with_empty_and_rectangular_sequences():
    w = gqa_inputs.varlen([33, 0, 50, 7], [40, 5, 50, 0], 6, 3, 32, seed=32, causal=True)
    cq, ck = w.cu_seqlens_q.tolist(), w.cu_seqlens_k.tolist()
    ro, rl = oracle.attention(w.q, w.k, w.v, w.scale, True, cq, ck)
    po, pl = pool.attention_pooled(w.q, w.k, w.v, w.scale, True, cq, ck, workers=2)
    _same(po, ro)
    _same(pl, rl)


def test_head_and_sequence_subsets():
    w = gqa_inputs.varlen([20, 30, 10], [20, 30, 10], 4, 2, 16, seed=33, causal=True)
    cq = w.cu_seqlens_q.tolist()
    ro, rl = oracle.attention(w.q, w.k, w.v, w.scale, True, cq, cq)
    po, pl = pool.attention_pooled(w.q, w.k, w.v, w.scale, True, cq, cq, workers=2,
                                   heads=[1, 2], seqs=[0, 2])
    for b in (0, 2):
        for h in (1, 2):
            _same(po[cq[b]:cq[b + 1], h], ro[cq[b]:cq[b + 1], h])
            _same(pl[cq[b]:cq[b + 1], h], rl[cq[b]:cq[b + 1], h])
    # rows outside the subset are left untouched
    assert not po[cq[1]:cq[2]].any() and np.isneginf(pl[cq[1]:cq[2]]).all()
    assert not po[:, 0].any() and not po[:, 3].any()


def test_fp32_inputs_and_stats():
    w = gqa_inputs.tiny_causal_gqa_fp32()
    ro, rl = oracle.attention(w.q, w.k, w.v, w.scale, True)
    st = {}
    po, pl = pool.attention_pooled(w.q, w.k, w.v, w.scale, True, workers=2, stats=st)
    _same(po, ro)
    _same(pl, rl)
    assert st["workers"] == 2 and st["units"] >= 8
    assert st["score_pairs"] == 8 * 16 * 16
