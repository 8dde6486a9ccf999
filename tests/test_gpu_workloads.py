"""GPU parity at the five named workloads' full sizes, in the launch
configuration the bench times.

Every output row of every workload is compared with the fp64 oracle element
by element: the tiny causal GQA workload in fp32, the BERT-base encoder, the
8192-token causal prefill (all 262,144 (row, head) outputs), decode at every
num_splits, and the packed variable-length batch (all 3.7 M outputs, in four
parts of eight sequences each so that every test stays short). The large
ones run the oracle as a process pool (``oracle.pool``: one process per core,
the plain definition per (sequence, head, row block)).
"""
import numpy as np
import pytest
import torch

import gqa_attention_amd as ga
import gqa_inputs
import oracle

from oracle import pool
from parity_util import compare, oracle_fwd, run_fwd

pytestmark = pytest.mark.gpu


def test_tiny_causal_gqa_fp32():
    w = gqa_inputs.tiny_causal_gqa_fp32()
    o, l = run_fwd(w)
    ro, rl = oracle_fwd(w)
    compare(o, l, ro, rl, torch.float32, "tiny fp32")


def test_bert_base_encoder_full():
    w = gqa_inputs.bert_base_encoder()
    o, l = run_fwd(w)
    ro, rl = pool.attention_pooled(w.q, w.k, w.v, w.scale, w.causal)
    do, dl = compare(o, l, ro, rl, torch.bfloat16, "bert encoder")
    print(f"bert encoder max|dO|={do:.3e} max|dLSE|={dl:.3e}")


def test_llama_prefill_every_row():
    """All 8192 positions x 32 heads of the causal prefill: 256 key tiles for
    the last row tiles, the lazy reference max over the whole length, every
    ring-slot reuse and the heaviest-first tile order."""
    w = gqa_inputs.llama31_8b_prefill()
    o, l = run_fwd(w)
    st = {}
    ro, rl = pool.attention_pooled(w.q, w.k, w.v, w.scale, True, stats=st)
    do, dl = compare(o, l, ro, rl, torch.bfloat16, "llama prefill")
    print(f"llama prefill every row max|dO|={do:.3e} max|dLSE|={dl:.3e} oracle {st}")


@pytest.mark.parametrize("ns", [1, 2, 4, 8])
def test_llama_decode_full(ns):
    w = gqa_inputs.llama31_8b_decode()
    o, l = ga.decode(w.q.cuda(), w.k.cuda(), w.v.cuda(), scale=w.scale, num_splits=ns)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(w.q, w.k, w.v, w.scale)
    do, dl = compare(o.cpu(), l.cpu(), ro, rl, torch.bfloat16, f"decode ns={ns}")
    print(f"decode ns={ns} max|dO|={do:.3e} max|dLSE|={dl:.3e}")


@pytest.fixture(scope="module")
def varlen_packed():
    w = gqa_inputs.varlen_packed_causal_48_12()
    o, l = run_fwd(w)
    return w, o, l


@pytest.mark.parametrize("part", range(4))
def test_varlen_packed_every_row(varlen_packed, part):
    """Every row and head of sequences part, part + 4, ... of the packed
    causal 48/12 batch (32 sequences of 128-4096 tokens; the four parts
    together cover all 3.7 M outputs)."""
    w, o, l = varlen_packed
    cu = w.cu_seqlens_q.tolist()
    seqs = list(range(part, len(cu) - 1, 4))
    st = {}
    ro, rl = pool.attention_pooled(w.q, w.k, w.v, w.scale, True, cu, cu, seqs=seqs, stats=st)
    idx = torch.cat([torch.arange(cu[b], cu[b + 1]) for b in seqs])
    do, dl = compare(o[idx], l[idx], ro[idx.numpy()], rl[idx.numpy()], torch.bfloat16,
                     f"varlen part {part}")
    print(f"varlen part {part}: {len(idx)} tokens max|dO|={do:.3e} max|dLSE|={dl:.3e} "
          f"oracle {st}")
