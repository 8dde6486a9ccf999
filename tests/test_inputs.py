"""The seeded generators are deterministic and reproduce the glossary snippet's draws."""
import torch

import gqa_inputs


def test_tiny_matches_snippet_draws():
    torch.manual_seed(0)
    q = torch.randn(1, 8, 16, 64)
    k = torch.randn(1, 2, 16, 64)
    v = torch.randn(1, 2, 16, 64)
    w = gqa_inputs.tiny_causal_gqa_fp32()
    assert torch.equal(w.q, q.transpose(1, 2))
    assert torch.equal(w.k, k.transpose(1, 2))
    assert torch.equal(w.v, v.transpose(1, 2))
    assert w.causal and abs(w.scale - 0.125) < 1e-12


def test_deterministic_and_shapes():
    a = gqa_inputs.fixed(2, 4, 2, 33, 17, 64, seed=9)
    b = gqa_inputs.fixed(2, 4, 2, 33, 17, 64, seed=9)
    assert torch.equal(a.q, b.q) and torch.equal(a.v, b.v)
    assert a.q.shape == (2, 33, 4, 64) and a.k.shape == (2, 17, 2, 64)
    assert a.q.dtype == torch.bfloat16
    w = gqa_inputs.varlen([3, 0, 5], [4, 1, 5], 4, 1, 128, seed=1, causal=True)
    assert w.cu_seqlens_q.tolist() == [0, 3, 3, 8] and w.cu_seqlens_k.tolist() == [0, 4, 5, 10]
    assert w.cu_seqlens_q.dtype == torch.int32 and w.max_seqlen_q == 5 and w.max_seqlen_k == 5
    d = gqa_inputs.decode(3, 8, 2, 40, 64, seed=2)
    assert d.q.shape == (3, 8, 64) and d.k.shape == (3, 40, 2, 64) and d.decode
