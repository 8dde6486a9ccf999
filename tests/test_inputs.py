"""The seeded generators are deterministic; the tiny workload keeps the
glossary example's draws (checked against stored checksums)."""
import hashlib
import json
import os

import torch

import gqa_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_inputs.json")


def test_tiny_draws_match_stored_checksums():
    """tests/golden/tiny_inputs.json (written by make_tiny_inputs.py next to
    it) holds the SHA-256 of q, k, v in the head-major order they are drawn
    in (glossary page "Grouped Query Attention (GQA)", section "How GQA
    works": seed 0, q [1, 8, 16, 64] then k and v [1, 2, 16, 64]), and their
    first values. The workload stores them token-major, causal, scale 1/8."""
    ref = json.load(open(GOLDEN))
    w = gqa_inputs.tiny_causal_gqa_fp32()
    for name, t in (("q", w.q), ("k", w.k), ("v", w.v)):
        bhsd = t.transpose(1, 2).contiguous()
        assert t.dtype == torch.float32
        assert list(bhsd.shape) == ref[name]["shape_bhsd"]
        assert hashlib.sha256(bhsd.numpy().tobytes()).hexdigest() == ref[name]["sha256_fp32"]
        assert bhsd.flatten()[:4].tolist() == ref[name]["first4"]
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
