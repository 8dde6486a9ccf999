"""GPU parity of the forward over fp8 e4m3 inputs (``gqa_attn_fwd_fp8``)
against the fp64 oracle ``oracle.fp8_forward`` on seeded inputs.

The kernel computes the attention of the dequantised inputs: scores from the
fp8 matrix cores (exact products of the codes, fp32 sums), probabilities and
the widened V in bf16, O rounded to bf16. Its rounding is that of the bf16
forward, so the bf16 bound applies (max |dO| <= 2e-2 with |v| <= v_scale x 6
and v_scale <= 1 here; max |dLSE| <= 1e-3). Shapes span several 32-key tiles
and 128 / 256-row tiles with ragged tails, both head dims, MHA / GQA (G = 3,
4) / MQA ratios, causal and not with Lq != Lk, fixed and variable length with
empty sequences, and the two full-size fp8 workloads at sampled rows.
"""
import numpy as np
import pytest
import torch

import gqa_attention_amd as ga
import gqa_inputs as gi
from oracle import fp8_forward as of8
from parity_util import compare

pytestmark = pytest.mark.gpu


def run_fp8(w):
    dev = "cuda"
    qs, ks, vs = w.fp8_scales
    kw = dict(causal=w.causal, scale=w.scale, q_scale=qs, k_scale=ks, v_scale=vs)
    if w.varlen:
        kw.update(cu_seqlens_q=w.cu_seqlens_q.to(dev), cu_seqlens_k=w.cu_seqlens_k.to(dev),
                  max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k)
    o, l = ga.fwd_fp8(w.q.to(dev), w.k.to(dev), w.v.to(dev), **kw)
    torch.cuda.synchronize()
    return o.cpu(), l.cpu()


def oracle_fp8(w):
    qs, ks, vs = w.fp8_scales
    cq = w.cu_seqlens_q.tolist() if w.varlen else None
    ck = w.cu_seqlens_k.tolist() if w.varlen else None
    return of8.attention_fp8(w.q, w.k, w.v, w.scale, w.causal, qs, ks, vs, cq, ck)


FIXED = [
    # B, Hq, Hkv, Sq, Sk, causal, (q_scale, k_scale, v_scale)
    (2, 8, 2, 300, 300, True, (0.5, 0.25, 0.5)),
    (2, 8, 2, 300, 300, False, (1.0, 1.0, 1.0)),
    (1, 4, 1, 130, 77, False, (0.25, 0.5, 1.0)),    # MQA
    (1, 4, 1, 77, 130, True, (0.5, 0.5, 0.5)),      # Lq < Lk: bottom-right causal
    (1, 6, 2, 65, 300, False, (1.0, 0.125, 0.25)),  # G = 3
    (1, 6, 2, 300, 65, True, (0.5, 0.25, 1.0)),     # Lq > Lk: early rows see no key
    (2, 3, 3, 257, 129, False, (0.5, 0.5, 0.5)),    # MHA
    (1, 2, 2, 1, 1, True, (1.0, 1.0, 1.0)),
    (1, 8, 1, 1, 333, False, (0.5, 0.25, 0.5)),     # a single query row
    (1, 16, 2, 33, 1, False, (0.5, 0.25, 0.5)),     # a single key
    (1, 32, 8, 700, 700, True, (0.5, 0.25, 0.5)),   # Llama heads, several 256-row tiles
    # head-group counts that are multiples of 16 (d = 64 pairs adjacent head
    # groups on one XCD)
    (2, 16, 16, 200, 200, False, (0.5, 0.25, 0.5)),
    (2, 32, 8, 150, 170, True, (0.5, 0.25, 0.5)),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", FIXED, ids=lambda s: "B{}_Hq{}_Hkv{}_Sq{}_Sk{}_{}".format(
    *s[:5], "causal" if s[5] else "full"))
def test_fp8_fixed(shape, d):
    B, hq, hkv, sq, sk, causal, (qs, ks, vs) = shape
    w = gi.fixed_fp8(B, hq, hkv, sq, sk, d, seed=5000 + sq * 7 + sk, causal=causal,
                     q_scale=qs, k_scale=ks, v_scale=vs)
    o, l = run_fp8(w)
    print(shape, d, compare(o, l, *oracle_fp8(w), torch.bfloat16, f"fp8 {shape} d={d}"))


VARLEN = [
    # lengths_q, lengths_k, Hq, Hkv, causal
    ([0, 1, 63, 64, 65, 200], [0, 1, 63, 64, 65, 200], 8, 2, True),
    ([5, 130, 0, 17], [9, 100, 3, 17], 4, 4, False),
    ([40, 300, 1], [20, 500, 7], 6, 2, True),
    ([3, 0], [0, 4], 4, 2, False),  # a sequence with no keys and one with no queries
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", VARLEN, ids=lambda c: f"n{len(c[0])}_Hq{c[2]}_Hkv{c[3]}_"
                         f"{'causal' if c[4] else 'full'}")
def test_fp8_varlen(case, d):
    lq, lk, hq, hkv, causal = case
    w = gi.varlen_fp8(lq, lk, hq, hkv, d, seed=6000 + sum(lq), causal=causal, q_scale=0.5,
                      k_scale=0.25, v_scale=0.5)
    o, l = run_fp8(w)
    print(case, d, compare(o, l, *oracle_fp8(w), torch.bfloat16, f"fp8 varlen {case} d={d}"))


def test_fp8_score_range_along_keys():
    """Scores that grow along the keys (the reference max moves up repeatedly)
    and a spike: K rows scaled by a ramp before the e4m3 rounding."""
    g = torch.Generator().manual_seed(47)
    B, S, hq, hkv, d = 1, 600, 8, 2, 128
    q = torch.randn(B, S, hq, d, generator=g)
    k = torch.randn(B, S, hkv, d, generator=g) * torch.linspace(0.2, 3.0, S)[None, :, None, None]
    k[0, 444] *= 4.0
    v = torch.randn(B, S, hkv, d, generator=g)
    w = gi.Workload("ramp_fp8", q.to(torch.float8_e4m3fn), k.to(torch.float8_e4m3fn),
                    v.to(torch.float8_e4m3fn), False, d ** -0.5, fp8_scales=(0.5, 0.5, 0.5))
    o, l = run_fp8(w)
    compare(o, l, *oracle_fp8(w), torch.bfloat16, "fp8 ramp")


def test_fp8_deterministic():
    w = gi.fixed_fp8(1, 8, 2, 300, 300, 128, seed=48, causal=True, q_scale=0.5, k_scale=0.5,
                     v_scale=0.5)
    a, b = run_fp8(w), run_fp8(w)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("name", ["llama31_8b_prefill_fp8", "bert_base_encoder_fp8"])
def test_fp8_full_size_sampled(name):
    """The full-size fp8 workloads: O and LSE at sampled rows (plus the first
    and last row) against the sampled oracle."""
    w = gi.NAMED[name]()
    o, l = run_fp8(w)
    B, S, Hq, _ = w.q.shape
    g = torch.Generator().manual_seed(49)
    pick = lambda n, hi: torch.randint(0, hi, (n,), generator=g).tolist()
    rows = list(zip(pick(40, B), pick(40, S), pick(40, Hq))) + [(0, 0, 0), (B - 1, S - 1, Hq - 1)]
    qs, ks, vs = w.fp8_scales
    ro, rl = of8.attention_rows_fp8(w.q, w.k, w.v, w.scale, w.causal, qs, ks, vs, rows)
    got_o = torch.stack([o[b, i, h] for b, i, h in rows])
    got_l = torch.tensor([float(l[b, h, i]) for b, i, h in rows])
    compare(got_o, got_l, ro, rl, torch.bfloat16, f"fp8 full-size {name}")
