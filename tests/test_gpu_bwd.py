"""GPU parity of the attention backward (``gqa_attn_bwd``) against the fp64
gradient oracle ``oracle.backward.attention_grad`` on seeded inputs.

The forward outputs the backward consumes (O and LSE) come from the HIP
forward; the oracle computes the gradients from q, k, v and dO alone. Shapes
span several 32-row and 128-key blocks with ragged tails, both head dims,
MHA / GQA / MQA ratios (including a group of 3), causal and not with Lq != Lk
(rows that see no key, keys no row sees), fixed and variable length with
empty sequences.

Tolerance: every product runs on bf16 operands with fp32 accumulation; P and
dS are rounded to bf16 (relative error <= 2^-9 each) before the dV, dK and dQ
products and the results are rounded to bf16 again, so each gradient element
carries a few units of 2^-9 relative to the magnitude of the terms it sums.
The test bounds max |g - g_ref| by BWD_RTOL (10 units of 2^-9) times
max |g_ref| of that tensor, plus BWD_ATOL for references that vanish
identically (a single key: dP = D exactly), where the kernel returns the
fp32 residue of summing the same terms in two orders.
"""
import numpy as np
import pytest
import torch

import gqa_attention_amd as ga
import gqa_inputs
from oracle import backward as ob

pytestmark = pytest.mark.gpu

BWD_RTOL = 2e-2
BWD_ATOL = 1e-4


def _dout(w, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(w.q.shape, generator=g).to(torch.bfloat16)


def run_bwd(w, do):
    dev = "cuda"
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    kw = dict(causal=w.causal, scale=w.scale)
    if w.varlen:
        kw.update(cu_seqlens_q=w.cu_seqlens_q.to(dev), cu_seqlens_k=w.cu_seqlens_k.to(dev),
                  max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k)
    o, lse = ga.fwd(q, k, v, **kw)
    dq, dk, dv = ga.bwd(q, k, v, o, lse, do.to(dev), **kw)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def oracle_bwd(w, do):
    cq = w.cu_seqlens_q.tolist() if w.varlen else None
    ck = w.cu_seqlens_k.tolist() if w.varlen else None
    return ob.attention_grad(w.q, w.k, w.v, do, w.scale, w.causal, cq, ck)


def compare_grads(got, ref, what):
    errs = []
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.to(torch.float64).numpy()
        assert g.shape == r.shape, (what, name, g.shape, r.shape)
        assert not np.isnan(g).any(), f"{what}: NaN in {name}"
        scale = float(np.max(np.abs(r))) if r.size else 0.0
        err = float(np.max(np.abs(g - r))) if r.size else 0.0
        errs.append((name, err, scale))
        assert err <= BWD_RTOL * scale + BWD_ATOL, \
            f"{what}: max|d{name}| = {err:.3e} > {BWD_RTOL} x {scale:.3e} + {BWD_ATOL}"
    return errs


FIXED = [
    # B, Hq, Hkv, Sq, Sk, causal
    (2, 8, 2, 200, 200, True),
    (2, 8, 2, 200, 200, False),
    (1, 4, 1, 130, 77, False),
    (1, 4, 1, 77, 130, True),     # Lq < Lk: bottom-right causal
    (1, 6, 2, 65, 300, False),    # G = 3
    (1, 6, 2, 300, 65, True),     # Lq > Lk: early rows see no key
    (2, 3, 3, 257, 129, False),   # MHA
    (1, 2, 2, 1, 1, True),
    (1, 8, 1, 1, 333, False),     # MQA, single query
    (1, 16, 2, 33, 1, False),     # single key
    (1, 32, 8, 512, 512, True),
    # fewer than 256 (sequence, K/V head, key block) units: the rows that see
    # each key block are split into chunks whose fp32 partial dK/dV are summed
    # afterwards (31, 28, 10 and 14 chunks here; causal key blocks use fewer)
    (1, 16, 1, 2100, 2100, True),
    (1, 16, 1, 1800, 2000, True),   # Lq < Lk
    (1, 16, 2, 1300, 1000, True),   # G = 8, Lq > Lk: early rows see no key
    (1, 16, 1, 900, 700, False),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", FIXED, ids=lambda s: "B{}_Hq{}_Hkv{}_Sq{}_Sk{}_{}".format(
    *s[:5], "causal" if s[5] else "full"))
def test_bwd_fixed(shape, d):
    B, hq, hkv, sq, sk, causal = shape
    w = gqa_inputs.fixed(B, hq, hkv, sq, sk, d, seed=3000 + sq * 7 + sk, causal=causal)
    do = _dout(w, 77)
    errs = compare_grads(run_bwd(w, do), oracle_bwd(w, do), f"bwd {shape} d={d}")
    print(shape, d, errs)


VARLEN = [
    # lengths_q, lengths_k, Hq, Hkv, causal
    ([0, 1, 63, 64, 65, 200], [0, 1, 63, 64, 65, 200], 8, 2, True),
    ([5, 130, 0, 17], [9, 100, 3, 17], 4, 4, False),
    ([40, 130, 1], [20, 300, 7], 6, 2, True),
    ([3, 0], [0, 4], 4, 2, False),   # a sequence with no keys and one with no queries
    ([700, 30, 1100, 0], [650, 30, 1100, 5], 16, 1, True),  # chunked and unchunked key blocks
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", VARLEN, ids=lambda c: f"n{len(c[0])}_Hq{c[2]}_Hkv{c[3]}_"
                         f"{'causal' if c[4] else 'full'}")
def test_bwd_varlen(case, d):
    lq, lk, hq, hkv, causal = case
    w = gqa_inputs.varlen(lq, lk, hq, hkv, d, seed=4000 + sum(lq), causal=causal)
    do = _dout(w, 78)
    errs = compare_grads(run_bwd(w, do), oracle_bwd(w, do), f"bwd varlen {case} d={d}")
    print(case, d, errs)


PAIRED = [
    # B, Hq, Hkv, S, d: causal, B * Hkv * ceil(S / 128) >= 256 key blocks, so
    # the rows are not chunked and a dK/dV workgroup takes key block i and
    # then n_kb - 1 - i
    (8, 8, 8, 512, 64),     # 4 key blocks per sequence: pairs (0, 3), (1, 2)
    (8, 8, 8, 640, 64),     # 5: the middle block runs alone
    (4, 16, 8, 1024, 128),  # GQA, 8 key blocks
    # more than 256 workgroups (one per CU on MI355X): the two-workgroups-per-CU
    # variant of the key-block pass; the smaller grids above run the variant
    # built for one workgroup per CU
    (16, 8, 8, 640, 128),   # 16 * 8 * 3 pairs
]

BIG_GRID_FULL = [
    # B, Hq, Hkv, S, d: non-causal, more than 256 key-block workgroups
    (6, 8, 8, 700, 128),    # 6 * 8 * 6 key blocks, ragged last block
    (6, 12, 4, 1100, 64),   # G = 3, 6 * 4 * 9
]


@pytest.mark.parametrize("shape", PAIRED, ids=lambda s: "B{}_Hq{}_Hkv{}_S{}_d{}".format(*s))
def test_bwd_paired_key_blocks(shape):
    B, hq, hkv, S, d = shape
    w = gqa_inputs.fixed(B, hq, hkv, S, S, d, seed=7000 + S + d, causal=True)
    do = _dout(w, 83)
    errs = compare_grads(run_bwd(w, do), oracle_bwd(w, do), f"bwd paired {shape}")
    print(shape, errs)


@pytest.mark.parametrize("shape", BIG_GRID_FULL, ids=lambda s: "B{}_Hq{}_Hkv{}_S{}_d{}".format(*s))
def test_bwd_big_grid_full(shape):
    B, hq, hkv, S, d = shape
    w = gqa_inputs.fixed(B, hq, hkv, S, S, d, seed=7200 + S + d, causal=False)
    do = _dout(w, 85)
    errs = compare_grads(run_bwd(w, do), oracle_bwd(w, do), f"bwd big grid {shape}")
    print(shape, errs)


def test_bwd_paired_key_blocks_varlen():
    """Paired key blocks over sequences of different lengths: each sequence
    pairs its own key blocks (n_kb of the longest sizes the grid)."""
    lens = [700, 130, 1, 640, 257, 0, 512, 385, 128, 600, 90, 700, 33, 256, 511, 640]
    w = gqa_inputs.varlen(lens, lens, 8, 8, 64, seed=7100, causal=True)
    do = _dout(w, 84)
    errs = compare_grads(run_bwd(w, do), oracle_bwd(w, do), "bwd paired varlen")
    print(errs)


def test_bwd_rows_without_keys_get_zero_dq():
    """Causal with Lq > Lk: the first Lq - Lk rows see no key; their dq is
    exactly zero and the other rows' is not."""
    w = gqa_inputs.fixed(1, 4, 2, 150, 40, 64, seed=9, causal=True)
    dq, _, _ = run_bwd(w, _dout(w, 79))
    assert torch.all(dq[0, :110] == 0)
    assert torch.any(dq[0, 110:] != 0)


def test_bwd_deterministic():
    w = gqa_inputs.fixed(1, 8, 2, 300, 300, 128, seed=10, causal=True)
    do = _dout(w, 80)
    a = run_bwd(w, do)
    b = run_bwd(w, do)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("which", ["bert_base_encoder", "causal_gqa_2048"])
def test_bwd_full_size_sampled(which):
    """The BERT-base encoder workload at full size (B 64, S 512, 12 heads,
    d 64) and a 2048-token causal GQA shape with the Llama 3.1 8B heads
    (32 / 8, d 128): gradients at sampled rows and keys against the sampled
    fp64 oracle (every row's LSE and D from the full fp64 forward)."""
    if which == "bert_base_encoder":
        w = gqa_inputs.bert_base_encoder()
    else:
        w = gqa_inputs.fixed(1, 32, 8, 2048, 2048, 128, seed=33, causal=True)
    do = _dout(w, 81)
    dq, dk, dv = run_bwd(w, do)
    B, S, Hq, _ = w.q.shape
    Hkv = w.k.shape[2]
    g = torch.Generator().manual_seed(82)
    pick = lambda n, hi: torch.randint(0, hi, (n,), generator=g).tolist()
    rows = list(zip(pick(24, B), pick(24, S), pick(24, Hq))) + [(0, 0, 0), (B - 1, S - 1, Hq - 1)]
    keys = list(zip(pick(24, B), pick(24, S), pick(24, Hkv))) + [(0, 0, 0), (B - 1, S - 1, Hkv - 1)]
    rq, rk, rv = ob.attention_grad_sampled(w.q, w.k, w.v, do, w.scale, w.causal, rows, keys)
    got = (torch.stack([dq[b, i, h] for b, i, h in rows]),
           torch.stack([dk[b, j, h] for b, j, h in keys]),
           torch.stack([dv[b, j, h] for b, j, h in keys]))
    # the scale of each tensor is the sampled reference's maximum
    compare_grads(got, (rq, rk, rv), f"bwd full-size {which}")
