"""GPU parity of the forward over fp8 e4m3 inputs (``gqa_attn_fwd_fp8``)
against the fp64 oracle ``oracle.fp8_forward`` on seeded inputs.

The kernel computes the attention of the dequantised inputs: scores from the
fp8 matrix cores, probabilities and the widened V in bf16, O rounded to
bf16. Its rounding is that of the bf16 forward, so the bf16 bounds apply
(max |dO| <= 2e-2, max |dLSE| <= 1e-3) at the ordinary dequantisation scales
of these cases. The fp8 matrix core does not add its 64 products in full
precision (``tests/fp8_mfma_model.py``, a model of its sums checked against
the hardware); at large q_scale k_scale the resulting score error grows past
1e-3, and those cases are bounded per row by 1e-3 plus the model's own
distance from the oracle (``model_bound``), with the model required to
reproduce the kernel's LSE within 1e-3. Shapes span several 32-key tiles
and 128 / 256-row tiles with ragged tails, both head dims, MHA / GQA (G = 3,
4) / MQA ratios, causal and not with Lq != Lk, fixed and variable length with
empty sequences, and the two full-size fp8 workloads at every row.
"""
import numpy as np
import pytest
import torch

import gqa_attention_amd as ga
import gqa_inputs as gi
from fp8_mfma_model import fp8_scores
from oracle import fp8_forward as of8
from oracle import pool
from parity_util import TOL

pytestmark = pytest.mark.gpu


def compare(o_gpu, l_gpu, o_ref, l_ref, dtype, what="", lse_bound=None):
    """Element-wise check against the oracle; returns (max|dO|, max|dLSE|).
    lse_bound: per-row LSE bounds (default: the dtype's flat bound)."""
    tol_o, tol_l = TOL[dtype]
    o = o_gpu.to(torch.float64).numpy()
    l = l_gpu.to(torch.float64).numpy()
    assert o.shape == o_ref.shape and l.shape == l_ref.shape, what
    assert not np.isnan(o).any() and not np.isnan(l).any(), f"{what}: NaN in GPU output"
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l), fin), f"{what}: -inf pattern of LSE differs"
    assert np.all(l[~fin] == l_ref[~fin]), f"{what}: LSE of empty rows"
    do = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    assert do <= tol_o, f"{what}: max|dO| = {do:.3e} > {tol_o}"
    if fin.any():
        err = np.abs(l[fin] - l_ref[fin])
        bound = tol_l if lse_bound is None else lse_bound[fin]
        assert np.all(err <= bound), f"{what}: max|dLSE| = {err.max():.3e}, worst excess " \
            f"{np.max(err - bound):.3e}"
        return do, float(err.max())
    return do, 0.0


def model_lse(w):
    """LSE [B, Hq, Sq] of the fixed-length fp8 workload w with the scores the
    fp8 matrix core forms (tests/fp8_mfma_model.py) instead of exact ones:
    log sum_j exp(S_model[i, j] scale q_scale k_scale) over visible keys."""
    qs, ks, _ = w.fp8_scales
    q = w.q.view(torch.uint8).numpy()
    k = w.k.view(torch.uint8).numpy()
    B, Sq, Hq, d = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    c = float(np.float32(w.scale)) * qs * ks
    out = np.full((B, Hq, Sq), -np.inf)
    vis = np.ones((Sq, Sk), dtype=bool)
    if w.causal:
        vis = np.arange(Sk)[None, :] <= np.arange(Sq)[:, None] + (Sk - Sq)
    for b in range(B):
        for h in range(Hq):
            s = fp8_scores(q[b, :, h, :], k[b, :, h // (Hq // Hkv), :]).astype(np.float64) * c
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1)
            live = np.isfinite(m)
            out[b, h, live] = m[live] + np.log(np.exp(s[live] - m[live, None]).sum(axis=1))
    return out


def model_bound(w, l_gpu, l_ref, what):
    """Per-row LSE bound 1e-3 + |LSE_model - LSE_oracle|, after checking that
    the model reproduces the kernel's LSE within 1e-3."""
    lm = model_lse(w)
    fin = np.isfinite(l_ref)
    gap = np.abs(l_gpu.double().numpy()[fin] - lm[fin])
    assert gap.max() <= 1e-3, f"{what}: the matrix-core model misses the kernel by {gap.max():.3e}"
    bound = np.full(l_ref.shape, 1e-3)
    bound[fin] += np.abs(lm[fin] - l_ref[fin])
    return bound


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
def test_fp8_full_size_every_row(name):
    """The full-size fp8 workloads, every row and head, against the oracle
    on the dequantised inputs (run as a process pool)."""
    w = gi.NAMED[name]()
    o, l = run_fp8(w)
    qv, kv, vv = of8.dequantised(w.q, w.k, w.v, *w.fp8_scales)
    ro, rl = pool.attention_pooled(qv, kv, vv, w.scale, w.causal)
    print(name, compare(o, l, ro, rl, torch.bfloat16, f"fp8 full-size {name}"))


@pytest.mark.parametrize("qs,ks", [(8.0, 8.0), (1.0 / 64, 1.0 / 64)])
def test_fp8_extreme_scales(qs, ks):
    """q_scale x k_scale of 64 (a sharply peaked softmax whose reference max
    moves often; scores up to ~340, where the matrix core's truncated sums
    move the LSE by up to ~1e-2) and of 1/4096 (a nearly uniform one). LSE
    bound per row from the matrix-core model."""
    w = gi.fixed_fp8(2, 8, 2, 200, 230, 128, seed=50, causal=True, q_scale=qs, k_scale=ks,
                     v_scale=0.5)
    o, l = run_fp8(w)
    ro, rl = oracle_fp8(w)
    bound = model_bound(w, l, rl, f"fp8 scales {qs} {ks}")
    print(qs, ks, "largest model-derived LSE bound", float(bound.max()),
          compare(o, l, ro, rl, torch.bfloat16, f"fp8 scales {qs} {ks}", lse_bound=bound))


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_every_v_code_widens_exactly(d):
    """All keys equal (code 0x38 = 1.0): every row attends uniformly with
    p = 1 exactly, so O is the mean of the visible values, formed in fp32 and
    rounded once to bf16: |dO| <= 2^-8 |O| (half a bf16 unit of O) + 1e-6.
    V cycles through all 254 finite e4m3 codes (subnormals and +-448
    included), so a wrong widening of any code shows."""
    S, hq, hkv = 254, 4, 2
    g = torch.Generator().manual_seed(51)
    q = torch.randn(1, S, hq, d, generator=g).to(torch.float8_e4m3fn)
    k = torch.full((1, S, hkv, d), 0x38, dtype=torch.uint8).view(torch.float8_e4m3fn)
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    codes = torch.tensor(finite, dtype=torch.uint8)
    vc = torch.empty(1, S, hkv, d, dtype=torch.uint8)
    for j in range(S):
        vc[0, j] = codes[(j + torch.arange(hkv * d)) % len(finite)].view(hkv, d)
    v = vc.view(torch.float8_e4m3fn)
    w = gi.Workload("every_v_code", q, k, v, True, d ** -0.5, fp8_scales=(0.5, 0.25, 1.0 / 64))
    o, l = run_fp8(w)
    ro, rl = oracle_fp8(w)
    err = np.abs(o.double().numpy() - ro)
    assert np.all(err <= 2.0 ** -8 * np.abs(ro) + 1e-6), float((err - 2.0 ** -8 * np.abs(ro)).max())
    bound = model_bound(w, l, rl, f"every v code d={d}")
    assert np.all(np.abs(l.double().numpy() - rl) <= bound)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_gqa_equals_expanded_mha_bitwise(causal, d):
    """GQA equals MHA on repeat-interleaved K/V (glossary snippet), bit for
    bit: each row's arithmetic is the same in both runs."""
    w = gi.fixed_fp8(2, 8, 2, 300, 300, d, seed=52, causal=causal, q_scale=0.5, k_scale=0.25,
                     v_scale=0.5)
    o1, l1 = run_fp8(w)
    rep = lambda t: t.view(torch.uint8).repeat_interleave(4, dim=2).contiguous().view(
        torch.float8_e4m3fn)
    wx = gi.Workload("mha_fp8", w.q, rep(w.k), rep(w.v), causal, w.scale, fp8_scales=w.fp8_scales)
    o2, l2 = run_fp8(wx)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_varlen_equals_per_sequence_bitwise():
    lens = [100, 1, 257, 64]
    w = gi.varlen_fp8(lens, lens, 8, 2, 128, seed=53, causal=True, q_scale=0.5, k_scale=0.25,
                      v_scale=0.5)
    o, l = run_fp8(w)
    cu = w.cu_seqlens_q.tolist()
    for b in range(len(lens)):
        sl = lambda t: t[None, cu[b]:cu[b + 1]].contiguous()
        wb = gi.Workload("seq_fp8", sl(w.q), sl(w.k), sl(w.v), True, w.scale,
                         fp8_scales=w.fp8_scales)
        ob, lb = run_fp8(wb)
        assert torch.equal(o[cu[b]:cu[b + 1]], ob[0])
        assert torch.equal(l[cu[b]:cu[b + 1]], lb[0].T)
