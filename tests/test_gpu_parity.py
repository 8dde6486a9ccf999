"""GPU parity: the HIP path against the fp64 oracle on seeded inputs.

Shapes span several row tiles (128 packed rows for bf16, 32 for fp32) and key
tiles (64 keys) with ragged tails, both head dims, MHA / GQA / MQA head
ratios (including a group size that is not a power of two), causal and not,
fixed and variable length, plus the degenerate cases: a single key, a single
query, causal rows with no visible key, and empty sequences.
"""
import numpy as np
import pytest
import torch

import gqa_attention_amd as ga
import gqa_inputs
import oracle

from parity_util import TOL, compare, oracle_fwd, run_fwd

pytestmark = pytest.mark.gpu

DTYPES = [torch.bfloat16, torch.float32]
DT_ID = {torch.bfloat16: "bf16", torch.float32: "fp32"}

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
    (1, 32, 1, 100, 100, True),    # MQA prefill: a row tile spans 4 (d 64) or 8 positions
    (1, 32, 1, 77, 140, False),
    (1, 16, 2, 1000, 1333, True),  # ragged tails on both axes, Lq < Lk
]


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DT_ID[d])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", FIXED, ids=lambda s: "B{}_Hq{}_Hkv{}_Sq{}_Sk{}_{}".format(
    *s[:5], "causal" if s[5] else "full"))
def test_fixed(shape, d, dtype):
    B, hq, hkv, sq, sk, causal = shape
    w = gqa_inputs.fixed(B, hq, hkv, sq, sk, d, seed=1000 + sq * 7 + sk, dtype=dtype,
                         causal=causal)
    o, l = run_fwd(w)
    ro, rl = oracle_fwd(w)
    compare(o, l, ro, rl, dtype, f"fixed {shape} d={d}")


def _scaled_keys(w, profile):
    """The same workload with each key row scaled by profile[j] (then rounded
    to the input dtype again), so that score magnitudes change along the keys."""
    f = torch.tensor(profile, dtype=torch.float32).view(1, -1, 1, 1)
    w.k = (w.k.float() * f).to(w.k.dtype)
    return w


KEY_PROFILES = {
    # later tiles reach scores tens of log2 units above every score of tile 0,
    # so the reference max must move many times
    "growing": lambda sk: [0.1 + 6.0 * j / sk for j in range(sk)],
    # the first tile holds the largest scores; later tiles underflow
    "shrinking": lambda sk: [6.0 - 5.9 * j / sk for j in range(sk)],
    # one key per 97 has scores 12x larger than the rest (spikes in any tile)
    "spikes": lambda sk: [12.0 if j % 97 == 41 else 1.0 for j in range(sk)],
}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("profile", sorted(KEY_PROFILES))
def test_score_range_along_keys(profile, causal, d):
    """Scores whose range moves along the key axis (bf16): the running
    reference of the streaming softmax is raised, or never raised, many times
    over a row, and the result still matches the oracle. (fp32 mode is left
    out: scores here reach about 50 in magnitude, and rounding s to fp32
    alone moves p by up to 50 x 2^-24 relative, above its 1e-5 bound.)"""
    dtype = torch.bfloat16
    w = gqa_inputs.fixed(2, 8, 2, 300, 700, d, seed=5000 + d + 7 * causal, dtype=dtype,
                         causal=causal)
    w = _scaled_keys(w, KEY_PROFILES[profile](700))
    o, l = run_fwd(w)
    ro, rl = oracle_fwd(w)
    compare(o, l, ro, rl, dtype, f"{profile} causal={causal} d={d}")


VARLEN = [
    # lengths_q, lengths_k, Hq, Hkv, causal
    ([0, 1, 63, 64, 65, 200], [0, 1, 63, 64, 65, 200], 8, 2, True),
    ([5, 130, 0, 17], [9, 100, 3, 17], 4, 4, False),
    ([40, 130, 1], [20, 300, 7], 6, 2, True),
    ([300], [300], 4, 1, True),
]


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DT_ID[d])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", VARLEN, ids=lambda c: f"n{len(c[0])}_Hq{c[2]}_Hkv{c[3]}_{c[4]}")
def test_varlen(case, d, dtype):
    lq, lk, hq, hkv, causal = case
    w = gqa_inputs.varlen(lq, lk, hq, hkv, d, seed=2000 + sum(lq), dtype=dtype, causal=causal)
    o, l = run_fwd(w)
    ro, rl = oracle_fwd(w)
    compare(o, l, ro, rl, dtype, f"varlen {case} d={d}")


DECODE = [
    # B, Hq, Hkv, Sk
    (3, 8, 2, 300),
    (2, 32, 8, 1000),
    (2, 32, 1, 129),   # MQA: 32 heads per K/V head (two 16-head slices)
    (2, 12, 4, 77),    # G = 3
    (1, 4, 4, 1),      # MHA, one cached key
]


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DT_ID[d])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("ns", [1, 2, 4, 8])
@pytest.mark.parametrize("shape", DECODE, ids=lambda s: "B{}_Hq{}_Hkv{}_Sk{}".format(*s))
def test_decode(shape, ns, d, dtype):
    B, hq, hkv, sk = shape
    w = gqa_inputs.decode(B, hq, hkv, sk, d, seed=3000 + sk, dtype=dtype)
    o, l = ga.decode(w.q.cuda(), w.k.cuda(), w.v.cuda(), scale=w.scale, num_splits=ns)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(w.q, w.k, w.v, w.scale)
    compare(o.cpu(), l.cpu(), ro, rl, dtype, f"decode {shape} ns={ns} d={d}")


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DT_ID[d])
def test_decode_partials_match_oracle_per_split(dtype):
    """The workspace holds each split's normalised output and LSE."""
    B, hq, hkv, sk, d, ns = 2, 8, 2, 300, 128, 4
    w = gqa_inputs.decode(B, hq, hkv, sk, d, seed=77, dtype=dtype)
    nbytes = ga.decode_workspace_bytes(B, hq, d, ns)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ga.decode(w.q.cuda(), w.k.cuda(), w.v.cuda(), scale=w.scale, num_splits=ns, workspace=ws)
    torch.cuda.synchronize()
    rows = B * hq
    o_bytes = ((ns * rows * d * 4 + 255) // 256) * 256
    wso = ws[:ns * rows * d * 4].view(torch.float32).view(ns, B, hq, d).cpu()
    wsl = ws[o_bytes:o_bytes + ns * rows * 4].view(torch.float32).view(ns, B, hq).cpu()
    po, pl = oracle.decode_partials(w.q, w.k, w.v, w.scale, ns, align=64)
    tol_o, tol_l = (2e-2, 1e-3) if dtype == torch.bfloat16 else (1e-5, 1e-5)
    for s in range(ns):
        compare(wso[s], wsl[s], po[s], pl[s], torch.float32 if dtype == torch.float32 else dtype,
                f"split {s}")


def test_decode_workspace_is_reusable_across_shapes():
    """One workspace, left as each call leaves it, serves later calls of
    other shapes and split counts."""
    ws = torch.empty(ga.decode_workspace_bytes(32, 32, 128, 8), dtype=torch.uint8, device="cuda")
    cases = [(32, 32, 8, 700, 128, 8), (5, 8, 2, 333, 64, 4), (32, 32, 8, 700, 128, 2),
             (3, 48, 12, 64, 128, 8), (32, 32, 8, 700, 128, 8)]
    for i, (B, hq, hkv, sk, d, ns) in enumerate(cases):
        w = gqa_inputs.decode(B, hq, hkv, sk, d, seed=78 + i)
        o, l = ga.decode(w.q.cuda(), w.k.cuda(), w.v.cuda(), scale=w.scale, num_splits=ns,
                         workspace=ws)
        torch.cuda.synchronize()
        ro, rl = oracle.decode(w.q, w.k, w.v, w.scale)
        compare(o.cpu(), l.cpu(), ro, rl, torch.bfloat16, f"decode reuse {i}")


# ---------------------------------------------------------------------------
# Invariants that hold bit for bit on the GPU.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [True, False])
def test_gqa_equals_expanded_mha_bitwise(causal):
    """Glossary snippet: GQA equals MHA on repeat-interleaved K/V. Each row's
    arithmetic is identical in both runs, so the results match bit for bit."""
    w = gqa_inputs.fixed(2, 8, 2, 300, 300, 128, seed=5, causal=causal)
    o1, l1 = run_fwd(w)
    wx = gqa_inputs.Workload("mha", w.q, w.k.repeat_interleave(4, dim=2).contiguous(),
                             w.v.repeat_interleave(4, dim=2).contiguous(), causal, w.scale)
    o2, l2 = run_fwd(wx)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_varlen_equals_per_sequence_bitwise():
    lens = [100, 1, 257, 64]
    w = gqa_inputs.varlen(lens, lens, 8, 2, 128, seed=6, causal=True)
    o, l = run_fwd(w)
    cu = w.cu_seqlens_q.tolist()
    for b in range(len(lens)):
        wb = gqa_inputs.Workload("seq", w.q[None, cu[b]:cu[b + 1]].contiguous(),
                                 w.k[None, cu[b]:cu[b + 1]].contiguous(),
                                 w.v[None, cu[b]:cu[b + 1]].contiguous(), True, w.scale)
        ob, lb = run_fwd(wb)
        assert torch.equal(o[cu[b]:cu[b + 1]], ob[0])
        assert torch.equal(l[cu[b]:cu[b + 1]], lb[0].T)


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DT_ID[d])
def test_causal_row0_is_v0(dtype):
    """Row 0 of a causal Lq = Lk call sees only key 0: O = V[0] exactly."""
    w = gqa_inputs.fixed(2, 8, 2, 100, 100, 128, seed=8, dtype=dtype, causal=True)
    o, l = run_fwd(w)
    for h in range(8):
        assert torch.equal(o[:, 0, h], w.v[:, 0, h // 4])
    q, k = w.q.double(), w.k.double()
    want = torch.stack([(q[:, 0, h] * k[:, 0, h // 4]).sum(-1) for h in range(8)], 1) * float(
        np.float32(w.scale))
    assert torch.allclose(l[:, :, 0].double(), want, atol=TOL[dtype][1], rtol=0)


def test_constant_v_gives_constant_output():
    w = gqa_inputs.fixed(1, 8, 2, 150, 150, 64, seed=9, causal=True)
    w.v = torch.full_like(w.v, 0.8125)  # exactly representable in bf16
    o, _ = run_fwd(w)
    assert torch.all(o == torch.tensor(0.8125, dtype=torch.bfloat16))


def test_deterministic():
    w = gqa_inputs.fixed(1, 32, 8, 700, 700, 128, seed=10, causal=True)
    a = run_fwd(w)
    b = run_fwd(w)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    d = gqa_inputs.decode(4, 32, 8, 999, 128, seed=11)
    r1 = ga.decode(d.q.cuda(), d.k.cuda(), d.v.cuda(), num_splits=4)
    r2 = ga.decode(d.q.cuda(), d.k.cuda(), d.v.cuda(), num_splits=4)
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


def test_num_splits_agree():
    d = gqa_inputs.decode(4, 32, 8, 2000, 128, seed=12)
    outs = [ga.decode(d.q.cuda(), d.k.cuda(), d.v.cuda(), num_splits=ns) for ns in (1, 2, 4, 8)]
    for o, l in outs[1:]:
        assert (o.float() - outs[0][0].float()).abs().max().item() <= 2e-2
        assert (l - outs[0][1]).abs().max().item() <= 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_many_sequences(causal):
    """More sequences than the longest-first ranking covers (70 > 64), and a
    ranked batch of 64 with equal lengths among them (ties by index)."""
    g = torch.Generator().manual_seed(31)
    for n in (70, 64):
        lens = torch.randint(0, 90, (n,), generator=g).tolist()
        lens[5] = lens[9] = lens[40] = 77
        w = gqa_inputs.varlen(lens, lens, 8, 2, 64, seed=32 + n, causal=causal)
        o, l = run_fwd(w)
        compare(o, l, *oracle_fwd(w), torch.bfloat16, f"varlen {n} sequences")


def test_varlen_beyond_the_dense_tile_lists():
    """1040 head groups (520 sequences x 2 K/V heads): more than the LDS list of
    live tiles holds, so every head group keeps its max-length row-tile count
    and the empty tiles end at once; lengths 0 .. 40 with many empty ones."""
    g = torch.Generator().manual_seed(41)
    lens = torch.randint(0, 41, (520,), generator=g)
    lens[::7] = 0
    lens = lens.tolist()
    for causal in (True, False):
        w = gqa_inputs.varlen(lens, lens, 4, 2, 64, seed=42, causal=causal)
        o, l = run_fwd(w)
        compare(o, l, *oracle_fwd(w), torch.bfloat16, f"varlen 1040 head groups causal={causal}")


def test_varlen_calls_reuse_scheduling_slots():
    """Seventy variable-length calls in a row (more than the 64 counter slots
    they take in turn), alternating two shapes: every call of a shape returns
    the same bits, and the first of each matches the oracle."""
    a = gqa_inputs.varlen([300, 0, 45, 1000], [300, 0, 45, 1000], 32, 8, 128, seed=43, causal=True)
    b = gqa_inputs.varlen([7, 513], [900, 513], 8, 8, 64, seed=44, causal=False)
    firsts = {}
    for i in range(70):
        w = a if i % 2 == 0 else b
        o, l = run_fwd(w)
        if i < 2:
            firsts[i] = (o, l)
            compare(o, l, *oracle_fwd(w), torch.bfloat16, f"slot reuse {i}")
        else:
            assert torch.equal(o, firsts[i % 2][0]) and torch.equal(l, firsts[i % 2][1]), i


def test_empty_varlen_batch():
    w = gqa_inputs.varlen([0, 0], [0, 5], 4, 2, 64, seed=13)
    o, l = ga.fwd(w.q.cuda(), w.k.cuda(), w.v.cuda(), cu_seqlens_q=w.cu_seqlens_q.cuda(),
                  cu_seqlens_k=w.cu_seqlens_k.cuda(), max_seqlen_q=0, max_seqlen_k=5)
    assert o.numel() == 0 and l.numel() == 0
