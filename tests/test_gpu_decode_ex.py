"""GPU parity of decode over a general K/V cache (``gqa_attn_decode_ex``)
against the fp64 oracle ``oracle.cache.decode_cache`` on seeded inputs.

Covers contiguous and paged caches (page sizes 1 to 256, a split spanning
more blocks than one staged window of the block table), per-sequence
lengths with empty and one-key caches and lengths around the 64-key split
granularity, ragged batches of up to 256 sequences (scheduled longest first)
and of more, sliding windows (one key, narrower and wider than the cache),
fp8 e4m3 storage with dequantisation scales, MHA / GQA / MQA head ratios
including groups of 16 and 24 query heads, and several split counts (also
over 1100 sequences, and repeated launches of interleaved shapes); plus
exact identities: the contiguous full-length call equals ``gqa_attn_decode``
bit for bit, a paged cache equals the same data stored contiguously, and
out-of-range lengths are clamped.
"""
import numpy as np
import pytest
import torch

import gqa_attention_amd as ga
import gqa_inputs as gi
from oracle import cache as oc

from parity_util import compare

pytestmark = pytest.mark.gpu


def to_dev(w):
    t = lambda x: None if x is None else x.cuda()
    return t(w.q), t(w.k_cache), t(w.v_cache), t(w.seqlens), t(w.block_table)


def run(w, num_splits=1, **over):
    q, k, v, sl, bt = to_dev(w)
    kw = dict(seqlens_k=sl, block_table=bt, window_left=w.window_left, k_scale=w.k_scale,
              v_scale=w.v_scale, scale=w.scale, num_splits=num_splits)
    kw.update(over)
    o, l = ga.decode_ex(q, k, v, **kw)
    torch.cuda.synchronize()
    return o.cpu(), l.cpu()


def reference(w):
    return oc.decode_cache(w.q, w.k_cache, w.v_cache, w.scale, seqlens=w.seqlens,
                           block_table=w.block_table, window_left=w.window_left, fp8=w.fp8,
                           k_scale=w.k_scale, v_scale=w.v_scale)


CASES = [
    # lengths, Hq, Hkv, d, block_size (0 = contiguous), window_left, fp8, num_splits
    ([0, 1, 63, 64, 65, 200, 1000], 32, 8, 128, 0, -1, False, 1),
    ([0, 1, 63, 64, 65, 200, 1000], 32, 8, 128, 0, -1, False, 3),
    ([513, 7, 2048], 8, 8, 64, 0, -1, False, 2),          # MHA
    ([300, 301], 24, 1, 64, 0, -1, False, 1),             # MQA, 24 heads: two query slices
    ([0, 1, 17, 100, 1000], 32, 8, 128, 16, -1, False, 1),
    ([0, 1, 17, 100, 1000], 32, 8, 128, 16, -1, False, 4),
    ([5000, 3], 8, 2, 128, 1, -1, False, 1),              # 5000 one-key pages in one split
    ([777, 64, 65], 16, 1, 64, 64, -1, False, 2),         # group of 16
    ([2000, 129], 48, 12, 128, 256, -1, False, 3),
    ([1, 50, 1000, 4097], 32, 8, 128, 16, 0, False, 1),   # window of one key
    ([1, 50, 1000, 4097], 32, 8, 128, 16, 63, False, 2),
    ([1, 50, 1000, 4097], 32, 8, 128, 0, 1000, False, 3),
    ([100, 100], 8, 2, 64, 0, 4095, False, 1),            # window wider than the cache
    ([0, 1, 63, 300, 1000], 32, 8, 128, 0, -1, True, 1),
    ([0, 1, 63, 300, 1000], 32, 8, 128, 16, -1, True, 3),
    ([129, 2000], 8, 2, 64, 32, 511, True, 2),
    ([333], 24, 3, 64, 8, -1, True, 1),                   # group of 8
    ([(37 * i) % 211 for i in range(300)], 8, 2, 64, 16, -1, False, 2),  # no longest-first
    ([(53 * i) % 997 for i in range(256)], 8, 2, 64, 0, -1, False, 3),   # longest-first, 256
]


def _id(c):
    lens, hq, hkv, d, bs, win, fp8, ns = c
    return (f"n{len(lens)}max{max(lens)}_h{hq}kv{hkv}_d{d}_"
            f"{'paged' + str(bs) if bs else 'contig'}_w{win}_{'fp8' if fp8 else 'bf16'}_ns{ns}")


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_decode_ex_matches_oracle(case):
    lens, hq, hkv, d, bs, win, fp8, ns = case
    seed = 5000 + 31 * CASES.index(case)
    w = gi.cache_decode(lens, hq, hkv, d, seed=seed, block_size=bs, window_left=win, fp8=fp8,
                        k_scale=0.25, v_scale=0.75)
    o, l = run(w, num_splits=ns)
    ro, rl = reference(w)
    compare(o, l, ro, rl, torch.bfloat16, _id(case))


def test_all_caches_empty():
    w = gi.cache_decode([0, 0, 0], 8, 2, 128, seed=7, block_size=16)
    for ns in (1, 4):
        o, l = run(w, num_splits=ns)
        assert torch.all(o == 0) and torch.all(torch.isneginf(l))


@pytest.mark.parametrize("ns", [1, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_contiguous_full_length_equals_decode_bitwise(d, ns):
    w = gi.cache_decode([700] * 3, 32, 8, d, seed=8, with_seqlens=False)
    q, k, v, _, _ = to_dev(w)
    o1, l1 = ga.decode(q, k, v, scale=w.scale, num_splits=ns)
    o2, l2 = ga.decode_ex(q, k, v, scale=w.scale, num_splits=ns)
    sl = torch.full((3,), 700, dtype=torch.int32, device="cuda")
    o3, l3 = ga.decode_ex(q, k, v, scale=w.scale, num_splits=ns, seqlens_k=sl)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("bs", [1, 16, 128])
def test_paged_equals_contiguous_bitwise(bs, fp8):
    """The same values stored in shuffled pages and contiguously give the
    same bits (the kernels differ only in addressing)."""
    lens = [0, 5, 130, 1001]
    w = gi.cache_decode(lens, 32, 8, 128, seed=9, fp8=fp8, k_scale=0.5, v_scale=2.0)
    S = w.k_cache.shape[1]
    nblk = -(-S // bs)
    perm = torch.randperm(len(lens) * nblk, generator=torch.Generator().manual_seed(bs))
    shape = (len(perm), bs) + tuple(w.k_cache.shape[2:])
    pk = torch.zeros(shape, dtype=torch.float32).to(w.k_cache.dtype)
    pv = pk.clone()
    pad = nblk * bs - S
    kpad = torch.cat([w.k_cache.float(), torch.zeros(len(lens), pad, *shape[2:])], 1)
    vpad = torch.cat([w.v_cache.float(), torch.zeros(len(lens), pad, *shape[2:])], 1)
    table = perm.view(len(lens), nblk).to(torch.int32)
    pk[table.view(-1).long()] = kpad.reshape(-1, bs, *shape[2:]).to(w.k_cache.dtype)
    pv[table.view(-1).long()] = vpad.reshape(-1, bs, *shape[2:]).to(w.v_cache.dtype)
    q, k, v, sl, _ = to_dev(w)
    args = dict(seqlens_k=sl, k_scale=w.k_scale, v_scale=w.v_scale, scale=w.scale)
    o1, l1 = ga.decode_ex(q, k, v, **args)
    o2, l2 = ga.decode_ex(q, pk.cuda(), pv.cuda(), block_table=table.cuda(), max_seqlen_k=S,
                          **args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_split_merge_over_many_sequences():
    """Split partials of 1100 sequences (8800 query rows, beyond the
    longest-first ranking), empty and one-key caches among them, merged."""
    lens = [(13 * i) % 97 for i in range(1100)]
    w = gi.cache_decode(lens, 8, 8, 64, seed=12)
    ro, rl = reference(w)
    for ns in (2, 3):
        o, l = run(w, num_splits=ns)
        compare(o, l, ro, rl, torch.bfloat16, f"1100 sequences ns={ns}")


def test_repeated_split_launches_agree():
    """80 launches with splits, two shapes interleaved (one with empty
    splits) through the same allocator: every repeat equals the first launch
    of its shape bit for bit, and the first ones equal the oracle."""
    wa = gi.cache_decode([0, 1, 40, 700, 2100], 32, 8, 128, seed=13)
    wb = gi.cache_decode([300] * 6, 16, 2, 64, seed=14, with_seqlens=False)
    first = {}
    for i in range(80):
        w, ns = (wa, 4) if i % 2 == 0 else (wb, 2 + (i // 2) % 2)
        key = (i % 2, ns)
        o, l = run(w, num_splits=ns)
        if key not in first:
            first[key] = (o, l)
            ro, rl = reference(w)
            compare(o, l, ro, rl, torch.bfloat16, f"reuse {key}")
        else:
            assert torch.equal(o, first[key][0]) and torch.equal(l, first[key][1]), (i, key)


def test_lengths_out_of_range_are_clamped():
    w = gi.cache_decode([90, 90, 90], 8, 2, 64, seed=10, with_seqlens=False)
    q, k, v, _, _ = to_dev(w)
    bad = torch.tensor([-5, 90, 1 << 20], dtype=torch.int32, device="cuda")
    good = torch.tensor([0, 90, 90], dtype=torch.int32, device="cuda")
    o1, l1 = ga.decode_ex(q, k, v, seqlens_k=bad, scale=w.scale)
    o2, l2 = ga.decode_ex(q, k, v, seqlens_k=good, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", sorted(gi.CACHE_NAMED))
def test_full_size_cache_workloads(name):
    """The full-size cache workloads, every output row, at the split counts
    the bench times (1 and 4)."""
    w = gi.CACHE_NAMED[name]()
    ro, rl = reference(w)
    for ns in (1, 4):
        o, l = run(w, num_splits=ns)
        compare(o, l, ro, rl, torch.bfloat16, f"{w.name} ns={ns}")
