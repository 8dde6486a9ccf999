"""Seeded synthetic inputs for grouped-query attention.

This module only draws random tensors and builds sequence offsets. It holds
none of the attention arithmetic, so both the fp64 oracle (``oracle/``) and
the HIP path (``gqa_attention_amd``) can take their inputs from it without
sharing any computation.

Recipe (every tensor is i.i.d. N(0, 1)):

* one ``torch.Generator('cpu')`` per workload, seeded with the workload's seed;
* draws happen in the order q, k, v (variable-length workloads draw the
  sequence lengths first);
* fp32 is drawn, then bf16 workloads are rounded to bf16 with round-to-nearest
  even (``.to(torch.bfloat16)``); the oracle reads those same bf16 values
  upcast to fp64.

Layouts: fixed length ``[B, S, H, d]`` (batch, sequence, head, head_dim);
variable length ``[T, H, d]`` with int32 ``cu_seqlens`` of length B+1;
decode ``q [B, Hq, d]`` with a cache ``[B, Sk, Hkv, d]``; general-cache decode
(``CacheWorkload``) with a contiguous or paged cache and per-sequence lengths.

The five named workloads take their shapes from the pages: the GQA snippet of
the Ultralytics glossary page "Grouped Query Attention (GQA)" (8 query heads,
2 KV heads, 16 tokens, head_dim 64), a BERT-base encoder (12 heads, d 64,
sequence 512, batch 64) from the gitcode GQA batch-size guide's A100 BERT
table, Llama 3.1 8B (32 query heads, 8 KV heads, d 128) from the glossary's
KV-cache section, the 48/12 (4:1) grouping from the guide's KV-memory
paragraph, and variable-length packed inputs from the Raptor-T abstract.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch


@dataclass
class Workload:
    """One seeded input set. Tensors live on the CPU; callers copy them."""

    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    causal: bool
    scale: float
    cu_seqlens_q: Optional[torch.Tensor] = None  # int32 [B+1]
    cu_seqlens_k: Optional[torch.Tensor] = None
    max_seqlen_q: Optional[int] = None
    max_seqlen_k: Optional[int] = None
    decode: bool = False
    # fp8 e4m3 inputs (q, k, v are torch.float8_e4m3fn): (q_scale, k_scale,
    # v_scale), the per-tensor dequantisation scales; None for bf16 / fp32.
    fp8_scales: Optional[tuple] = None

    @property
    def varlen(self) -> bool:
        return self.cu_seqlens_q is not None


def _randn(g: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(*shape, dtype=torch.float32, generator=g)
    return x.to(dtype) if dtype != torch.float32 else x


def fixed(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, d: int, *, seed: int,
          dtype: torch.dtype = torch.bfloat16, causal: bool = False,
          scale: Optional[float] = None, name: str = "fixed") -> Workload:
    """Fixed-length q [B, Sq, Hq, d], k/v [B, Sk, Hkv, d]."""
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (B, Sq, Hq, d), dtype)
    k = _randn(g, (B, Sk, Hkv, d), dtype)
    v = _randn(g, (B, Sk, Hkv, d), dtype)
    return Workload(name, q, k, v, causal, d ** -0.5 if scale is None else scale)


def varlen(lengths_q, lengths_k, Hq: int, Hkv: int, d: int, *, seed: int,
           dtype: torch.dtype = torch.bfloat16, causal: bool = False,
           scale: Optional[float] = None, name: str = "varlen") -> Workload:
    """Packed q [sum Lq, Hq, d], k/v [sum Lk, Hkv, d] with int32 cu_seqlens."""
    lq = [int(x) for x in lengths_q]
    lk = [int(x) for x in lengths_k]
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (sum(lq), Hq, d), dtype)
    k = _randn(g, (sum(lk), Hkv, d), dtype)
    v = _randn(g, (sum(lk), Hkv, d), dtype)
    cq = torch.tensor([0] + lq, dtype=torch.int64).cumsum(0).to(torch.int32)
    ck = torch.tensor([0] + lk, dtype=torch.int64).cumsum(0).to(torch.int32)
    return Workload(name, q, k, v, causal, d ** -0.5 if scale is None else scale,
                    cq, ck, max(lq) if lq else 0, max(lk) if lk else 0)


def fixed_fp8(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, d: int, *, seed: int,
              causal: bool = False, q_scale: float = 1.0, k_scale: float = 1.0,
              v_scale: float = 1.0, scale: Optional[float] = None,
              name: str = "fixed_fp8") -> Workload:
    """As ``fixed``, with the N(0, 1) draws rounded to e4m3
    (``.to(torch.float8_e4m3fn)``) and the given dequantisation scales."""
    w = fixed(B, Hq, Hkv, Sq, Sk, d, seed=seed, dtype=torch.float8_e4m3fn, causal=causal,
              scale=scale, name=name)
    w.fp8_scales = (float(q_scale), float(k_scale), float(v_scale))
    return w


def varlen_fp8(lengths_q, lengths_k, Hq: int, Hkv: int, d: int, *, seed: int,
               causal: bool = False, q_scale: float = 1.0, k_scale: float = 1.0,
               v_scale: float = 1.0, scale: Optional[float] = None,
               name: str = "varlen_fp8") -> Workload:
    """As ``varlen``, with e4m3 storage and dequantisation scales."""
    w = varlen(lengths_q, lengths_k, Hq, Hkv, d, seed=seed, dtype=torch.float8_e4m3fn,
               causal=causal, scale=scale, name=name)
    w.fp8_scales = (float(q_scale), float(k_scale), float(v_scale))
    return w


def decode(B: int, Hq: int, Hkv: int, Sk: int, d: int, *, seed: int,
           dtype: torch.dtype = torch.bfloat16, scale: Optional[float] = None,
           name: str = "decode") -> Workload:
    """One new token per sequence: q [B, Hq, d]; cache k/v [B, Sk, Hkv, d]."""
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (B, Hq, d), dtype)
    k = _randn(g, (B, Sk, Hkv, d), dtype)
    v = _randn(g, (B, Sk, Hkv, d), dtype)
    return Workload(name, q, k, v, False, d ** -0.5 if scale is None else scale,
                    decode=True)


# Stored value of cache slots that no sequence owns (the tail of a sequence's
# last page, the tail of a contiguous cache row, the spare page that unused
# block-table entries point to). Exactly representable in bf16 and e4m3; large
# enough that attending to it by mistake changes the result visibly.
POISON = 16.0


@dataclass
class CacheWorkload:
    """Decode against a general K/V cache (per-sequence lengths, optional
    paging, sliding window, bf16 or fp8 e4m3 storage). CPU tensors."""

    name: str
    q: torch.Tensor                       # [B, Hq, d] bf16
    k_cache: torch.Tensor                 # [B, S, Hkv, d] or [pages, block_size, Hkv, d]
    v_cache: torch.Tensor
    seqlens: Optional[torch.Tensor]       # int32 [B], None: every sequence holds S keys
    block_table: Optional[torch.Tensor]   # int32 [B, blocks_per_seq], None: contiguous
    block_size: int                       # 0 for a contiguous cache
    max_seqlen_k: int
    window_left: int                      # -1: no window
    k_scale: float                        # dequantisation scales (1 for bf16)
    v_scale: float
    scale: float

    @property
    def fp8(self) -> bool:
        return self.k_cache.dtype == torch.float8_e4m3fn

    @property
    def batch(self) -> int:
        return self.q.shape[0]

    def lengths(self):
        if self.seqlens is None:
            return [self.max_seqlen_k] * self.batch
        return [int(x) for x in self.seqlens.tolist()]


def cache_decode(lengths, Hq: int, Hkv: int, d: int, *, seed: int, block_size: int = 0,
                 window_left: int = -1, fp8: bool = False, k_scale: float = 1.0,
                 v_scale: float = 1.0, with_seqlens: bool = True,
                 scale: Optional[float] = None, name: str = "cache_decode") -> CacheWorkload:
    """q [B, Hq, d] bf16 and a K/V cache holding lengths[b] keys of sequence b.

    Draw order: q, then the page permutation (paged only), then k, then v.
    Contiguous (block_size 0): caches [B, max(lengths), Hkv, d]. Paged: each
    sequence gets ceil(L / block_size) pages taken from a random permutation
    of all pages; one extra page is left unowned; caches
    [pages, block_size, Hkv, d], block table int32 [B, ceil(max L / block_size)]
    with every unused entry naming the unowned page. Stored values are
    N(0, 1) rounded to bf16, or to e4m3 (``.to(torch.float8_e4m3fn)``) when
    fp8; unowned slots hold POISON. ``with_seqlens=False`` (all lengths
    equal) gives no length array.
    """
    lens = [int(x) for x in lengths]
    if not with_seqlens and len(set(lens)) != 1:
        raise ValueError("with_seqlens=False needs equal lengths")
    B = len(lens)
    S = max(max(lens), 1)
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (B, Hq, d), torch.bfloat16)
    if block_size == 0:
        k = torch.randn(B, S, Hkv, d, generator=g)
        v = torch.randn(B, S, Hkv, d, generator=g)
        for b, L in enumerate(lens):
            k[b, L:] = POISON
            v[b, L:] = POISON
        table = None
    else:
        nblk = -(-S // block_size)
        used = [-(-L // block_size) for L in lens]
        n_pages = sum(used) + 1
        perm = torch.randperm(n_pages, generator=g).tolist()
        spare = perm[-1]
        table = torch.full((B, nblk), spare, dtype=torch.int32)
        k = torch.randn(n_pages, block_size, Hkv, d, generator=g)
        v = torch.randn(n_pages, block_size, Hkv, d, generator=g)
        k[spare] = POISON
        v[spare] = POISON
        at = 0
        for b, L in enumerate(lens):
            pages = perm[at:at + used[b]]
            at += used[b]
            table[b, :used[b]] = torch.tensor(pages, dtype=torch.int32)
            if used[b] and L % block_size:
                k[pages[-1], L % block_size:] = POISON
                v[pages[-1], L % block_size:] = POISON
    dt = torch.float8_e4m3fn if fp8 else torch.bfloat16
    k, v = k.to(dt), v.to(dt)
    seqlens = torch.tensor(lens, dtype=torch.int32) if with_seqlens else None
    return CacheWorkload(name, q, k, v, seqlens, table, block_size, S, window_left,
                         k_scale if fp8 else 1.0, v_scale if fp8 else 1.0,
                         d ** -0.5 if scale is None else scale)


# ---------------------------------------------------------------------------
# The five named workloads.
# ---------------------------------------------------------------------------

def tiny_causal_gqa_fp32() -> Workload:
    """8 query heads, 2 KV heads, 16 tokens, d 64, causal, fp32.

    Drawn exactly as the glossary snippet draws them: seed 0, then
    randn(1, 8, 16, 64) for q and randn(1, 2, 16, 64) for k and v in the
    [batch, heads, seq, d] layout; transposed here to [batch, seq, heads, d].
    """
    g = torch.Generator().manual_seed(0)
    q = torch.randn(1, 8, 16, 64, generator=g)
    k = torch.randn(1, 2, 16, 64, generator=g)
    v = torch.randn(1, 2, 16, 64, generator=g)
    t = lambda x: x.transpose(1, 2).contiguous()
    return Workload("tiny_causal_gqa_fp32", t(q), t(k), t(v), True, 64 ** -0.5)


def bert_base_encoder() -> Workload:
    """Non-causal MHA: B 64, S 512, 12 heads, d 64, bf16 (seed 2)."""
    return fixed(64, 12, 12, 512, 512, 64, seed=2, causal=False,
                 name="bert_base_encoder_b64_s512_h12_d64")


def llama31_8b_prefill() -> Workload:
    """Causal GQA prefill: B 1, S 8192, 32 query / 8 KV heads, d 128, bf16 (seed 3)."""
    return fixed(1, 32, 8, 8192, 8192, 128, seed=3, causal=True,
                 name="llama31_8b_prefill_s8192_h32_kv8_d128")


def llama31_8b_decode() -> Workload:
    """Decode: B 64, 32 query / 8 KV heads, d 128, 4096-token cache, bf16 (seed 4)."""
    return decode(64, 32, 8, 4096, 128, seed=4,
                  name="llama31_8b_decode_b64_kv4096_h32_kv8_d128")


def varlen_packed_causal_48_12() -> Workload:
    """Packed causal GQA 4:1: 48 query / 12 KV heads, d 128, 32 sequences.

    Lengths are drawn first, uniform on [128, 4096] from seed 5.
    """
    g = torch.Generator().manual_seed(5)
    lengths = torch.randint(128, 4097, (32,), generator=g).tolist()
    T = sum(lengths)
    q = _randn(g, (T, 48, 128), torch.bfloat16)
    k = _randn(g, (T, 12, 128), torch.bfloat16)
    v = _randn(g, (T, 12, 128), torch.bfloat16)
    cu = torch.tensor([0] + lengths, dtype=torch.int64).cumsum(0).to(torch.int32)
    return Workload("varlen_packed_causal_h48_kv12_d128_n32", q, k, v, True,
                    128 ** -0.5, cu, cu.clone(), max(lengths), max(lengths))


def llama31_8b_prefill_fp8() -> Workload:
    """The Llama 3.1 8B causal prefill shape (B 1, S 8192, 32 / 8 heads, d 128)
    over e4m3 inputs with q_scale 0.5, k_scale 0.25, v_scale 0.5 (seed 10)."""
    return fixed_fp8(1, 32, 8, 8192, 8192, 128, seed=10, causal=True, q_scale=0.5,
                     k_scale=0.25, v_scale=0.5, name="llama31_8b_prefill_fp8_s8192_h32_kv8_d128")


def bert_base_encoder_fp8() -> Workload:
    """The BERT-base encoder shape (B 64, S 512, 12 heads, d 64, non-causal)
    over e4m3 inputs with q_scale 0.5, k_scale 0.25, v_scale 0.5 (seed 11)."""
    return fixed_fp8(64, 12, 12, 512, 512, 64, seed=11, causal=False, q_scale=0.5,
                     k_scale=0.25, v_scale=0.5, name="bert_base_encoder_fp8_b64_s512_h12_d64")


def llama31_8b_decode_ragged_paged(fp8: bool = False) -> CacheWorkload:
    """Decode over a paged cache of ragged lengths: B 64, 32 query / 8 KV
    heads, d 128, cache lengths uniform on [1, 8192] (drawn first from seed 6),
    16-key pages; bf16, or e4m3 with k_scale 0.25 and v_scale 0.5."""
    g = torch.Generator().manual_seed(6)
    lengths = torch.randint(1, 8193, (64,), generator=g).tolist()
    tag = "fp8" if fp8 else "bf16"
    return cache_decode(lengths, 32, 8, 128, seed=7, block_size=16, fp8=fp8,
                        k_scale=0.25, v_scale=0.5,
                        name=f"llama31_8b_decode_ragged_paged16_{tag}_b64_h32_kv8_d128")


def sliding_window_decode() -> CacheWorkload:
    """Sliding-window decode (window of 4096 keys, as Mistral 7B pairs with
    GQA): B 32, 32 query / 8 KV heads, d 128, cache lengths uniform on
    [1, 16384] (drawn first from seed 8), 16-key pages, bf16."""
    g = torch.Generator().manual_seed(8)
    lengths = torch.randint(1, 16385, (32,), generator=g).tolist()
    return cache_decode(lengths, 32, 8, 128, seed=9, block_size=16, window_left=4095,
                        name="sliding_window4096_decode_paged16_b32_h32_kv8_d128")


CACHE_NAMED = {
    "decode_ragged_paged": lambda: llama31_8b_decode_ragged_paged(False),
    "decode_ragged_paged_fp8": lambda: llama31_8b_decode_ragged_paged(True),
    "decode_sliding_window": sliding_window_decode,
}


NAMED = {
    "tiny_causal_gqa_fp32": tiny_causal_gqa_fp32,
    "bert_base_encoder": bert_base_encoder,
    "llama31_8b_prefill": llama31_8b_prefill,
    "llama31_8b_decode": llama31_8b_decode,
    "varlen_packed_causal": varlen_packed_causal_48_12,
    "llama31_8b_prefill_fp8": llama31_8b_prefill_fp8,
    "bert_base_encoder_fp8": bert_base_encoder_fp8,
}
