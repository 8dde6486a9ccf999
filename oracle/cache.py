"""fp64 CPU oracle for decode over a general K/V cache: per-sequence lengths,
paged storage, a sliding window, and fp8 (e4m3) storage.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, links or runs
this module: only the tests, the smoke check and the bench's CPU-baseline leg
do. It shares no code with the HIP kernels.

Each variant changes only WHICH keys a decode query sees and HOW the stored
values are read; the attention itself is the exact definition of
``oracle.gqa`` (one query row per sequence, no mask over the chosen keys).

* Per-sequence cache lengths: decode batches hold caches of different
  lengths. Sequence b owns keys 0 .. L_b - 1.
* Paged cache: Ultralytics glossary "Grouped Query Attention (GQA)", section
  "GQA and related techniques", PagedAttention item: the cache lives in
  fixed-size blocks. Reading taken here: block table row b lists the pages of
  sequence b in key order, so key j sits in slot j mod block_size of page
  table[b][j // block_size].
* Sliding window: same section, sliding-window item: a cap on how many cached
  tokens a layer attends to. Reading taken here: with window_left = W >= 0
  the query (the newest token, position L_b - 1) sees keys j with
  L_b - 1 - W <= j <= L_b - 1, i.e. the last W + 1 keys; W = -1 means no cap.
* fp8 storage: gitcode GQA batch-size guide, hardware section (FP8 precision
  to cut memory-bandwidth pressure) and the precision row of its parameter
  table. The pages fix no format; the OCP 8-bit floating point specification's
  E4M3 format is taken (1 sign bit, 4 exponent bits with bias 7, 3 mantissa
  bits, subnormals, no infinities, S.1111.111 = NaN), with one dequantisation
  scale per tensor: value = decoded code x scale.

Parity pins for every function here live in ``tests/test_oracle_cache.py``.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import gqa as _gqa


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Exact fp64 value of each E4M3 byte code (any integer array shape)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (m == 7), np.nan, val)


def stored_values(cache, fp8: bool, scale: float) -> np.ndarray:
    """fp64 values that stored cache elements stand for: bf16/fp32 exactly;
    fp8 (a float8_e4m3fn tensor or its uint8 codes) as decoded code x the
    per-tensor scale."""
    if not fp8:
        return _gqa.as_f64(cache)
    import torch
    if isinstance(cache, torch.Tensor):
        if cache.dtype != torch.uint8:
            cache = cache.contiguous().view(torch.uint8)
        cache = cache.numpy()
    table = fp8_e4m3_decode(np.arange(256))   # value of every code, looked up below
    return table[np.asarray(cache, dtype=np.uint8)] * float(scale)


def key_slots(b: int, n_keys: int, block_table: Optional[np.ndarray], block_size: int):
    """(page, slot) of keys 0 .. n_keys - 1 of sequence b.

    Contiguous caches are their own pages: page b, slot j.
    """
    j = np.arange(n_keys)
    if block_table is None:
        return np.full(n_keys, b), j
    return np.asarray(block_table)[b, j // block_size], j % block_size


def visible_range(L: int, window_left: int):
    """Keys [lo, L) the newest token of a length-L sequence attends to."""
    if window_left < 0:
        return 0, L
    return max(0, L - 1 - window_left), L


def decode_cache(q, k_cache, v_cache, scale: float, *, seqlens=None, block_table=None,
                 window_left: int = -1, fp8: bool = False, k_scale: float = 1.0,
                 v_scale: float = 1.0):
    """Decode of one new query token per sequence against a general cache.

    q [B, Hq, d]. Contiguous caches [B, S, Hkv, d] (block_table None); paged
    caches [num_pages, block_size, Hkv, d] with block_table int [B, nblk].
    seqlens int [B] (None: every sequence holds S = max_blocks * block_size or
    the contiguous cache's length). Returns O [B, Hq, d], LSE [B, Hq]; a
    sequence that sees no key gets O = 0, LSE = -inf.
    """
    import torch
    qf = _gqa.as_f64(q)
    # Gather each sequence's visible rows first (as raw storage: uint8 codes
    # for fp8), then read their values.
    kraw = k_cache.view(torch.uint8) if fp8 else k_cache
    vraw = v_cache.view(torch.uint8) if fp8 else v_cache
    B, hq, d = qf.shape
    if block_table is None:
        bs, cap = 0, kraw.shape[1]
        table = None
    else:
        table = np.asarray(_gqa.as_f64(block_table), dtype=np.int64)
        bs = kraw.shape[1]
        cap = table.shape[1] * bs
    lens = [cap] * B if seqlens is None else [int(x) for x in np.asarray(_gqa.as_f64(seqlens))]
    out = np.zeros((B, hq, d))
    lse = np.full((B, hq), -np.inf)
    for b in range(B):
        L = lens[b]
        lo, hi = visible_range(L, window_left)
        page, slot = key_slots(b, L, table, bs)
        pi = torch.as_tensor(page[lo:hi], dtype=torch.int64)
        si = torch.as_tensor(slot[lo:hi], dtype=torch.int64)
        keys = stored_values(kraw[pi, si], fp8, k_scale)      # [n, Hkv, d]
        vals = stored_values(vraw[pi, si], fp8, v_scale)
        o, l = _gqa._sequence(qf[b][None], keys, vals, scale, False)
        out[b], lse[b] = o[0], l[:, 0]
    return out, lse
