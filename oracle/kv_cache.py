"""KV-cache size arithmetic.

TEST INFRASTRUCTURE ONLY (see ``oracle/gqa.py``).

gitcode GQA batch-size guide, section on the grouped-sharing mechanism: the
KV memory is 2 x batch x sequence length x head_dim x number of KV heads
(elements, per layer); the factor 2 counts K and V. The Ultralytics glossary
("How GQA shrinks the KV cache") works the same count for Llama 3.1 8B with
32 layers and 16-bit values; ``tests/golden/kv_cache.json`` holds its printed
figures and the glossary snippet's printed per-token counts.
"""
from __future__ import annotations


def kv_cache_elements(batch: int, seq_len: int, head_dim: int, kv_heads: int,
                      layers: int = 1) -> int:
    """Number of cached K and V values."""
    return 2 * batch * seq_len * head_dim * kv_heads * layers


def kv_cache_bytes(batch: int, seq_len: int, head_dim: int, kv_heads: int,
                   layers: int = 1, bytes_per_value: int = 2) -> int:
    """Bytes of the K and V cache."""
    return kv_cache_elements(batch, seq_len, head_dim, kv_heads, layers) * bytes_per_value
