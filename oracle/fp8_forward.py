"""fp64 CPU oracle for the attention forward over fp8 (e4m3) inputs.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, links or runs
this module: only the tests, the smoke check and the bench's CPU-baseline leg
do. It shares no code with the HIP kernels.

* gitcode GQA batch-size guide, hardware section (FP8 precision to relieve
  memory bandwidth) and the precision row of its parameter table: the inputs
  are stored in 8 bits. The pages fix no format; the OCP E4M3 format is taken
  (decoded by ``oracle.cache.fp8_e4m3_decode``), with one dequantisation scale
  per tensor: the value of a stored code is its decoded value times the scale.
* What is computed is the exact attention of those values: the definition in
  ``oracle.gqa`` (FlashAttention-2 summary, standard-attention paragraph;
  Ultralytics glossary "Grouped Query Attention (GQA)", section "How GQA
  works"), unchanged. Reading taken here: the quantisation is the caller's
  (the codes and scales are the inputs), so the oracle applies no rounding of
  its own; the rounding of P and O inside a kernel is covered by the parity
  tolerance, as for bf16 inputs.

Parity pins live in ``tests/test_oracle_fp8_forward.py``.
"""
from __future__ import annotations

from typing import Optional, Sequence

from . import gqa as _gqa
from .cache import stored_values


def dequantised(q, k, v, q_scale: float, k_scale: float, v_scale: float):
    """fp64 values of e4m3-stored q, k, v (float8_e4m3fn tensors or uint8 codes)."""
    return (stored_values(q, True, q_scale), stored_values(k, True, k_scale),
            stored_values(v, True, v_scale))


def attention_fp8(q, k, v, scale: float, causal: bool, q_scale: float, k_scale: float,
                  v_scale: float, cu_seqlens_q: Optional[Sequence[int]] = None,
                  cu_seqlens_k: Optional[Sequence[int]] = None):
    """Exact attention (O, LSE) of the dequantised inputs, in the layouts of
    ``oracle.gqa.attention``."""
    qv, kv, vv = dequantised(q, k, v, q_scale, k_scale, v_scale)
    return _gqa.attention(qv, kv, vv, scale, causal, cu_seqlens_q, cu_seqlens_k)


def attention_rows_fp8(q, k, v, scale: float, causal: bool, q_scale: float, k_scale: float,
                       v_scale: float, rows, cu_seqlens_q=None, cu_seqlens_k=None):
    """The same at chosen (sequence, row, head) triples (``oracle.gqa.attention_rows``)."""
    qv, kv, vv = dequantised(q, k, v, q_scale, k_scale, v_scale)
    return _gqa.attention_rows(qv, kv, vv, scale, causal, rows, cu_seqlens_q, cu_seqlens_k)
