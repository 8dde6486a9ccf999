"""fp64 CPU oracle for grouped-query attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check in
``__graft_entry__.py`` and by the CPU-baseline leg of ``bench.py``, never by
the ``gqa_attention_amd`` package. It shares no code with the HIP path.

Modules:
  gqa        the plain definition (materialised S and P, K/V expanded per head)
  brute      a pure-Python scalar restatement used to pin ``attention``
  kv_cache   KV-cache size arithmetic pinned to the glossary's printed figures
  cache      decode over a general cache: per-sequence lengths, pages, a
             sliding window, fp8 (e4m3) storage
  backward   gradients dq, dk, dv of the definition (chain rule, materialised)
  fp8_forward  the definition over fp8 (e4m3) inputs with per-tensor scales
"""
from .gqa import (attention, attention_rows, decode, decode_partials,  # noqa: F401
                        merge_partials, split_ranges, attention_flops, head_rows,
                        expand_kv, kv_head_of, visible, as_f64)
from .kv_cache import kv_cache_bytes, kv_cache_elements  # noqa: F401
from .cache import decode_cache, fp8_e4m3_decode  # noqa: F401
from .backward import attention_grad, attention_grad_flops  # noqa: F401
from .fp8_forward import attention_fp8, attention_rows_fp8  # noqa: F401
