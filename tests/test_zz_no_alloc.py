"""gqa_attn_decode_noalloc (the decode entry point that allocates nothing:
its split partials live in the library's static device scratch) against
gqa_attn_decode with a caller workspace, through the C ABI.

Both run the same kernels on the same inputs, so the outputs must agree bit
for bit; both are also checked against the fp64 oracle at the bf16 bounds.
Two calls in a row, the second on a smaller input, show that the scratch's
leftover contents from the first call do not leak into the second.
"""
import numpy as np
import pytest
import torch

import gqa_attention_amd as ga
import gqa_inputs
import oracle
from parity_util import compare

pytestmark = pytest.mark.gpu


def _both(w, ns):
    q, k, v = w.q.cuda(), w.k.cuda(), w.v.cuda()
    ref_o, ref_l = ga.decode(q, k, v, scale=w.scale, num_splits=ns)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    got_o, got_l = ga.decode_noalloc(q, k, v, scale=w.scale, num_splits=ns, out=out, lse=lse)
    torch.cuda.synchronize()
    return got_o.cpu(), got_l.cpu(), ref_o.cpu(), ref_l.cpu()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_noalloc_equals_workspace_decode_twice(dtype):
    big = gqa_inputs.decode(16, 32, 8, 1500, 128, seed=71, dtype=dtype)
    small = gqa_inputs.decode(3, 8, 2, 300, 64, seed=72, dtype=dtype)
    for w, ns in ((big, 8), (small, 4)):
        go, gl, ro, rl = _both(w, ns)
        assert torch.equal(go, ro) and torch.equal(gl, rl), (w.q.shape, ns)
        eo, el = oracle.decode(w.q, w.k, w.v, w.scale)
        compare(go, gl, eo, el, dtype, f"noalloc {tuple(w.q.shape)} ns={ns}")


def test_noalloc_single_split_and_full_decode_workload_shape():
    w = gqa_inputs.decode(64, 32, 8, 512, 128, seed=73)
    for ns in (1, 8):
        go, gl, ro, rl = _both(w, ns)
        assert torch.equal(go, ro) and torch.equal(gl, rl), ns


def test_noalloc_rejects_partials_beyond_the_scratch():
    # 1024 x 64 heads x 129 floats x 4 bytes x 64 splits = 2.2 GB of partials
    q = torch.zeros(1024, 64, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1024, 64, 8, 128, dtype=torch.bfloat16, device="cuda")
    need = ga.decode_workspace_bytes(1024, 64, 128, 64)
    assert need > ga.NOALLOC_SCRATCH_BYTES
    with pytest.raises(ValueError, match="static scratch"):
        ga.decode_noalloc(q, k, k, num_splits=64)
