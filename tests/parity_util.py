"""Helpers for GPU-vs-oracle parity tests (test infrastructure)."""
import numpy as np
import torch

import gqa_attention_amd as ga
import oracle

# Tolerances against the exact fp64 result: bf16 inputs (bf16 products, fp32
# accumulation, bf16 output) and fp32 mode.
TOL = {torch.bfloat16: (2e-2, 1e-3), torch.float32: (1e-5, 1e-5)}


def to_dev(w, device="cuda"):
    t = lambda x: None if x is None else x.to(device)
    return t(w.q), t(w.k), t(w.v), t(w.cu_seqlens_q), t(w.cu_seqlens_k)


def run_fwd(w, device="cuda"):
    q, k, v, cq, ck = to_dev(w, device)
    if w.varlen:
        o, l = ga.fwd(q, k, v, causal=w.causal, scale=w.scale, cu_seqlens_q=cq, cu_seqlens_k=ck,
                      max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k)
    else:
        o, l = ga.fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o.cpu(), l.cpu()


def oracle_fwd(w):
    if w.varlen:
        return oracle.attention(w.q, w.k, w.v, w.scale, w.causal, w.cu_seqlens_q.tolist(),
                                w.cu_seqlens_k.tolist())
    return oracle.attention(w.q, w.k, w.v, w.scale, w.causal)


def compare(o_gpu, l_gpu, o_ref, l_ref, dtype, what=""):
    """Element-wise check against the oracle; returns (max|dO|, max|dLSE|)."""
    tol_o, tol_l = TOL[dtype]
    o = o_gpu.to(torch.float64).numpy()
    l = l_gpu.to(torch.float64).numpy()
    assert o.shape == o_ref.shape, (what, o.shape, o_ref.shape)
    assert l.shape == l_ref.shape, (what, l.shape, l_ref.shape)
    assert not np.isnan(o).any() and not np.isnan(l).any(), f"{what}: NaN in GPU output"
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l), fin), f"{what}: -inf pattern of LSE differs"
    assert np.all(l[~fin] == l_ref[~fin]), f"{what}: LSE of empty rows"
    do = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    dl = float(np.max(np.abs(l[fin] - l_ref[fin]))) if fin.any() else 0.0
    assert do <= tol_o, f"{what}: max|dO| = {do:.3e} > {tol_o}"
    assert dl <= tol_l, f"{what}: max|dLSE| = {dl:.3e} > {tol_l}"
    return do, dl
