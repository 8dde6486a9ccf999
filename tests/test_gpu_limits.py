"""GPU parity at the largest K/V row pitch the boundary accepts.

The forward, dQ and fp8-forward kernels address a key tile as a 64-bit tile
base plus 24-bit per-lane byte offsets, and the boundary accepts Hkv x d up to
4194304 (a bf16 K row of 8 MiB). These cases sit exactly on that limit
(32768 K/V heads at d = 128, 65536 at d = 64), with a ragged key tail, and are
checked at sampled rows (and keys, for the gradients) against the fp64
oracle; one element past the limit is rejected (``tests/test_host_abi.py``).
"""
import numpy as np
import pytest
import torch

import gqa_attention_amd as ga
import gqa_inputs as gi
from oracle import backward as ob
from oracle import fp8_forward as of8
from oracle import gqa as oa
from parity_util import compare

pytestmark = pytest.mark.gpu

S = 40  # two 32-key tiles, the second ragged


def _rows(g, n, S, H):
    pick = lambda hi: torch.randint(0, hi, (n,), generator=g).tolist()
    return list(zip([0] * n, pick(S), pick(H))) + [(0, 0, 0), (0, S - 1, H - 1)]


@pytest.mark.parametrize("hkv,d", [(32768, 128), (65536, 64)])
def test_fwd_at_max_row_pitch(hkv, d):
    assert hkv * d == 1 << 22
    w = gi.fixed(1, hkv, hkv, S, S, d, seed=60 + d, causal=True)
    o, l = ga.fwd(w.q.cuda(), w.k.cuda(), w.v.cuda(), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    rows = _rows(torch.Generator().manual_seed(61), 24, S, hkv)
    ro, rl = oa.attention_rows(w.q, w.k, w.v, w.scale, True, rows)
    got_o = torch.stack([o[b, i, h].cpu() for b, i, h in rows])
    got_l = torch.tensor([float(l[b, h, i]) for b, i, h in rows])
    compare(got_o, got_l, ro, rl, torch.bfloat16, f"fwd max pitch hkv={hkv} d={d}")


@pytest.mark.parametrize("hkv,d,causal", [(32768, 128, False), (65536, 64, True)])
def test_fwd_fp8_at_max_row_pitch(hkv, d, causal):
    w = gi.fixed_fp8(1, hkv, hkv, S, S, d, seed=62 + d, causal=causal, q_scale=0.5,
                     k_scale=0.25, v_scale=0.5)
    o, l = ga.fwd_fp8(w.q.cuda(), w.k.cuda(), w.v.cuda(), q_scale=0.5, k_scale=0.25,
                      v_scale=0.5, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    rows = _rows(torch.Generator().manual_seed(63), 24, S, hkv)
    ro, rl = of8.attention_rows_fp8(w.q, w.k, w.v, w.scale, causal, 0.5, 0.25, 0.5, rows)
    got_o = torch.stack([o[b, i, h].cpu() for b, i, h in rows])
    got_l = torch.tensor([float(l[b, h, i]) for b, i, h in rows])
    compare(got_o, got_l, ro, rl, torch.bfloat16, "fwd fp8 max pitch")


@pytest.mark.parametrize("hkv,d", [(32768, 128), (65536, 64)])
def test_bwd_at_max_row_pitch(hkv, d):
    w = gi.fixed(1, hkv, hkv, S, S, d, seed=64 + d, causal=True)
    g = torch.Generator().manual_seed(65)
    do = torch.randn(w.q.shape, generator=g).to(torch.bfloat16)
    q, k, v = w.q.cuda(), w.k.cuda(), w.v.cuda()
    o, l = ga.fwd(q, k, v, causal=True, scale=w.scale)
    dq, dk, dv = ga.bwd(q, k, v, o, l, do.cuda(), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    rows = _rows(torch.Generator().manual_seed(66), 16, S, hkv)
    keys = _rows(torch.Generator().manual_seed(67), 16, S, hkv)
    refs = ob.attention_grad_sampled(w.q, w.k, w.v, do, w.scale, True, rows, keys)
    got = (torch.stack([dq[b, i, h].cpu() for b, i, h in rows]),
           torch.stack([dk[b, j, h].cpu() for b, j, h in keys]),
           torch.stack([dv[b, j, h].cpu() for b, j, h in keys]))
    for name, gg, r in zip(("dq", "dk", "dv"), got, refs):
        err = float(np.max(np.abs(gg.double().numpy() - r)))
        assert err <= 2e-2 * float(np.max(np.abs(r))) + 1e-4, (name, err)
