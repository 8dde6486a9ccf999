"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: the persistent variable-length forward (its scheduling counters
must be back at zero after every execution), the split-KV decode with a
caller workspace, and the decode that allocates nothing. Each of four
replays, with other eager forward calls between them, must equal the eager
results bit for bit."""
import pytest
import torch

import gqa_attention_amd as ga
import gqa_inputs

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager_calls():
    wv = gqa_inputs.varlen([700, 1, 300, 1200, 64], [700, 1, 300, 1200, 64], 8, 2, 128, seed=81,
                           causal=True)
    wd = gqa_inputs.decode(8, 32, 8, 1000, 128, seed=82)
    wo = gqa_inputs.varlen([500, 90], [500, 90], 16, 4, 64, seed=83, causal=False)
    q, k, v = wv.q.cuda(), wv.k.cuda(), wv.v.cuda()
    cq, ck = wv.cu_seqlens_q.cuda(), wv.cu_seqlens_k.cuda()
    dq, dk, dv = wd.q.cuda(), wd.k.cuda(), wd.v.cuda()
    oq, ok_, ov = wo.q.cuda(), wo.k.cuda(), wo.v.cuda()
    ocq, ock = wo.cu_seqlens_q.cuda(), wo.cu_seqlens_k.cuda()
    ws = torch.empty(ga.decode_workspace_bytes(8, 32, 128, 4), dtype=torch.uint8, device="cuda")

    def calls():
        o1, l1 = ga.fwd(q, k, v, causal=True, scale=wv.scale, cu_seqlens_q=cq, cu_seqlens_k=ck,
                        max_seqlen_q=wv.max_seqlen_q, max_seqlen_k=wv.max_seqlen_k)
        o2, l2 = ga.decode(dq, dk, dv, scale=wd.scale, num_splits=4, workspace=ws)
        o3, l3 = ga.decode_noalloc(dq, dk, dv, scale=wd.scale, num_splits=4)
        return [o1, l1, o2, l2, o3, l3]

    def other():
        ga.fwd(oq, ok_, ov, causal=False, scale=wo.scale, cu_seqlens_q=ocq, cu_seqlens_k=ock,
               max_seqlen_q=wo.max_seqlen_q, max_seqlen_k=wo.max_seqlen_k)

    ref = [t.clone() for t in calls()]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = calls()
    for r in range(4):
        other()
        torch.cuda.synchronize()
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), (r, i)
