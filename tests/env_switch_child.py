"""Child process of tests/test_gpu_env_switches.py (test infrastructure): the
forward under one of the library's environment switches, which it reads once
per process, against the fp64 oracle. argv[1]: "unpacked" (GQA_ATTN_PACK=0:
one query head per row tile) or "one_tile" (GQA_FWD_PERSISTENT=0: one
workgroup per row tile for variable-length batches). Exits non-zero on a
mismatch."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import torch  # noqa: E402

import gqa_inputs  # noqa: E402
from parity_util import compare, oracle_fwd, run_fwd  # noqa: E402

mode = sys.argv[1]
if mode == "unpacked":
    assert os.environ.get("GQA_ATTN_PACK") == "0"
    cases = [
        gqa_inputs.fixed(2, 8, 2, 200, 200, 128, seed=901, causal=True),
        gqa_inputs.fixed(1, 6, 2, 77, 130, 64, seed=902, causal=False),
        gqa_inputs.fixed(1, 12, 4, 300, 65, 128, seed=903, causal=True),
        gqa_inputs.varlen([3, 0, 257, 130], [5, 1, 257, 90], 8, 2, 128, seed=904, causal=True),
        gqa_inputs.varlen([64, 1, 500], [64, 700, 500], 16, 4, 64, seed=905, causal=False),
    ]
elif mode == "one_tile":
    assert os.environ.get("GQA_FWD_PERSISTENT") == "0"
    cases = [
        gqa_inputs.varlen([3, 0, 257, 130, 1000], [5, 1, 257, 90, 1000], 8, 2, 128, seed=911, causal=True),
        gqa_inputs.varlen([64, 1, 500, 333], [64, 700, 500, 2], 16, 4, 64, seed=912, causal=False),
        gqa_inputs.varlen([700] * 3 + [17] * 5, [700] * 3 + [17] * 5, 12, 3, 64, seed=913, causal=True),
    ]
else:
    raise SystemExit(f"unknown mode {mode}")
for i, w in enumerate(cases):
    o, l = run_fwd(w)
    ro, rl = oracle_fwd(w)
    do, dl = compare(o, l, ro, rl, torch.bfloat16, f"{mode} case {i}")
    print(f"{mode} case {i}: max|dO| {do:.2e} max|dLSE| {dl:.2e}", flush=True)
print(f"{mode} ok")
