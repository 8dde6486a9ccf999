"""Writes tiny_inputs.json: checksums of the tiny causal GQA workload's draws.

The workload takes the draws of the glossary page "Grouped Query Attention
(GQA)" (section "How GQA works", its code example): one generator seeded with
0, then q of shape [1, 8, 16, 64] and k, v of shape [1, 2, 16, 64] (batch,
head, token, head_dim), i.i.d. N(0, 1) in fp32. The workload stores them
token-major ([batch, token, head, head_dim]). This script records the SHA-256
of each tensor's fp32 bytes in the drawn head-major order, and its first four
values, so the test can check the generator without restating its draws.

Run from the repository root: python tests/golden/make_tiny_inputs.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import gqa_inputs  # noqa: E402


def main():
    w = gqa_inputs.tiny_causal_gqa_fp32()
    rec = {"source": "glossary page 'Grouped Query Attention (GQA)', section 'How GQA works', "
                     "code example: seed 0, q [1,8,16,64], k and v [1,2,16,64] (BHSD), N(0,1) fp32"}
    for name, t in (("q", w.q), ("k", w.k), ("v", w.v)):
        bhsd = t.transpose(1, 2).contiguous()
        rec[name] = {"shape_bhsd": list(bhsd.shape),
                     "sha256_fp32": hashlib.sha256(bhsd.numpy().tobytes()).hexdigest(),
                     "first4": [float(x) for x in bhsd.flatten()[:4]]}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_inputs.json"), "w") as fh:
        json.dump(rec, fh, indent=1)


if __name__ == "__main__":
    main()
