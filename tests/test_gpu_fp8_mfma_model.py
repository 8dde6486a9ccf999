"""The fp8 matrix-core model of ``tests/fp8_mfma_model.py`` against the
hardware: ``gqa_attention_amd/mfma_fp8_probe --dump`` runs one
v_mfma_scale_f32_32x32x64_f8f6f4 per block of crafted and random e4m3 codes
(and fp32 accumulators) and prints the codes and the results. Every result of
the crafted blocks, of the random sums with a zero accumulator and of the
sums of one or two products with a random accumulator must equal the model's
bit for bit; on random sums with random accumulators (block c0rand) at least
95 % must, and every result lies within 2^-23 (|C| + sum |a_k b_k|) of the
model's. The fp8-forward parity bound at large dequantisation scales is
derived from this model."""
import os
import subprocess

import numpy as np
import pytest

from fp8_mfma_model import e4m3_value, mfma_f8_sum

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "gqa_attention_amd", "mfma_fp8_probe")


def _blocks(text):
    blocks = {}
    for line in text.splitlines():
        if not line.startswith("dump "):
            continue
        _, name, kind, *vals = line.split()
        if kind in ("A", "B"):
            arr = np.array([int(v, 16) for v in vals], dtype=np.uint8)
        else:
            arr = np.array([float.fromhex(v) for v in vals], dtype=np.float32)
        blocks.setdefault(name, {})[kind] = arr
    return blocks


def test_model_reproduces_the_fp8_matrix_core():
    assert os.path.exists(PROBE), "build the probe: python -m gqa_attention_amd.build"
    out = subprocess.run([PROBE, "--dump"], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout[-2000:] + out.stderr[-2000:]
    blocks = _blocks(out.stdout)
    assert {"gap", "c0", "cancel", "pos", "neg", "frac", "random", "c0rand", "c0one",
            "c0two"} <= set(blocks)
    for name, d in blocks.items():
        A = d["A"].reshape(32, 64)
        B = d["B"].reshape(64, 32)
        a = np.broadcast_to(A[:, None, :], (32, 32, 64))
        b = np.broadcast_to(B.T[None, :, :], (32, 32, 64))
        c0 = d["C0"].reshape(32, 32)
        model = mfma_f8_sum(a, b, c0)
        got = d["OUT"].reshape(32, 32)
        same = model.view(np.uint32) == got.view(np.uint32)
        scale = np.abs(c0.astype(np.float64)) + np.abs(e4m3_value(a) * e4m3_value(b)).sum(-1)
        dev = np.abs(got.astype(np.float64) - model.astype(np.float64))
        assert np.all(dev <= 2.0 ** -23 * scale), f"block {name}: max deviation {dev.max()}"
        if name == "c0rand":
            assert same.mean() >= 0.95, f"block {name}: only {same.sum()} of 1024 equal"
        else:
            assert same.all(), f"block {name}: {(~same).sum()} of 1024 differ, e.g. " \
                f"{got[~same][:3]} vs model {model[~same][:3]}"
