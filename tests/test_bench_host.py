"""Host-side pieces of bench.py that need no GPU."""
import itertools
import subprocess
import sys
import os

import bench
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_flop_formula_matches_brute_count():
    for lq, lk, causal in itertools.product([1, 2, 5, 16, 33], [1, 3, 16, 40], [False, True]):
        assert bench.fwd_flops(lq, lk, 3, 8, causal) == oracle.attention_flops(lq, lk, 3, 8, causal)


def test_named_workload_flops():
    # 8192-token causal prefill, 32 query heads, d 128: 4*32*128*8192*8193/2
    assert bench.fwd_flops(8192, 8192, 32, 128, True) == 549_822_922_752
    # BERT-base encoder: 64 sequences x 4*12*512*512*64
    assert 64 * bench.fwd_flops(512, 512, 12, 64, False) == 51_539_607_552


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_source_digest_ignores_comments_not_code(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n    return x + 1;\n}\n")
    b.write_text("// header\nint f(int x) {  /* note */\n\n    return x + 1;  // inc\n}\n")
    c.write_text("int f(int x) {\n    return x + 2;\n}\n")
    assert bench.source_digest([str(a)]) == bench.source_digest([str(b)])
    assert bench.source_digest([str(a)]) != bench.source_digest([str(c)])


def test_cpu_baseline_pool_on_a_small_varlen_batch():
    import gqa_inputs
    w = gqa_inputs.varlen([40, 10, 70, 30], [40, 10, 70, 30], 4, 1, 64, seed=3, causal=True)
    cb = bench.cpu_baseline(w, frac=0.5)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0
    assert 1 <= cb["cores"] <= cb["affinity_cores"] or cb["cores"] <= 16
    assert "first 3 of 4 sequences" in cb["sample"]  # 40^2 + 10^2 < 50 % <= + 70^2
    assert cb["cpu_model"]
