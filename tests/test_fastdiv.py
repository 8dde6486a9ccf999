"""The forward's division by launch constants (gqa_attention_amd/csrc/fastdiv.h:
multiply-high and shift, Granlund and Montgomery 1994) against plain integer
division, on the host: every divisor 1..1024 and a set of large ones, with
dividends covering small values, every value around multiples of d, and the
top of the range up to 2^31 - 1."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SRC = r"""
#include <cstdio>
#include <cstdlib>
#include "fastdiv.h"
using namespace gqa;
static long long bad = 0, checks = 0;
static void check(int n, int d, FastDiv f) {
    ++checks;
    if (fastdiv_apply(n, f) != n / d && bad++ < 10) std::printf("n=%d d=%d got %d\n", n, d, fastdiv_apply(n, f));
}
int main() {
    const int big[] = {1025, 3000, 4095, 4097, 65535, 65536, 65537, 1000003, 16777215, 16777217,
                       1 << 30, (1 << 30) + 1, 2147483646, 2147483647};
    for (int k = 0; k < 1024 + 14; ++k) {
        const int d = k < 1024 ? k + 1 : big[k - 1024];
        const FastDiv f = fastdiv_for(d);
        if (d > 1 && (f.m < 0x80000000u)) { std::printf("multiplier out of range d=%d\n", d); return 1; }
        for (int n = 0; n < 70000; ++n) check(n, d, f);
        for (long long q = 1; q * d < 2147483647LL && q < (1LL << 31); q = q * 3 + 1)
            for (int e = -2; e <= 2; ++e) {
                const long long n = q * d + e;
                if (n >= 0 && n <= 2147483647LL) check((int)n, d, f);
            }
        for (long long n = 2147483647LL; n > 2147483647LL - 70000; --n) check((int)n, d, f);
        unsigned s = 12345u + d;
        for (int i = 0; i < 20000; ++i) { s = s * 1664525u + 1013904223u; check((int)(s >> 1), d, f); }
    }
    std::printf("%lld checks, %lld wrong\n", checks, bad);
    return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_fastdiv_matches_integer_division(tmp_path):
    src = tmp_path / "fastdiv_check.cpp"
    src.write_text(SRC)
    exe = tmp_path / "fastdiv_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "gqa_attention_amd", "csrc"),
                    str(src), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout
