"""Build libgqa_attn.so in-tree with hipcc for gfx950.

Usage: python -m gqa_attention_amd.build [-v]

Every library source under csrc/ is compiled to an object in parallel, then linked
into ``gqa_attention_amd/libgqa_attn.so``; ``csrc/hbm_probe.hip`` becomes the
``gqa_attention_amd/hbm_probe`` program (copy and read-stream reference
kernels used to scale HBM byte counters). Packed-fp32 VALU instructions are
disabled for device code (-packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgqa_attn.so")
PROBE = os.path.join(PKG, "hbm_probe")  # copy / read-stream reference program
ARCH = "gfx950"

SOURCES = ["api.cpp", "fwd_bf16.hip", "fwd_f32.hip", "decode_bf16.hip", "bwd_bf16.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libgqa_attn.so")
    return path


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc(), *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops" not in l)  # host pass does not know the feature
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    cmd = [hipcc(), *COMMON, os.path.join(CSRC, "hbm_probe.hip"), "-o", PROBE + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hbm_probe build failed:\n{res.stderr}")
    os.replace(PROBE + ".tmp", PROBE)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
