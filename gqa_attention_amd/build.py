"""Build libgqa_attn.so in-tree with hipcc for gfx950.

Usage: python -m gqa_attention_amd.build [-v]

Every library source under csrc/ is compiled to an object in parallel, then linked
into ``gqa_attention_amd/libgqa_attn.so`` (and ``libgqa_attn_timeline.so``, the
same library with the forward's per-tile timestamps compiled in, a probe for
``bench.py --tile-timeline``); ``csrc/hbm_probe.hip`` becomes the
``gqa_attention_amd/hbm_probe`` program (copy and read-stream reference
kernels used to scale HBM byte counters) and ``csrc/issue_probe.hip`` the
``gqa_attention_amd/issue_probe`` program (whether the matrix cores run while
the same SIMD issues vector instructions; ``issue_probe_vform`` is the same
program with the matrix accumulators forced into ordinary VGPRs) and
``csrc/mfma_fp8_probe.hip`` the ``gqa_attention_amd/mfma_fp8_probe`` program
(how the fp8 matrix core sums its 64 products). Packed-fp32 VALU instructions are
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
TIMELINE_LIB = os.path.join(PKG, "libgqa_attn_timeline.so")  # probe build of the same library
PROBE = os.path.join(PKG, "hbm_probe")  # copy / read-stream reference program
PROBES = {"hbm_probe": ("hbm_probe.hip", []), "issue_probe": ("issue_probe.hip", []),
          "issue_probe_vform": ("issue_probe.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
          "mfma_fp8_probe": ("mfma_fp8_probe.hip", [])}
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


def _compile(src: str, verbose: bool, extra=(), suffix: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + suffix + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc(), *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
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
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        futs = [ex.submit(_compile, s, verbose) for s in SOURCES]
        # the timeline probe: the same library with the forward's per-tile
        # timestamps compiled in (bench.py --tile-timeline)
        tl_fut = ex.submit(_compile, "fwd_bf16.hip", verbose, ["-DGQA_TILE_TIMELINE=1"], "_timeline")
        objs = [f.result() for f in futs]
        tl_obj = tl_fut.result()
    for out, members in ((LIB, objs), (TIMELINE_LIB, [tl_obj if o.endswith("fwd_bf16.o") else o
                                                     for o in objs])):
        tmp = out + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *members]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stderr}")
        os.replace(tmp, out)
    for prog, (src, extra) in PROBES.items():
        out = os.path.join(PKG, prog)
        cmd = [hipcc(), *COMMON, *extra, os.path.join(CSRC, src), "-o", out + ".tmp"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"{prog} build failed:\n{res.stderr}")
        os.replace(out + ".tmp", out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
