"""Host-side checks of the C ABI that need no GPU.

The library must load and export every function the header declares, and
every argument error must be reported before anything is launched (so these
calls never reach the device: the pointers below are fake but never
dereferenced).
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import gqa_attention_amd as ga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")

needs_lib = pytest.mark.skipif(not os.path.exists(ga.library_path()),
                               reason="libgqa_attn.so not built")

FAKE = 0x10000  # 16-byte aligned, never dereferenced (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(gqa_attn_\w+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_api():
    assert declared_functions() == ["gqa_attn_bwd", "gqa_attn_bwd_workspace_bytes",
                                    "gqa_attn_decode", "gqa_attn_decode_ex",
                                    "gqa_attn_decode_noalloc", "gqa_attn_decode_num_splits",
                                    "gqa_attn_decode_workspace_bytes", "gqa_attn_fwd",
                                    "gqa_attn_fwd_fp8", "gqa_attn_strerror"]


@needs_lib
def test_library_exports_every_declared_symbol():
    L = ga.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ga.library_path()], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (gqa_attn_\w+)", out))
    assert set(declared_functions()) <= exported


@needs_lib
def test_strerror():
    assert ga.strerror(0) == "success"
    for s in (1, 2, 3, 4, 5):
        assert ga.strerror(s) and ga.strerror(s) != "unknown status"
    assert ga.strerror(99) == "unknown status"


def fwd_call(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, B=1, Hq=8, Hkv=2, Sq=16, Sk=16, d=64,
             scale=0.125, causal=1, cu_q=None, cu_k=None, dtype=0, stream=None)
    a.update(kw)
    return ga.lib().gqa_attn_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"],
                                 a["Hkv"], a["Sq"], a["Sk"], a["d"], a["scale"], a["causal"],
                                 a["cu_q"], a["cu_k"], a["dtype"], a["stream"])


def dec_call(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, B=2, Hq=8, Hkv=2, Sk=100, d=128,
             scale=0.1, ns=4, ws=FAKE, ws_bytes=1 << 30, dtype=0, stream=None)
    a.update(kw)
    return ga.lib().gqa_attn_decode(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"],
                                    a["Hkv"], a["Sk"], a["d"], a["scale"], a["ns"], a["ws"],
                                    a["ws_bytes"], a["dtype"], a["stream"])


FWD_ERRORS = [
    (dict(q=None), ga.GQA_EINVAL),
    (dict(lse=None), ga.GQA_EINVAL),
    (dict(d=96), ga.GQA_EUNSUPPORTED),
    (dict(d=256), ga.GQA_EUNSUPPORTED),
    (dict(dtype=7), ga.GQA_EUNSUPPORTED),
    (dict(Hq=6, Hkv=4), ga.GQA_EINVAL),
    (dict(Hkv=0), ga.GQA_EINVAL),
    (dict(B=0), ga.GQA_EINVAL),
    (dict(Sq=0), ga.GQA_EINVAL),
    (dict(Sk=0), ga.GQA_EINVAL),
    (dict(scale=float("nan")), ga.GQA_EINVAL),
    (dict(scale=float("inf")), ga.GQA_EINVAL),
    (dict(scale=0.0), ga.GQA_EINVAL),
    (dict(scale=-0.5), ga.GQA_EINVAL),
    (dict(cu_q=FAKE), ga.GQA_EINVAL),  # only one of the two offset arrays
    (dict(cu_q=FAKE, cu_k=FAKE, Sq=-1), ga.GQA_EINVAL),
    (dict(q=FAKE + 8), ga.GQA_EINVAL),  # misaligned
    (dict(out=FAKE + 4), ga.GQA_EINVAL),
    (dict(lse=FAKE + 2), ga.GQA_EINVAL),
    (dict(cu_q=FAKE + 2, cu_k=FAKE), ga.GQA_EINVAL),
    (dict(Hq=65536, Hkv=65536, d=128), ga.GQA_EINVAL),  # K/V row pitch >= 2^24 bytes
]


@needs_lib
@pytest.mark.parametrize("kw,code", FWD_ERRORS, ids=lambda x: str(x))
def test_fwd_argument_errors(kw, code):
    assert fwd_call(**kw) == code


@needs_lib
def test_fwd_varlen_without_rows_is_a_noop():
    # variable length with max_seqlen_q == 0: nothing to compute, nothing launched
    assert fwd_call(cu_q=FAKE, cu_k=FAKE, Sq=0, Sk=0) == ga.GQA_OK


def fwd8_call(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, B=1, Hq=8, Hkv=2, Sq=16, Sk=16, d=64,
             scale=0.125, causal=1, cu_q=None, cu_k=None, qs=0.5, ks=0.25, vs=2.0, stream=None)
    a.update(kw)
    return ga.lib().gqa_attn_fwd_fp8(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"],
                                     a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"], a["scale"],
                                     a["causal"], a["cu_q"], a["cu_k"], a["qs"], a["ks"], a["vs"],
                                     a["stream"])


FWD8_ERRORS = [
    (dict(q=None), ga.GQA_EINVAL),
    (dict(d=96), ga.GQA_EUNSUPPORTED),
    (dict(Hq=6, Hkv=4), ga.GQA_EINVAL),
    (dict(Sq=0), ga.GQA_EINVAL),
    (dict(scale=0.0), ga.GQA_EINVAL),
    (dict(qs=0.0), ga.GQA_EINVAL),
    (dict(ks=-1.0), ga.GQA_EINVAL),
    (dict(vs=float("nan")), ga.GQA_EINVAL),
    (dict(qs=float("inf")), ga.GQA_EINVAL),
    (dict(scale=1e30, qs=1e30, ks=1e30), ga.GQA_EINVAL),  # combined score scale overflows
    (dict(cu_q=FAKE), ga.GQA_EINVAL),
    (dict(k=FAKE + 8), ga.GQA_EINVAL),
]


@needs_lib
@pytest.mark.parametrize("kw,code", FWD8_ERRORS, ids=lambda x: str(x))
def test_fwd_fp8_argument_errors(kw, code):
    assert fwd8_call(**kw) == code


def test_python_fwd_fp8_rejects_other_dtypes():
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="float8_e4m3fn"):
        ga.fwd_fp8(q, q, q)


@needs_lib
def test_fwd_fp8_varlen_without_rows_is_a_noop():
    assert fwd8_call(cu_q=FAKE, cu_k=FAKE, Sq=0, Sk=0) == ga.GQA_OK


DEC_ERRORS = [
    (dict(q=None), ga.GQA_EINVAL),
    (dict(v=None), ga.GQA_EINVAL),
    (dict(d=32), ga.GQA_EUNSUPPORTED),
    (dict(dtype=-1), ga.GQA_EUNSUPPORTED),
    (dict(Hq=9), ga.GQA_EINVAL),
    (dict(Sk=0), ga.GQA_EINVAL),
    (dict(ns=0), ga.GQA_EINVAL),
    (dict(ns=65), ga.GQA_EINVAL),
    (dict(scale=float("nan")), ga.GQA_EINVAL),
    (dict(k=FAKE + 8), ga.GQA_EINVAL),
    (dict(ws=None), ga.GQA_EWORKSPACE),
    (dict(ws_bytes=1000), ga.GQA_EWORKSPACE),
    (dict(ws=FAKE + 8), ga.GQA_EWORKSPACE),
]


@needs_lib
@pytest.mark.parametrize("kw,code", DEC_ERRORS, ids=lambda x: str(x))
def test_decode_argument_errors(kw, code):
    assert dec_call(**kw) == code


def dex_call(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, B=2, Hq=8, Hkv=2, d=128, scale=0.1,
             seqlens=FAKE, smax=100, table=FAKE, bs=16, nblk=7, window=-1, kv_dtype=0,
             k_scale=1.0, v_scale=1.0, ns=4, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return ga.lib().gqa_attn_decode_ex(
        a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["d"],
        a["scale"], a["seqlens"], a["smax"], a["table"], a["bs"], a["nblk"], a["window"],
        a["kv_dtype"], a["k_scale"], a["v_scale"], a["ns"], a["ws"], a["ws_bytes"], a["stream"])


DEX_ERRORS = [
    (dict(q=None), ga.GQA_EINVAL),
    (dict(lse=None), ga.GQA_EINVAL),
    (dict(d=96), ga.GQA_EUNSUPPORTED),
    (dict(kv_dtype=1), ga.GQA_EUNSUPPORTED),   # fp32 caches are not a decode_ex format
    (dict(kv_dtype=3), ga.GQA_EUNSUPPORTED),
    (dict(Hq=9), ga.GQA_EINVAL),
    (dict(smax=0), ga.GQA_EINVAL),
    (dict(window=-2), ga.GQA_EINVAL),
    (dict(ns=0), ga.GQA_EINVAL),
    (dict(ns=65), ga.GQA_EINVAL),
    (dict(scale=float("nan")), ga.GQA_EINVAL),
    (dict(kv_dtype=2, k_scale=0.0), ga.GQA_EINVAL),
    (dict(kv_dtype=2, v_scale=float("inf")), ga.GQA_EINVAL),
    (dict(bs=24), ga.GQA_EINVAL),              # page size not a power of two
    (dict(bs=8192, nblk=1), ga.GQA_EINVAL),     # page size above 4096
    (dict(bs=0), ga.GQA_EINVAL),
    (dict(nblk=6), ga.GQA_EINVAL),             # 6 * 16 < max_seqlen_k 100
    (dict(table=FAKE + 2), ga.GQA_EINVAL),
    (dict(seqlens=FAKE + 2), ga.GQA_EINVAL),
    (dict(v=FAKE + 8), ga.GQA_EINVAL),
    (dict(ws=None), ga.GQA_EWORKSPACE),
    (dict(ws_bytes=1000), ga.GQA_EWORKSPACE),
]


@needs_lib
@pytest.mark.parametrize("kw,code", DEX_ERRORS, ids=lambda x: str(x))
def test_decode_ex_argument_errors(kw, code):
    assert dex_call(**kw) == code


@needs_lib
def test_decode_ex_ignores_scales_and_page_size_when_unused():
    # bf16 caches ignore the fp8 scales; a contiguous cache ignores the page geometry.
    # Both calls still fail validation on a later, deliberate error (no launch).
    assert dex_call(k_scale=0.0, v_scale=-1.0, ws=None) == ga.GQA_EWORKSPACE
    assert dex_call(table=None, bs=24, nblk=0, ws=None) == ga.GQA_EWORKSPACE


@needs_lib
def test_workspace_size():
    f = ga.decode_workspace_bytes
    assert f(64, 32, 128, 1) == 0
    rows = 64 * 32 * 8
    o = rows * 128 * 4
    assert f(64, 32, 128, 8) == ((o + 255) // 256) * 256 + rows * 4
    assert f(2, 8, 64, 2) >= 2 * 8 * 2 * 65 * 4
    assert f(0, 8, 64, 2) == 0 and f(2, 8, 96, 2) == 0 and f(2, 8, 64, 0) == 0
    assert f(2, 8, 64, 65) == 0
    # exactly enough workspace is accepted by validation (fails only at launch, not run here)
    need = f(2, 8, 128, 4)
    assert dec_call(ws_bytes=need - 1) == ga.GQA_EWORKSPACE


def test_python_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises((ValueError, RuntimeError)):
        ga.fwd(q, q[:, :, :1].contiguous(), q[:, :, :1].contiguous())


@needs_lib
def test_decode_num_splits_rule():
    f = ga.decode_num_splits
    # Llama 3.1 8B heads (32 / 8, one 16-head slice per K/V head)
    assert f(64, 32, 8, 128, 4096) == 1          # 512 workgroups already
    assert f(16, 32, 8, 128, 8192) == 2          # 128 -> 2 splits
    assert f(8, 32, 8, 128, 8192) == 4           # 64 -> 4
    assert f(4, 32, 8, 128, 32768) == 8          # 32 -> 8
    assert f(1, 32, 8, 128, 32768) == 16         # 8 -> 16
    assert f(1, 32, 8, 128, 2048) == 4           # capped: at least 512 keys per split
    assert f(1, 32, 8, 128, 512) == 1
    assert f(1, 32, 8, 128, 100000, 1023) == 2   # a 1024-key window bounds the range
    assert f(1, 48, 1, 64, 32768) == 16          # 48 heads on one K/V head: 3 slices
    assert f(4, 48, 1, 64, 32768) == 8
    assert f(64, 32, 8, 128, 8192, ragged=True) == 2   # ragged: at least 2 splits
    assert f(64, 32, 8, 128, 800, ragged=True) == 1    # ... unless splits get < 512 keys
    # ... or a window of at most half the longest length evens the ranges out
    assert f(32, 32, 8, 128, 16384, 4095, ragged=True) == 1
    assert f(32, 32, 8, 128, 6000, 4095, ragged=True) == 2
    for bad in [(0, 32, 8, 128, 10), (1, 30, 8, 128, 10), (1, 32, 8, 96, 10),
                (1, 32, 8, 128, 0), (1, 32, 8, 128, 10, -2)]:
        assert f(*bad) == 0, bad


def bwd_call(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             B=2, Hq=8, Hkv=2, Sq=100, Sk=120, d=128, scale=0.1, causal=1, cu_q=None, cu_k=None,
             ws=FAKE, ws_bytes=1 << 30, dtype=0, stream=None)
    a.update(kw)
    return ga.lib().gqa_attn_bwd(
        a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"], a["B"],
        a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"], a["scale"], a["causal"], a["cu_q"],
        a["cu_k"], a["ws"], a["ws_bytes"], a["dtype"], a["stream"])


BWD_ERRORS = [
    (dict(q=None), ga.GQA_EINVAL),
    (dict(dout=None), ga.GQA_EINVAL),
    (dict(dq=None), ga.GQA_EINVAL),
    (dict(dk=None), ga.GQA_EINVAL),
    (dict(dv=None), ga.GQA_EINVAL),
    (dict(dv=FAKE + 8), ga.GQA_EINVAL),
    (dict(d=96), ga.GQA_EUNSUPPORTED),
    (dict(dtype=1), ga.GQA_EUNSUPPORTED),      # fp32 has no backward
    (dict(Hq=9), ga.GQA_EINVAL),
    (dict(Sq=0), ga.GQA_EINVAL),
    (dict(scale=0.0), ga.GQA_EINVAL),
    (dict(ws=None), ga.GQA_EWORKSPACE),
    (dict(ws=FAKE + 8), ga.GQA_EWORKSPACE),
    (dict(ws_bytes=1000), ga.GQA_EWORKSPACE),
]


@needs_lib
@pytest.mark.parametrize("kw,code", BWD_ERRORS, ids=lambda x: str(x))
def test_bwd_argument_errors(kw, code):
    assert bwd_call(**kw) == code


@needs_lib
def test_bwd_workspace_size():
    f = ga.bwd_workspace_bytes
    # two fp32 arrays of B * Hkv * round4(Sq * G) rows plus 128 spare floats each
    assert f(2, 8, 2, 100, 120, 128) == 2 * 4 * (2 * 2 * 400 + 128)
    assert f(1, 12, 12, 77, 77, 64) == 2 * 4 * (12 * 80 + 128)
    assert f(0, 8, 2, 10, 10, 64) == 0 and f(1, 9, 2, 10, 10, 64) == 0
    assert f(1, 8, 2, -1, 10, 64) == 0 and f(1, 8, 2, 10, 10, 96) == 0
    # 8 K/V heads x 64 key blocks = 512 dK/dV workgroups: no row chunks
    assert f(1, 32, 8, 8192, 8192, 128) == 4 * 2 * (8 * 32768 + 128)
    # MQA, one sequence: 64 key blocks (< 256) -> ceil(512 / 64) = 8 row chunks
    # per key block, each with fp32 partial dK and dV of 128 keys x d
    stats = 2 * (1 * 262144 + 128)
    assert f(1, 32, 1, 8192, 8192, 128) == 4 * (stats + 1 * 64 * 8 * 2 * 128 * 128)
    need = f(2, 8, 2, 100, 120, 128)
    assert bwd_call(ws_bytes=need - 1) == ga.GQA_EWORKSPACE
    need = f(1, 32, 1, 8192, 8192, 128)
    assert bwd_call(B=1, Hq=32, Hkv=1, Sq=8192, Sk=8192, ws_bytes=need - 1) == ga.GQA_EWORKSPACE


def noalloc_call(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, B=2, Hq=8, Hkv=2, Sk=100, d=128,
             scale=0.1, ns=4, dtype=0, stream=None)
    a.update(kw)
    return ga.lib().gqa_attn_decode_noalloc(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"],
                                            a["Hq"], a["Hkv"], a["Sk"], a["d"], a["scale"],
                                            a["ns"], a["dtype"], a["stream"])


@needs_lib
def test_noalloc_decode_host_errors():
    """The static-scratch decode checks its arguments like gqa_attn_decode and
    rejects partials larger than its scratch, all before any launch."""
    assert noalloc_call(q=None) == ga.GQA_EINVAL
    assert noalloc_call(ns=0) == ga.GQA_EINVAL
    assert noalloc_call(d=96) == ga.GQA_EUNSUPPORTED
    # 1024 x 64 heads x (128 + 1) floats x 64 splits: 2.2 GB > 16 MiB
    assert noalloc_call(B=1024, Hq=64, Hkv=8, Sk=4096, ns=64) == ga.GQA_ESCRATCH
    assert ga.decode_workspace_bytes(1024, 64, 128, 64) > ga.NOALLOC_SCRATCH_BYTES
    # the largest decode-workload shape it is meant for fits: B 64, 32 heads, d 128, 8 splits
    assert ga.decode_workspace_bytes(64, 32, 128, 8) <= ga.NOALLOC_SCRATCH_BYTES
