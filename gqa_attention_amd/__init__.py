"""Python binding of libgqa_attn.so (argument marshalling only).

Every step of the attention computation runs in the HIP kernels behind the C
ABI declared in ``include/gqa_attn.h``; this module only checks tensor
metadata, allocates outputs with ``torch.empty`` on the tensors' device, and
passes raw device pointers plus the current HIP stream. There is no CPU
fallback: if the library is missing, importing works but every call raises.

Functions mirror the C entry points:

* ``fwd(q, k, v, causal=False, scale=None, cu_seqlens_q=None, cu_seqlens_k=None,
  max_seqlen_q=None, max_seqlen_k=None)`` -> ``(out, lse)``
* ``fwd_fp8(q, k, v, q_scale=1.0, k_scale=1.0, v_scale=1.0, causal=False, ...)`` ->
  ``(out, lse)``: the forward over float8_e4m3fn inputs with per-tensor
  dequantisation scales (bf16 out); ``FwdPlan(..., fp8_scales=(qs, ks, vs))``
* ``decode(q, k_cache, v_cache, scale=None, num_splits=1, workspace=None)`` ->
  ``(out, lse)``
* ``bwd(q, k, v, out, lse, dout, causal=False, scale=None, cu_seqlens_q=None,
  cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None)`` -> ``(dq, dk, dv)``
* ``decode_ex(q, k_cache, v_cache, seqlens_k=None, block_table=None,
  window_left=-1, k_scale=1.0, v_scale=1.0, ...)`` -> ``(out, lse)``: decode
  over a ragged, paged, windowed, bf16 or fp8 e4m3 cache
* ``decode_workspace_bytes(B, Hq, d, num_splits)``,
  ``decode_num_splits(B, Hq, Hkv, d, max_seqlen_k, window_left=-1, ragged=False)``
* ``FwdPlan`` / ``BwdPlan`` / ``DecodePlan`` / ``DecodeExPlan``: the same
  calls marshalled once, re-issued by ``run()`` (for loops over fixed shapes
  and buffers)
* ``strerror(status)``
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = ["fwd", "fwd_fp8", "bwd", "decode", "decode_ex", "FwdPlan", "BwdPlan", "DecodePlan", "DecodeExPlan",
           "bwd_workspace_bytes",
           "decode_workspace_bytes", "decode_num_splits", "strerror", "lib", "library_path",
           "GQA_OK", "GQA_EINVAL", "GQA_EUNSUPPORTED", "GQA_EWORKSPACE", "GQA_ELAUNCH",
           "GQA_DTYPE_BF16", "GQA_DTYPE_FP32", "GQA_DTYPE_FP8_E4M3", "GqaError"]

GQA_OK, GQA_EINVAL, GQA_EUNSUPPORTED, GQA_EWORKSPACE, GQA_ELAUNCH, GQA_ESCRATCH = 0, 1, 2, 3, 4, 5
# bytes of the static device scratch behind decode_noalloc (per GPU)
NOALLOC_SCRATCH_BYTES = 16 << 20
GQA_DTYPE_BF16, GQA_DTYPE_FP32, GQA_DTYPE_FP8_E4M3 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgqa_attn.so")
_lib = None


class GqaError(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {strerror(status)} (status {status})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m gqa_attention_amd.build` "
            "(there is no fallback implementation)")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.gqa_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32,
                               vp, vp, i32, vp]
    L.gqa_attn_fwd.restype = i32
    L.gqa_attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32,
                                   vp, vp, f32, f32, f32, vp]
    L.gqa_attn_fwd_fp8.restype = i32
    L.gqa_attn_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, sz,
                                  i32, vp]
    L.gqa_attn_decode.restype = i32
    L.gqa_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                                          i32, vp]
    L.gqa_attn_decode_noalloc.restype = i32
    L.gqa_attn_decode_ex.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, i32, vp,
                                     i32, i32, i32, i32, f32, f32, i32, vp, sz, vp]
    L.gqa_attn_decode_ex.restype = i32
    L.gqa_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                               f32, i32, vp, vp, vp, sz, i32, vp]
    L.gqa_attn_bwd.restype = i32
    L.gqa_attn_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    L.gqa_attn_bwd_workspace_bytes.restype = sz
    L.gqa_attn_decode_num_splits.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.gqa_attn_decode_num_splits.restype = i32
    L.gqa_attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.gqa_attn_decode_workspace_bytes.restype = sz
    L.gqa_attn_strerror.argtypes = [i32]
    L.gqa_attn_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().gqa_attn_strerror(int(status)).decode()


def _raise(status: int, where: str):
    if status == GQA_OK:
        return
    if status == GQA_ELAUNCH:
        raise GqaError(status, where)
    raise ValueError(f"{where}: {strerror(status)} (status {status})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GQA_DTYPE_BF16
    if t.dtype == torch.float32:
        return GQA_DTYPE_FP32
    raise ValueError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _check(name: str, t: torch.Tensor, ndim: int, dtype: torch.dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _prepare_fwd(q, k, v, causal, scale, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                 max_seqlen_k, out, lse, fp8_scales=None):
    """Check tensor metadata, allocate outputs, build the C argument tuple.

    fp8_scales = (q_scale, k_scale, v_scale) for gqa_attn_fwd_fp8: q, k, v are
    float8_e4m3fn and out is bfloat16."""
    dt = q.dtype
    varlen = cu_seqlens_q is not None or cu_seqlens_k is not None
    nd = 3 if varlen else 4
    dev = q.device
    if fp8_scales is not None and dt != torch.float8_e4m3fn:
        raise ValueError(f"q has dtype {dt}, expected torch.float8_e4m3fn")
    _check("q", q, nd, dt, None)
    _check("k", k, nd, dt, dev)
    _check("v", v, nd, dt, dev)
    code = _dtype_code(q) if fp8_scales is None else None
    out_dt = dt if fp8_scales is None else torch.bfloat16
    d = q.shape[-1]
    if k.shape[-1] != d or v.shape[-1] != d or k.shape != v.shape:
        raise ValueError("q, k, v head_dim and k/v shapes must agree")
    Hq, Hkv = q.shape[-2], k.shape[-2]
    if varlen:
        if cu_seqlens_q is None or cu_seqlens_k is None:
            raise ValueError("give both cu_seqlens_q and cu_seqlens_k")
        _check("cu_seqlens_q", cu_seqlens_q, 1, torch.int32, dev)
        _check("cu_seqlens_k", cu_seqlens_k, 1, torch.int32, dev)
        if cu_seqlens_q.shape != cu_seqlens_k.shape:
            raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
        if max_seqlen_q is None or max_seqlen_k is None:
            raise ValueError("variable length needs max_seqlen_q and max_seqlen_k")
        B = cu_seqlens_q.shape[0] - 1
        Sq, Sk = int(max_seqlen_q), int(max_seqlen_k)
        lse_shape = (q.shape[0], Hq)
        cq, ck = cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr()
    else:
        B, Sq = q.shape[0], q.shape[1]
        Sk = k.shape[1]
        if k.shape[0] != B:
            raise ValueError("q and k/v batch sizes differ")
        lse_shape = (B, Hq, Sq)
        cq = ck = None
    if out is None:
        out = torch.empty(q.shape, dtype=out_dt, device=dev)
    else:
        _check("out", out, nd, out_dt, dev)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if lse is None:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=dev)
    else:
        _check("lse", lse, len(lse_shape), torch.float32, dev)
        if tuple(lse.shape) != lse_shape:
            raise ValueError(f"lse must have shape {lse_shape}")
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq,
            Hkv, Sq, Sk, d, sc, int(bool(causal)), cq, ck)
    args += (code,) if fp8_scales is None else tuple(float(x) for x in fp8_scales)
    return out, lse, args, q.numel() == 0


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
        scale: Optional[float] = None, cu_seqlens_q: Optional[torch.Tensor] = None,
        cu_seqlens_k: Optional[torch.Tensor] = None, max_seqlen_q: Optional[int] = None,
        max_seqlen_k: Optional[int] = None, out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Exact GQA attention forward through ``gqa_attn_fwd``.

    Fixed length: q [B, Sq, Hq, d], k/v [B, Sk, Hkv, d] -> out like q,
    lse fp32 [B, Hq, Sq]. Variable length: q [Tq, Hq, d], k/v [Tk, Hkv, d],
    int32 cu_seqlens [B+1] on the device and the maximum lengths (which size
    the grid; no host read of device data happens) -> lse fp32 [Tq, Hq].
    ``scale`` defaults to 1/sqrt(d).
    """
    out, lse, args, empty = _prepare_fwd(q, k, v, causal, scale, cu_seqlens_q, cu_seqlens_k,
                                         max_seqlen_q, max_seqlen_k, out, lse)
    if not empty:
        with torch.cuda.device(q.device):
            st = lib().gqa_attn_fwd(*args, _stream_handle(q.device))
        _raise(st, "gqa_attn_fwd")
    return out, lse


def fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, q_scale: float = 1.0,
            k_scale: float = 1.0, v_scale: float = 1.0, causal: bool = False,
            scale: Optional[float] = None, cu_seqlens_q: Optional[torch.Tensor] = None,
            cu_seqlens_k: Optional[torch.Tensor] = None, max_seqlen_q: Optional[int] = None,
            max_seqlen_k: Optional[int] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention forward over fp8 e4m3 inputs through ``gqa_attn_fwd_fp8``.

    q, k, v are torch.float8_e4m3fn tensors in the layouts of :func:`fwd`;
    the values they stand for are code x q_scale (k_scale, v_scale). Returns
    out (bfloat16, q's shape) and lse (fp32) as :func:`fwd` does.
    """
    out, lse, args, empty = _prepare_fwd(q, k, v, causal, scale, cu_seqlens_q, cu_seqlens_k,
                                         max_seqlen_q, max_seqlen_k, out, lse,
                                         (q_scale, k_scale, v_scale))
    if not empty:
        with torch.cuda.device(q.device):
            st = lib().gqa_attn_fwd_fp8(*args, _stream_handle(q.device))
        _raise(st, "gqa_attn_fwd_fp8")
    return out, lse


class FwdPlan:
    """A forward call with its arguments checked and marshalled once.

    ``run()`` re-issues the same ``gqa_attn_fwd`` call on the current stream
    (the tensors given at construction must stay alive and keep their
    addresses); meant for loops that call the same shapes repeatedly.
    """

    def __init__(self, q, k, v, *, causal=False, scale=None, cu_seqlens_q=None,
                 cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, out=None, lse=None,
                 fp8_scales=None):
        self.out, self.lse, self._args, self._empty = _prepare_fwd(
            q, k, v, causal, scale, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
            out, lse, fp8_scales)
        self._keep = (q, k, v, cu_seqlens_q, cu_seqlens_k)
        self._dev = q.device
        self._name = "gqa_attn_fwd" if fp8_scales is None else "gqa_attn_fwd_fp8"
        self._fn = getattr(lib(), self._name)

    def run(self):
        if not self._empty:
            st = self._fn(*self._args, _stream_handle(self._dev))
            if st:
                _raise(st, self._name)
        return self.out, self.lse


def bwd_workspace_bytes(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, d: int) -> int:
    return int(lib().gqa_attn_bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, d))


def _prepare_bwd(q, k, v, out, lse, dout, causal, scale, cu_seqlens_q, cu_seqlens_k,
                 max_seqlen_q, max_seqlen_k, dq, dk, dv, workspace):
    """Check metadata, allocate gradients and workspace, build the C arguments."""
    _, _, fargs, empty = _prepare_fwd(q, k, v, causal, scale, cu_seqlens_q, cu_seqlens_k,
                                      max_seqlen_q, max_seqlen_k, out, lse)
    dev = q.device
    _check("dout", dout, q.dim(), q.dtype, dev)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    if q.dtype != torch.bfloat16:
        raise ValueError("the backward supports bfloat16 inputs")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check(name, t, ref.dim(), ref.dtype, dev)
        if t.shape != ref.shape:
            raise ValueError(f"{name} must have shape {tuple(ref.shape)}")
    (qp, kp, vp_, op, lp, B, Hq, Hkv, Sq, Sk, d, sc, causal_i, cq, ck, code) = fargs
    need = bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    args = (qp, kp, vp_, op, lp, dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
            B, Hq, Hkv, Sq, Sk, d, sc, causal_i, cq, ck, workspace.data_ptr(), ws_bytes, code)
    return dq, dk, dv, workspace, args


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, *, causal: bool = False, scale: Optional[float] = None,
        cu_seqlens_q: Optional[torch.Tensor] = None, cu_seqlens_k: Optional[torch.Tensor] = None,
        max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
        dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
        dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None
        ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradients of ``fwd`` through ``gqa_attn_bwd`` (bf16).

    ``out`` and ``lse`` are ``fwd``'s results for the same inputs and
    arguments; ``dout`` is the gradient of ``out``. Returns (dq, dk, dv) in
    the layouts of q, k, v.
    """
    dq, dk, dv, _, args = _prepare_bwd(q, k, v, out, lse, dout, causal, scale, cu_seqlens_q,
                                       cu_seqlens_k, max_seqlen_q, max_seqlen_k, dq, dk, dv,
                                       workspace)
    with torch.cuda.device(q.device):
        st = lib().gqa_attn_bwd(*args, _stream_handle(q.device))
    _raise(st, "gqa_attn_bwd")
    return dq, dk, dv


class BwdPlan:
    """A backward call checked and marshalled once; ``run()`` re-issues it."""

    def __init__(self, q, k, v, out, lse, dout, *, causal=False, scale=None, cu_seqlens_q=None,
                 cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, dq=None, dk=None,
                 dv=None, workspace=None):
        self.dq, self.dk, self.dv, self.workspace, self._args = _prepare_bwd(
            q, k, v, out, lse, dout, causal, scale, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
            max_seqlen_k, dq, dk, dv, workspace)
        self._keep = (q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_k)
        self._dev = q.device
        self._fn = lib().gqa_attn_bwd

    def run(self):
        st = self._fn(*self._args, _stream_handle(self._dev))
        if st:
            _raise(st, "gqa_attn_bwd")
        return self.dq, self.dk, self.dv


def decode_num_splits(B: int, Hq: int, Hkv: int, d: int, max_seqlen_k: int,
                      window_left: int = -1, ragged: bool = False) -> int:
    """Split count the library recommends for a decode of this shape (0 if
    invalid); ``ragged``: the sequences' cache lengths differ."""
    return int(lib().gqa_attn_decode_num_splits(B, Hq, Hkv, d, max_seqlen_k, window_left,
                                                int(bool(ragged))))


def decode_workspace_bytes(B: int, Hq: int, d: int, num_splits: int) -> int:
    return int(lib().gqa_attn_decode_workspace_bytes(B, Hq, d, num_splits))


def _prepare_decode(q, k_cache, v_cache, scale, num_splits, workspace, out, lse):
    """Check tensor metadata, allocate outputs / workspace, build the C arguments."""
    dt = q.dtype
    dev = q.device
    _check("q", q, 3, dt, None)
    _check("k_cache", k_cache, 4, dt, dev)
    _check("v_cache", v_cache, 4, dt, dev)
    code = _dtype_code(q)
    B, Hq, d = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[-1] != d:
        raise ValueError("cache shapes must be [B, Sk, Hkv, d] matching q")
    Sk, Hkv = k_cache.shape[1], k_cache.shape[2]
    if out is None:
        out = torch.empty(q.shape, dtype=dt, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    _check("out", out, 3, dt, dev)
    _check("lse", lse, 2, torch.float32, dev)
    need = decode_workspace_bytes(B, Hq, d, num_splits) if num_splits >= 1 else 0
    if num_splits > 1 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
            lse.data_ptr(), B, Hq, Hkv, Sk, d, sc, int(num_splits), ws_ptr, ws_bytes, code)
    return out, lse, workspace, args


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, *,
           scale: Optional[float] = None, num_splits: int = 1,
           workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-KV decode through ``gqa_attn_decode``.

    q [B, Hq, d]; caches [B, Sk, Hkv, d] -> out [B, Hq, d], lse fp32 [B, Hq].
    For num_splits > 1 a uint8 device workspace of
    ``decode_workspace_bytes(B, Hq, d, num_splits)`` bytes is allocated unless
    one is passed.
    """
    out, lse, _, args = _prepare_decode(q, k_cache, v_cache, scale, num_splits, workspace,
                                        out, lse)
    with torch.cuda.device(q.device):
        st = lib().gqa_attn_decode(*args, _stream_handle(q.device))
    _raise(st, "gqa_attn_decode")
    return out, lse


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, *,
                   scale: Optional[float] = None, num_splits: int = 1,
                   out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-KV decode through ``gqa_attn_decode_noalloc``: the library's
    static device scratch holds the split partials, so the call itself
    allocates nothing (pass ``out`` and ``lse`` to allocate nothing here
    either). Same layouts and results as ``decode``; calls that overlap on
    one GPU race on the shared scratch."""
    out, lse, _, args = _prepare_decode(q, k_cache, v_cache, scale, 1, None, out, lse)
    args = args[:11] + (int(num_splits), args[14])
    with torch.cuda.device(q.device):
        st = lib().gqa_attn_decode_noalloc(*args, _stream_handle(q.device))
    _raise(st, "gqa_attn_decode_noalloc")
    return out, lse


class DecodePlan:
    """A decode call checked and marshalled once; ``run()`` re-issues it."""

    def __init__(self, q, k_cache, v_cache, *, scale=None, num_splits=1, workspace=None,
                 out=None, lse=None):
        self.out, self.lse, self.workspace, self._args = _prepare_decode(
            q, k_cache, v_cache, scale, num_splits, workspace, out, lse)
        self._keep = (q, k_cache, v_cache)
        self._dev = q.device
        self._fn = lib().gqa_attn_decode

    def run(self):
        st = self._fn(*self._args, _stream_handle(self._dev))
        if st:
            _raise(st, "gqa_attn_decode")
        return self.out, self.lse


def _prepare_decode_ex(q, k_cache, v_cache, seqlens_k, block_table, max_seqlen_k,
                       window_left, k_scale, v_scale, scale, num_splits, workspace, out, lse):
    """Check tensor metadata, allocate outputs / workspace, build the C arguments."""
    dev = q.device
    _check("q", q, 3, torch.bfloat16, None)
    kv_dt = k_cache.dtype
    if kv_dt == torch.bfloat16:
        code = GQA_DTYPE_BF16
    elif kv_dt == torch.float8_e4m3fn:
        code = GQA_DTYPE_FP8_E4M3
    else:
        raise ValueError(f"k_cache dtype {kv_dt}: expected bfloat16 or float8_e4m3fn")
    _check("k_cache", k_cache, 4, kv_dt, dev)
    _check("v_cache", v_cache, 4, kv_dt, dev)
    B, Hq, d = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[-1] != d:
        raise ValueError("k_cache and v_cache must have the same shape, head_dim as q")
    Hkv = k_cache.shape[2]
    if block_table is None:
        if k_cache.shape[0] != B:
            raise ValueError("contiguous caches must be [B, max_seqlen_k, Hkv, d]")
        cap = k_cache.shape[1]
        if max_seqlen_k is not None and int(max_seqlen_k) != cap:
            raise ValueError("a contiguous cache's max_seqlen_k is its second dimension")
        bptr, bsize, nblk = None, 0, 0
    else:
        _check("block_table", block_table, 2, torch.int32, dev)
        if block_table.shape[0] != B:
            raise ValueError("block_table must be [B, max_blocks_per_seq]")
        bsize, nblk = k_cache.shape[1], block_table.shape[1]
        cap = bsize * nblk
        bptr = block_table.data_ptr()
    smax = cap if max_seqlen_k is None else int(max_seqlen_k)
    if seqlens_k is not None:
        _check("seqlens_k", seqlens_k, 1, torch.int32, dev)
        if seqlens_k.shape[0] != B:
            raise ValueError("seqlens_k must be [B]")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    _check("out", out, 3, torch.bfloat16, dev)
    _check("lse", lse, 2, torch.float32, dev)
    need = decode_workspace_bytes(B, Hq, d, num_splits) if num_splits >= 1 else 0
    if num_splits > 1 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
            lse.data_ptr(), B, Hq, Hkv, d, sc,
            seqlens_k.data_ptr() if seqlens_k is not None else None, smax, bptr, bsize, nblk,
            int(window_left), code, float(k_scale), float(v_scale), int(num_splits), ws_ptr,
            ws_bytes)
    return out, lse, workspace, args


def decode_ex(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, *,
              seqlens_k: Optional[torch.Tensor] = None,
              block_table: Optional[torch.Tensor] = None, max_seqlen_k: Optional[int] = None,
              window_left: int = -1, k_scale: float = 1.0, v_scale: float = 1.0,
              scale: Optional[float] = None, num_splits: int = 1,
              workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Decode through ``gqa_attn_decode_ex`` over a general K/V cache.

    q [B, Hq, d] bf16. Contiguous caches [B, S, Hkv, d]; paged caches
    [pages, block_size, Hkv, d] with an int32 device ``block_table``
    [B, max_blocks_per_seq]. Cache dtype bfloat16 or float8_e4m3fn (then
    ``k_scale`` / ``v_scale`` dequantise). ``seqlens_k`` int32 [B] on the
    device gives each sequence's key count (None: all hold ``max_seqlen_k``,
    which defaults to the cache's capacity). ``window_left`` W >= 0 keeps the
    last W + 1 keys. Returns out [B, Hq, d] bf16, lse fp32 [B, Hq].
    """
    out, lse, _, args = _prepare_decode_ex(q, k_cache, v_cache, seqlens_k, block_table,
                                           max_seqlen_k, window_left, k_scale, v_scale, scale,
                                           num_splits, workspace, out, lse)
    with torch.cuda.device(q.device):
        st = lib().gqa_attn_decode_ex(*args, _stream_handle(q.device))
    _raise(st, "gqa_attn_decode_ex")
    return out, lse


class DecodeExPlan:
    """A ``decode_ex`` call checked and marshalled once; ``run()`` re-issues it."""

    def __init__(self, q, k_cache, v_cache, *, seqlens_k=None, block_table=None,
                 max_seqlen_k=None, window_left=-1, k_scale=1.0, v_scale=1.0, scale=None,
                 num_splits=1, workspace=None, out=None, lse=None):
        self.out, self.lse, self.workspace, self._args = _prepare_decode_ex(
            q, k_cache, v_cache, seqlens_k, block_table, max_seqlen_k, window_left, k_scale,
            v_scale, scale, num_splits, workspace, out, lse)
        self._keep = (q, k_cache, v_cache, seqlens_k, block_table)
        self._dev = q.device
        self._fn = lib().gqa_attn_decode_ex

    def run(self):
        st = self._fn(*self._args, _stream_handle(self._dev))
        if st:
            _raise(st, "gqa_attn_decode_ex")
        return self.out, self.lse
