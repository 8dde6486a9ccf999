"""Process-pool driver for the fp64 oracle at full workload sizes.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, links or runs
this module: only the tests and the bench's CPU-baseline leg do. It shares no
code with the HIP kernels.

It computes nothing of its own. The work of ``oracle.gqa.attention`` is cut
into independent units, one per (sequence, query head, block of rows), and
each unit is exactly one call of ``oracle.gqa.head_rows`` on that head's query
rows, the keys and values of the K/V head ``oracle.gqa.kv_head_of`` gives, and
the rows of ``oracle.gqa.visible``. Softmax is per row, so the units are
independent and their union is the whole definition; the result equals the
serial ``attention`` bit for bit (``tests/test_oracle_pool.py``).

Scheduling: one worker process per core the process may run on
(``os.sched_getaffinity``), capped at ``max_workers`` (16 by default, one GPU's
share of a host), each with its BLAS limited to one thread. Units are issued
largest first. Inputs reach the workers through memory-mapped files in a
temporary directory (exact float32 copies of bf16/fp32 inputs, or float64),
and the workers write O and LSE into memory-mapped fp64 files that the caller
receives as arrays.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import shutil
import tempfile
import time
from functools import lru_cache
from typing import Optional, Sequence

import numpy as np

from . import gqa as _gqa

_ROW_BLOCK_BYTES = 64 << 20  # cap on one unit's materialised S/P block


def affinity_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def default_workers(max_workers: int = 16) -> int:
    """Worker count: the cores this process may run on, at most max_workers."""
    env = os.environ.get("GQA_ORACLE_WORKERS")
    if env:
        return max(1, int(env))
    return max(1, min(affinity_cores(), max_workers))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def _stage(x, path: str) -> str:
    """Write x to an .npy file: float32 when the values are float32-exact
    (bf16, fp16 and fp32 tensors), else float64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            if x.dtype in (torch.bfloat16, torch.float16, torch.float32):
                a = x.detach().to("cpu", torch.float32).numpy()
            else:
                a = _gqa.as_f64(x)
            np.save(path, a)
            return path
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    np.save(path, a if a.dtype in (np.float32, np.float64) else a.astype(np.float64))
    return path


# ---- worker side ----
_W = {}


def _init_worker(paths):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass
    _W.clear()
    for name, p in paths.items():
        _W[name] = np.load(p, mmap_mode="r+" if name in ("o", "lse") else "r")


@lru_cache(maxsize=64)
def _visible(lq: int, lk: int, causal: bool) -> np.ndarray:
    return _gqa.visible(lq, lk, causal)


def _run_unit(unit):
    """One (sequence, head, row block): oracle.gqa.head_rows on it."""
    (q0, lq, k0, lk, b, h, r0, r1, hq, hkv, scale, causal, varlen) = unit
    q, k, v, o, lse = _W["q"], _W["k"], _W["v"], _W["o"], _W["lse"]
    kvh = _gqa.kv_head_of(h, hq, hkv)
    if varlen:
        qr = np.asarray(q[q0 + r0:q0 + r1, h, :], dtype=np.float64)
        kh = np.asarray(k[k0:k0 + lk, kvh, :], dtype=np.float64)
        vh = np.asarray(v[k0:k0 + lk, kvh, :], dtype=np.float64)
    else:
        qr = np.asarray(q[b, r0:r1, h, :], dtype=np.float64)
        kh = np.asarray(k[b, :, kvh, :], dtype=np.float64)
        vh = np.asarray(v[b, :, kvh, :], dtype=np.float64)
    out, l = _gqa.head_rows(qr, kh, vh, scale, _visible(lq, lk, causal)[r0:r1])
    if varlen:
        o[q0 + r0:q0 + r1, h, :] = out
        lse[q0 + r0:q0 + r1, h] = l
    else:
        o[b, r0:r1, h, :] = out
        lse[b, h, r0:r1] = l
    return (r1 - r0) * lk


def _units(q_shape, k_shape, scale, causal, cu_q, cu_k, heads=None, seqs=None):
    """Units largest first. heads / seqs restrict the work to some query
    heads / sequences (the rest of O stays 0 and of LSE -inf)."""
    units = []
    varlen = cu_q is not None
    if varlen:
        hq, hkv = q_shape[1], k_shape[1]
        nb = len(cu_q) - 1
        bounds = [(int(cu_q[b]), int(cu_q[b + 1]) - int(cu_q[b]), int(cu_k[b]),
                   int(cu_k[b + 1]) - int(cu_k[b])) for b in range(nb)]
    else:
        hq, hkv = q_shape[2], k_shape[2]
        nb = q_shape[0]
        bounds = [(0, q_shape[1], 0, k_shape[1])] * nb
    for b in (range(nb) if seqs is None else seqs):
        q0, lq, k0, lk = bounds[b]
        if lq == 0:
            continue
        step = max(1, _ROW_BLOCK_BYTES // (8 * max(lk, 1)))
        for h in (range(hq) if heads is None else heads):
            for r0 in range(0, lq, step):
                units.append((q0, lq, k0, lk, b, h, r0, min(lq, r0 + step), hq, hkv, scale,
                              causal, varlen))
    units.sort(key=lambda u: -(u[7] - u[6]) * max(u[3], 1))
    return units


def attention_pooled(q, k, v, scale: float, causal: bool,
                     cu_seqlens_q: Optional[Sequence[int]] = None,
                     cu_seqlens_k: Optional[Sequence[int]] = None, *,
                     workers: Optional[int] = None, heads=None, seqs=None,
                     tmpdir: Optional[str] = None, stats: Optional[dict] = None):
    """``oracle.gqa.attention`` computed by a pool of processes.

    Same arguments, layouts and result as ``attention`` (O and LSE as fp64
    arrays). ``heads`` / ``seqs`` limit the evaluation to those query heads /
    sequences; rows outside them are left at O = 0, LSE = -inf. ``stats``, if
    given, receives the worker count, the wall time and the units run.
    """
    scale = float(np.float32(scale))
    if q.shape[-2] % k.shape[-2] != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    nw = workers or default_workers()
    cq = None if cu_seqlens_q is None else [int(x) for x in cu_seqlens_q]
    ck = None if cu_seqlens_k is None else [int(x) for x in cu_seqlens_k]
    units = _units(tuple(q.shape), tuple(k.shape), scale, causal, cq, ck, heads, seqs)
    if cq is None:
        o_shape = tuple(q.shape[:-1]) + (v.shape[-1],)
        lse_shape = (q.shape[0], q.shape[2], q.shape[1])
    else:
        o_shape = tuple(q.shape[:-1]) + (v.shape[-1],)
        lse_shape = (q.shape[0], q.shape[1])
    d = tempfile.mkdtemp(prefix="gqa_oracle_", dir=tmpdir)
    try:
        paths = {n: _stage(x, os.path.join(d, n + ".npy")) for n, x in (("q", q), ("k", k), ("v", v))}
        paths["o"] = os.path.join(d, "o.npy")
        paths["lse"] = os.path.join(d, "lse.npy")
        np.lib.format.open_memmap(paths["o"], mode="w+", dtype=np.float64, shape=o_shape)[...] = 0.0
        np.lib.format.open_memmap(paths["lse"], mode="w+", dtype=np.float64,
                                  shape=lse_shape)[...] = -np.inf
        t0 = time.perf_counter()
        saved = {key: os.environ.get(key) for key in
                 ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
        for key in saved:
            os.environ[key] = "1"
        try:
            # A worker that dies makes the executor raise (BrokenProcessPool)
            # instead of being replaced, so a failure cannot loop.
            with cf.ProcessPoolExecutor(nw, mp_context=mp.get_context("spawn"),
                                        initializer=_init_worker, initargs=(paths,)) as ex:
                futs = [ex.submit(_run_unit, u) for u in units]
                pairs = sum(f.result() for f in cf.as_completed(futs))
        finally:
            for key, val in saved.items():
                if val is None:
                    os.environ.pop(key, None)
                else:
                    os.environ[key] = val
        wall = time.perf_counter() - t0
        out = np.array(np.load(paths["o"], mmap_mode="r"))
        lse = np.array(np.load(paths["lse"], mmap_mode="r"))
    finally:
        shutil.rmtree(d, ignore_errors=True)
    if stats is not None:
        stats.update(workers=nw, wall_s=wall, units=len(units), score_pairs=pairs)
    return out, lse
