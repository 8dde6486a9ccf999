#!/usr/bin/env python3
"""Benchmark of the fused GQA attention forward / split-KV decode on one MI355X.

Default run (N = 1): the largest single-GPU workload, the packed
variable-length causal GQA batch (48 query / 12 K/V heads, d 128, 32
sequences of 128-4096 tokens, T = 77,493, bf16) through ``gqa_attn_fwd``; one
step = one forward over the whole packed batch with inputs already resident
in HBM (2.4 GB per launch, far above the 256 MB Infinity Cache).

Printed: ONE JSON line with the metric, the dominant kernel's roofline
(algorithmic flops or bytes per launch / launch time from HIP events on the
launch stream; median and minimum of single launches too), the CPU oracle
timed on a bounded sample as a process pool (rank 0, N = 1) and, under
"extra", the other workloads (8192-token causal GQA prefill, the BERT-base
encoder, split-KV decode at num_splits 1/2/4/8, tiny fp32,
the backward pass on the encoder, prefill and varlen workloads, and decode over
general caches: ragged paged bf16 and fp8, sliding window; the fp8-input
forward on the prefill and encoder shapes).

Other modes (each prints its own table and exits): --workload W (any named
workload as the main line), --pass backward, --split-sweep (decode split
counts over a grid of caches), --length-sweep (forward and backward against
sequence length), --tile-timeline (per-row-tile forward timeline on the probe
build), --summarize-counters DIR (HBM bytes from rocprofv3 counter runs).

Flop count: 4 * d per visible (query, key) pair per query head (two products,
multiply-add = 2 flops); the backward counts 10 * d (five products). Decode bytes: the K and V cache bytes read,
2 * B * Sk * Hkv * d * 2; for a general cache, the visible keys of every
sequence x Hkv x d x element size x 2.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E bandwidth (published)
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix peak (published)
# The fp8-input forward runs half of its algorithmic flops (S = Q K^T) on the
# fp8 matrix cores and half (O = P V, P in bf16) on the bf16 ones: its peak is
# the rate at which that mix could run, 1 / (0.5 / 5000 + 0.5 / 2500).
PEAK_FP8_FWD_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
METRIC = "fwd attention TFLOP/s (% MFMA peak); decode KV GB/s (% HBM peak)"


def fwd_flops(lq: int, lk: int, hq: int, d: int, causal: bool) -> int:
    """Algorithmic flops of one sequence (4 d per visible pair per query head)."""
    if not causal:
        return 4 * d * hq * lq * lk
    shift = lk - lq
    pairs = 0
    # visible keys of row i: min(lk, max(0, i + 1 + shift))
    lo = max(0, -shift)            # first row with >= 1 visible key
    hi = min(lq, lk - shift)       # rows before hi see fewer than lk keys
    if hi > lo:
        a, b = lo + 1 + shift, hi + shift  # arithmetic series of visible counts
        pairs += (a + b) * (hi - lo) // 2
    pairs += max(0, lq - max(hi, lo)) * lk if lk > 0 else 0
    return 4 * d * hq * pairs


def source_digest(files) -> str:
    """Digest of the kernel sources' code: comments and blank lines are left
    out, so a comment edit does not void counters taken on the same code."""
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())
        h.update(code.encode())
    return h.hexdigest()[:16]


_FWD_SOURCES = ["gqa_attention_amd/csrc/fwd_bf16.hip", "gqa_attention_amd/csrc/device_util.h",
                "gqa_attention_amd/csrc/params.h", "gqa_attention_amd/csrc/fastdiv.h"]
KERNEL_SOURCES = {
    "fwd_bf16": _FWD_SOURCES,
    "fwd_fp8": _FWD_SOURCES,
    "decode_bf16": ["gqa_attention_amd/csrc/decode_bf16.hip",
                    "gqa_attention_amd/csrc/device_util.h", "gqa_attention_amd/csrc/params.h"],
}


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel}:{workload}")
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_digest") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


def run_timed(torch, step, steps, warmup, warm_seconds=0.0, timed_seconds=None):
    """W untimed steps, then exactly K timed steps between two synchronisations.

    Two HIP events on the launch stream (torch's current stream, which the
    binding passes to the library) bracket the K launches; their elapsed time
    / K is the average launch duration. Returns (wall seconds, average ms, K).

    The secondary workloads pass warm_seconds (keep warming up until the GPU
    clocks have ramped: about 20 ms of back-to-back launches on MI355X) and
    timed_seconds (K sized to about that much GPU time); the headline line
    uses exactly the W and K it is given.
    """
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    i = warmup
    if warm_seconds > 0:
        t0, n0 = time.perf_counter(), i
        while time.perf_counter() - t0 < warm_seconds:
            for _ in range(4):
                step(i)
                i += 1
            torch.cuda.synchronize()
        per = (time.perf_counter() - t0) / (i - n0)
        if timed_seconds:
            steps = max(10, min(5000, math.ceil(timed_seconds / per)))
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for j in range(steps):
        step(i + j)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / steps, steps


def single_launches(torch, step, n, first=0):
    """n back-to-back launches with an event between consecutive ones (after
    the timed region): median and minimum single-launch time in ms."""
    import statistics
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record()
    for j in range(n):
        step(first + j)
        ev[j + 1].record()
    torch.cuda.synchronize()
    ts = [ev[j].elapsed_time(ev[j + 1]) for j in range(n)]
    return statistics.median(ts), min(ts)


def to_device(torch, w, sets):
    import gqa_inputs  # noqa: F401
    out = []
    for s in range(sets):
        if s == 0:
            q, k, v = w.q, w.k, w.v
        else:  # further sets: same distribution, different draws
            g = torch.Generator().manual_seed(10_000 + s)
            q = torch.randn(w.q.shape, generator=g).to(w.q.dtype)
            k = torch.randn(w.k.shape, generator=g).to(w.k.dtype)
            v = torch.randn(w.v.shape, generator=g).to(w.v.dtype)
        out.append((q.cuda(), k.cuda(), v.cuda()))
    return out


def bench_fwd(torch, ga, w, steps, warmup, sets, singles=0, **warm):
    dev_sets = to_device(torch, w, sets)
    cq = w.cu_seqlens_q.cuda() if w.varlen else None
    ck = w.cu_seqlens_k.cuda() if w.varlen else None
    out_dt = torch.bfloat16 if w.fp8_scales is not None else w.q.dtype
    outs = [(torch.empty(q.shape, dtype=out_dt, device="cuda"), None) for q, _, _ in dev_sets]
    lses = []
    for q, _, _ in dev_sets:
        shape = (q.shape[0], q.shape[1]) if w.varlen else (q.shape[0], q.shape[2], q.shape[1])
        lses.append(torch.empty(shape, dtype=torch.float32, device="cuda"))

    # Arguments are checked and marshalled once per input set (ga.FwdPlan);
    # each step re-issues the same gqa_attn_fwd call.
    plans = []
    for j, (q, k, v) in enumerate(dev_sets):
        if w.varlen:
            plans.append(ga.FwdPlan(q, k, v, causal=w.causal, scale=w.scale, cu_seqlens_q=cq,
                                    cu_seqlens_k=ck, max_seqlen_q=w.max_seqlen_q,
                                    max_seqlen_k=w.max_seqlen_k, out=outs[j][0], lse=lses[j],
                                    fp8_scales=w.fp8_scales))
        else:
            plans.append(ga.FwdPlan(q, k, v, causal=w.causal, scale=w.scale, out=outs[j][0],
                                    lse=lses[j], fp8_scales=w.fp8_scales))

    def step(i):
        plans[i % sets].run()

    wall, avg_ms, steps = run_timed(torch, step, steps, warmup, **warm)
    med_ms = min_ms = None
    if singles:
        med_ms, min_ms = single_launches(torch, step, singles)
    if w.varlen:
        cu = w.cu_seqlens_q.tolist()
        flops = sum(fwd_flops(cu[b + 1] - cu[b], cu[b + 1] - cu[b], w.q.shape[1], w.q.shape[2],
                              w.causal) for b in range(len(cu) - 1))
    else:
        B, S, H, d = w.q.shape
        flops = B * fwd_flops(S, w.k.shape[1], H, d, w.causal)
    return dict(flops=flops, wall=wall, avg_ms=avg_ms, steps=steps, med_ms=med_ms, min_ms=min_ms)


def bench_decode(torch, ga, w, ns, steps, warmup, sets, singles=0, **warm):
    dev_sets = to_device(torch, w, sets)
    B, Hq, d = w.q.shape
    out = torch.empty_like(dev_sets[0][0])
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, ga.decode_workspace_bytes(B, Hq, d, ns)), dtype=torch.uint8,
                     device="cuda")

    plans = [ga.DecodePlan(q, k, v, scale=w.scale, num_splits=ns,
                           workspace=ws if ns > 1 else None, out=out, lse=lse)
             for q, k, v in dev_sets]

    def step(i):
        plans[i % sets].run()

    wall, avg_ms, steps = run_timed(torch, step, steps, warmup, **warm)
    med_ms = min_ms = None
    if singles:
        med_ms, min_ms = single_launches(torch, step, singles)
    kv_bytes = 2 * w.k.numel() * w.k.element_size()
    return dict(bytes=kv_bytes, wall=wall, avg_ms=avg_ms, steps=steps, med_ms=med_ms,
                min_ms=min_ms)


def bench_bwd(torch, ga, w, steps, warmup, **warm):
    """Time gqa_attn_bwd alone (its O and LSE come from one forward first).
    Flops: 10 d per visible (query, key) pair per query head (the five
    products S, dP, dV, dQ, dK)."""
    q, k, v = w.q.cuda(), w.k.cuda(), w.v.cuda()
    kw = dict(causal=w.causal, scale=w.scale)
    if w.varlen:
        kw.update(cu_seqlens_q=w.cu_seqlens_q.cuda(), cu_seqlens_k=w.cu_seqlens_k.cuda(),
                  max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k)
    o, lse = ga.fwd(q, k, v, **kw)
    g = torch.Generator().manual_seed(20_000)
    do = torch.randn(w.q.shape, generator=g).to(w.q.dtype).cuda()
    plan = ga.BwdPlan(q, k, v, o, lse, do, **kw)
    wall, avg_ms, steps = run_timed(torch, lambda i: plan.run(), steps, warmup, **warm)
    flops = fwd_flops_of(w) // 4 * 10
    return dict(flops=flops, wall=wall, avg_ms=avg_ms, steps=steps)


def fwd_flops_of(w) -> int:
    if w.varlen:
        cu = w.cu_seqlens_q.tolist()
        ck = w.cu_seqlens_k.tolist()
        return sum(fwd_flops(cu[b + 1] - cu[b], ck[b + 1] - ck[b], w.q.shape[1], w.q.shape[2],
                             w.causal) for b in range(len(cu) - 1))
    B, sq, hq, d = w.q.shape
    return B * fwd_flops(sq, w.k.shape[1], hq, d, w.causal)


def cache_kv_bytes(wc) -> int:
    """K and V bytes a decode over a general cache must read: the visible keys
    of every sequence x Hkv x d x element size, for K and for V."""
    hkv, d = wc.k_cache.shape[2], wc.k_cache.shape[3]
    n = 0
    for L in wc.lengths():
        lo = 0 if wc.window_left < 0 else max(0, L - 1 - wc.window_left)
        n += L - lo
    return 2 * n * hkv * d * wc.k_cache.element_size()


def bench_decode_ex(torch, ga, wc, ns, steps, warmup, **warm):
    q, k, v = wc.q.cuda(), wc.k_cache.cuda(), wc.v_cache.cuda()
    sl = wc.seqlens.cuda() if wc.seqlens is not None else None
    bt = wc.block_table.cuda() if wc.block_table is not None else None
    plan = ga.DecodeExPlan(q, k, v, seqlens_k=sl, block_table=bt, window_left=wc.window_left,
                           k_scale=wc.k_scale, v_scale=wc.v_scale, scale=wc.scale,
                           num_splits=ns)
    wall, avg_ms, steps = run_timed(torch, lambda i: plan.run(), steps, warmup, **warm)
    return dict(bytes=cache_kv_bytes(wc), wall=wall, avg_ms=avg_ms, steps=steps)


def cpu_baseline(w, frac=0.5):
    """The fp64 oracle as it stands, run as a process pool (one worker per
    core this process may use, capped at 16, BLAS threads 1; oracle.pool) on
    a bounded sample of the same workload: the leading sequences (varlen) or
    batches (fixed length) that hold about `frac` of its work. Reported in the
    metric's unit: algorithmic flops of the sample / wall time."""
    import numpy as np
    from oracle import pool as opool
    if w.varlen:
        cu = w.cu_seqlens_q.tolist()
        ck = w.cu_seqlens_k.tolist()
        work = [(cu[b + 1] - cu[b]) * (ck[b + 1] - ck[b]) for b in range(len(cu) - 1)]
        n, acc = 0, 0
        while n < len(work) and (acc < frac * sum(work) or n == 0):
            acc += work[n]
            n += 1
        q, k, v = w.q[:cu[n]], w.k[:ck[n]], w.v[:ck[n]]
        cq, ckk = cu[:n + 1], ck[:n + 1]
        flops = sum(fwd_flops(cu[b + 1] - cu[b], ck[b + 1] - ck[b], w.q.shape[1], w.q.shape[2],
                              w.causal) for b in range(n))
        what = f"the first {n} of {len(cu) - 1} sequences ({cu[n]} of {cu[-1]} tokens)"
    else:
        B = w.q.shape[0]
        n = max(1, int(round(frac * B)))
        q, k, v = w.q[:n], w.k[:n], w.v[:n]
        cq = ckk = None
        flops = n * fwd_flops(w.q.shape[1], w.k.shape[1], w.q.shape[2], w.q.shape[3], w.causal)
        what = f"the first {n} of {B} batch entries"
    if w.fp8_scales is not None:
        from oracle import fp8_forward as of8
        q, k, v = of8.dequantised(q, k, v, *w.fp8_scales)
    st = {}
    opool.attention_pooled(q, k, v, w.scale, w.causal, cq, ckk, stats=st)
    el = st["wall_s"]
    return {"value": round(flops / el / 1e12, 5), "unit": "TFLOP/s", "cores": int(st["workers"]),
            "kind": "oracle",
            "sample": f"{what}, all {w.q.shape[-2]} heads; fp64 NumPy oracle (S and P "
                      f"materialised, so causal work is done in full) as {st['workers']} "
                      f"processes x 1 BLAS thread, {st['units']} (sequence, head, row block) "
                      f"units, {el:.1f} s wall",
            "affinity_cores": opool.affinity_cores(), "cpu_model": opool.cpu_model(),
            "wall_s": round(el, 2), "sample_gflop": round(flops / 1e9, 3)}


def summarize_counters(pmc_dir: str, out_path: str) -> dict:
    """Turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs into HBM bytes per launch.

    Expects <pmc_dir>/copy_fetch, copy_write (gqa_attention_amd/hbm_probe
    268435456: one copy of 256 MiB read + 256 MiB written, and a 256 MiB read
    stream) and <workload>_fetch, <workload>_write directories (bench.py
    --workload <workload>). Each counter is scaled by the ratio between the
    copy kernel's known bytes and what the same counter reports for it.
    """
    import csv
    import glob
    import statistics

    def read(name):
        files = glob.glob(os.path.join(pmc_dir, name, "*_counter_collection.csv"))
        per_kernel = {}
        for f in files:
            for r in csv.DictReader(open(f)):
                per_kernel.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return per_kernel

    copy_bytes = 268435456
    fetch = read("copy_fetch")
    write = read("copy_write")
    kf = [v for k, v in fetch.items() if k.startswith("copy_kernel")][0]
    kw = [v for k, v in write.items() if k.startswith("copy_kernel")][0]
    scale_fetch = copy_bytes / (statistics.mean(kf) * 1024)
    scale_write = copy_bytes / (statistics.mean(kw) * 1024)
    out = {"_scale": {"fetch_size_bytes_per_kib": scale_fetch * 1024,
                      "write_size_bytes_per_kib": scale_write * 1024,
                      "reference": "copy_kernel of gqa_attention_amd/hbm_probe, 256 MiB read + 256 MiB "
                                   "written per launch"}}
    kernels = {"fwd_bf16_kernel": "fwd_bf16", "decode_bf16_kernel": "decode_bf16"}
    for d in sorted(glob.glob(os.path.join(pmc_dir, "*_fetch"))):
        wl = os.path.basename(d)[:-len("_fetch")]
        if wl == "copy":
            continue
        f, w = read(wl + "_fetch"), read(wl + "_write")
        for kname, vals in f.items():
            tag = next((v for k, v in kernels.items() if k in kname), None)
            # the forward's fp8-input instances: fwd_bf16_kernel<D, causal, varlen, true>
            if tag == "fwd_bf16" and kname.split(">")[0].replace(" ", "").endswith(",true"):
                tag = "fwd_fp8"
            if tag is None or kname not in w:
                continue
            fb = statistics.mean(vals) * 1024 * scale_fetch
            wb = statistics.mean(w[kname]) * 1024 * scale_write
            out[f"{tag}:{WORKLOAD_NAMES[wl]}"] = {
                "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                "bytes_per_launch": round(fb + wb), "kernel": kname[:120],
                "source_digest": source_digest(KERNEL_SOURCES[tag]),
                "command": f"rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -- python3 bench.py "
                           f"--workload {wl} --steps 3 --warmup 1 --no-extra --no-cpu-baseline"}
    with open(out_path, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
    return out


WORKLOAD_NAMES = {
    "llama31_8b_prefill_fp8": "llama31_8b_prefill_fp8_s8192_h32_kv8_d128",
    "bert_base_encoder_fp8": "bert_base_encoder_fp8_b64_s512_h12_d64",
    "bert_base_encoder": "bert_base_encoder_b64_s512_h12_d64",
    "llama31_8b_prefill": "llama31_8b_prefill_s8192_h32_kv8_d128",
    "llama31_8b_decode": "llama31_8b_decode_b64_kv4096_h32_kv8_d128",
    "varlen_packed_causal": "varlen_packed_causal_h48_kv12_d128_n32",
}


def split_sweep(torch, ga):
    """Decode time at num_splits 1, 2, 4, 8, 16 for contiguous bf16 caches
    (Llama heads: 32 query, 8 K/V heads), B 1..128, 512..32768 keys, d 64 and
    128, against the count gqa_attn_decode_num_splits picks. Each time is the
    smallest of three averages over 20 back-to-back launches, after a warm-up
    that lets the clocks ramp. Prints a markdown table and a summary line."""
    Hq, Hkv = 32, 8
    counts = (1, 2, 4, 8, 16)
    rows, worst = [], 1.0
    gen = torch.Generator(device="cuda").manual_seed(0)
    for d in (64, 128):
        for Sk in (512, 2048, 8192, 32768):
            for B in (1, 2, 4, 8, 16, 32, 64, 128):
                q = torch.randn(B, Hq, d, device="cuda", generator=gen).to(torch.bfloat16)
                k = torch.randn(B, Sk, Hkv, d, device="cuda", generator=gen).to(torch.bfloat16)
                v = torch.randn(B, Sk, Hkv, d, device="cuda", generator=gen).to(torch.bfloat16)
                times = {}
                for ns in counts:
                    plan = ga.DecodePlan(q, k, v, num_splits=ns)
                    t_end = time.perf_counter() + 0.03
                    while time.perf_counter() < t_end:
                        plan.run()
                        torch.cuda.synchronize()
                    best = float("inf")
                    for _ in range(3):
                        e0 = torch.cuda.Event(enable_timing=True)
                        e1 = torch.cuda.Event(enable_timing=True)
                        e0.record()
                        for _ in range(20):
                            plan.run()
                        e1.record()
                        torch.cuda.synchronize()
                        best = min(best, e0.elapsed_time(e1) / 20)
                    times[ns] = best
                pick = ga.decode_num_splits(B, Hq, Hkv, d, Sk)
                fastest = min(times, key=times.get)
                ratio = times[fastest] / times[pick]
                worst = min(worst, ratio)
                gbs = 2 * k.numel() * 2 / (times[pick] * 1e-3) / 1e9
                rows.append((d, Sk, B, times, pick, fastest, ratio, gbs))
                del q, k, v
                torch.cuda.empty_cache()
    print("| d | keys | B | " + " | ".join(f"ns={c} µs" for c in counts) +
          " | best | picked | best/picked time | picked GB/s |")
    print("|---" * (len(counts) + 7) + "|")
    for d, Sk, B, times, pick, fastest, ratio, gbs in rows:
        print(f"| {d} | {Sk} | {B} | " + " | ".join(f"{times[c] * 1e3:.1f}" for c in counts) +
              f" | {fastest} | {pick} | {ratio:.3f} | {gbs:.0f} |")
    ratios = [r[6] for r in rows]
    print(json.dumps({"points": len(rows), "picked_is_best": sum(r[4] == r[5] for r in rows),
                      "worst_best_over_picked": round(worst, 4),
                      "median_best_over_picked": round(float(sorted(ratios)[len(ratios) // 2]), 4)}))


def length_sweep(torch, ga, gqa_inputs):
    """Forward (bf16 and fp8 inputs) and backward throughput against sequence
    length: GQA 32 / 8 heads, max(1, 16384 / S) sequences of S tokens, N(0, 1)
    inputs (e4m3 with q/k/v scales 0.5 / 0.25 / 0.5 for fp8), each entry
    timed with HIP events over about 50 ms of back-to-back launches after a
    50 ms warm-up. TFLOP/s of algorithmic work: 4 d per visible (query, key)
    pair and query head for the forward, 10 d for the backward. Prints a
    markdown table."""
    rows = [(1024, True, 128), (4096, True, 128), (8192, True, 128), (32768, True, 128),
            (1024, False, 128), (8192, False, 128), (32768, False, 128),
            (1024, True, 64), (8192, True, 64), (32768, False, 64)]
    warm = dict(warm_seconds=0.05, timed_seconds=0.05)
    print("| S | causal | d | forward bf16 | forward fp8 | backward bf16 |")
    print("|---|---|---|---|---|---|")
    for i, (S, causal, d) in enumerate(rows):
        B = max(1, 16384 // S)
        w = gqa_inputs.fixed(B, 32, 8, S, S, d, seed=40 + i, causal=causal)
        w8 = gqa_inputs.fixed_fp8(B, 32, 8, S, S, d, seed=60 + i, causal=causal, q_scale=0.5,
                                  k_scale=0.25, v_scale=0.5)
        tf = []
        for wk in (w, w8):
            r = bench_fwd(torch, ga, wk, 20, 5, 1, **warm)
            tf.append(r["flops"] / (r["avg_ms"] * 1e-3) / 1e12)
        r = bench_bwd(torch, ga, w, 10, 3, **warm)
        tf.append(r["flops"] / (r["avg_ms"] * 1e-3) / 1e12)
        print(f"| {S} | {'yes' if causal else 'no'} | {d} | {tf[0]:.0f} | {tf[1]:.0f} | {tf[2]:.0f} |",
              flush=True)
        del w, w8
        torch.cuda.empty_cache()


def tile_timeline(torch, ga, gqa_inputs):
    """Where a forward's time goes, per row tile, on the timeline probe build
    (gqa_attention_amd/libgqa_attn_timeline.so: the library with per-tile
    s_memrealtime stamps compiled in). For the encoder, prefill and packed
    varlen workloads: after about 200 ms of back-to-back launches, one launch
    records every row
    tile's start, prologue end (its first K/V tiles and Q have landed and its
    first scores are formed), loop end and end (output stores landed). Prints
    a markdown table: per-tile prologue / loop / epilogue times, key-tile rate,
    the CU time between consecutive tiles, the average number of tiles
    resident per CU, and the idle tail."""
    import ctypes
    import numpy as np

    ga._LIB_PATH = os.path.join(ROOT, "gqa_attention_amd", "libgqa_attn_timeline.so")
    ga._lib = None
    L = ga.lib()
    L.gqa_attn_timeline_buffer.argtypes = [ctypes.c_void_p, ctypes.c_int]
    L.gqa_attn_timeline_buffer.restype = None
    cap = 40000
    buf = torch.zeros(8 * (cap + 1), dtype=torch.int64, device="cuda")
    print("| workload | launch µs (not recording / recording) | tiles | prologue µs | loop µs | "
          "ns per key tile | epilogue µs | µs between tiles on a CU | tiles resident per CU | "
          "idle tail µs (mean / max) |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for w in (gqa_inputs.bert_base_encoder(), gqa_inputs.llama31_8b_prefill(),
              gqa_inputs.varlen_packed_causal_48_12()):
        q, k, v = w.q.cuda(), w.k.cuda(), w.v.cuda()
        kw = dict(causal=w.causal, scale=w.scale)
        if w.varlen:
            kw.update(cu_seqlens_q=w.cu_seqlens_q.cuda(), cu_seqlens_k=w.cu_seqlens_k.cuda(),
                      max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k)
        plan = ga.FwdPlan(q, k, v, **kw)
        plan.run()
        torch.cuda.synchronize()
        t = time.perf_counter()
        plan.run()
        torch.cuda.synchronize()
        # about 200 ms of back-to-back launches, so that the clocks have ramped
        for _ in range(max(20, int(0.2 / max(time.perf_counter() - t, 1e-5)))):
            plan.run()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        plan.run()
        e[1].record()
        buf.zero_()
        L.gqa_attn_timeline_buffer(buf.data_ptr(), cap)
        e[2].record()
        plan.run()
        e[3].record()
        torch.cuda.synchronize()
        L.gqa_attn_timeline_buffer(None, 0)
        plain_us, rec_us = e[0].elapsed_time(e[1]) * 1e3, e[2].elapsed_time(e[3]) * 1e3
        a = buf.cpu().numpy()
        n = min(int(a[0]), cap)
        r = a[8:8 + 8 * n].reshape(n, 8).astype(np.float64) / 100.0  # µs (100 MHz clock)
        t0, t1, t2, t3 = r[:, 0], r[:, 1], r[:, 2], r[:, 3]
        hw = a[8:8 + 8 * n].reshape(n, 8)[:, 4]
        wg = a[8:8 + 8 * n].reshape(n, 8)[:, 6]
        cu = (wg % 8) * 4096 + ((hw >> 8) & 0xFF)  # XCD (round-robin dispatch) + CU within it
        gaps, tails, busy = [], [], 0.0
        for c in np.unique(cu):
            o = np.nonzero(cu == c)[0]
            o = o[np.argsort(t0[o])]
            busy += (t3[o] - t0[o]).sum()
            g = t0[o[1:]] - t3[o[:-1]]
            gaps.extend(g[g > 0].tolist())
            tails.append(t3.max() - t3[o[-1]])
        span = t3.max() - t0.min()
        keyt = r[:, 5] * 100.0
        print(f"| {w.name} | {plain_us:.1f} / {rec_us:.1f} | {n} | {np.mean(t1 - t0):.2f} | {np.mean(t2 - t1):.2f} | "
              f"{np.sum(t2 - t1) / np.sum(keyt) * 1e3:.0f} | {np.mean(t3 - t2):.2f} | "
              f"{np.mean(gaps) if gaps else 0.0:.2f} | {busy / len(np.unique(cu)) / span:.2f} | "
              f"{np.mean(tails):.1f} / {np.max(tails):.1f} |", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # MI355X clocks ramp over the first ~20 ms of back-to-back work (launches
    # there run up to 25 % slower): after the W warm-up steps the main line
    # keeps warming up until --warm-ms of launches have run, then times
    # exactly K steps.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warm-ms", type=float, default=100.0)
    ap.add_argument("--singles", type=int, default=50,
                    help="single launches timed one by one after the K steps (median, min)")
    ap.add_argument("--workload", default="varlen_packed_causal",
                    choices=["bert_base_encoder", "llama31_8b_prefill", "llama31_8b_decode",
                             "varlen_packed_causal", "tiny_causal_gqa_fp32",
                             "decode_ragged_paged", "decode_ragged_paged_fp8",
                             "decode_sliding_window", "llama31_8b_prefill_fp8",
                             "bert_base_encoder_fp8"])
    ap.add_argument("--num-splits", type=int, default=1, help="decode workload only")
    ap.add_argument("--pass", dest="pass_", choices=["forward", "backward"], default="forward",
                    help="backward: time gqa_attn_bwd on a forward workload (prints that line only)")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-counters", metavar="PMC_DIR",
                    help="write profiles/hbm_traffic.json from rocprofv3 counter runs and exit")
    ap.add_argument("--tile-timeline", action="store_true",
                    help="per-row-tile forward timeline on the probe build libgqa_attn_timeline.so "
                         "(markdown table) and exit")
    ap.add_argument("--length-sweep", action="store_true",
                    help="forward (bf16, fp8) and backward TFLOP/s against sequence length "
                         "(markdown table) and exit")
    ap.add_argument("--split-sweep", action="store_true",
                    help="time gqa_attn_decode at every split count over a grid of contiguous "
                         "bf16 caches, compare with gqa_attn_decode_num_splits (markdown table) "
                         "and exit")
    args = ap.parse_args()

    if args.summarize_counters:
        res = summarize_counters(args.summarize_counters,
                                 os.path.join(ROOT, "profiles", "hbm_traffic.json"))
        print(json.dumps(res, indent=1))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gqa_attention_amd as ga
    import gqa_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ga.lib()  # fail loudly if the HIP library is missing

    if args.split_sweep:
        split_sweep(torch, ga)
        return
    if args.tile_timeline:
        tile_timeline(torch, ga, gqa_inputs)
        return
    if args.length_sweep:
        length_sweep(torch, ga, gqa_inputs)
        return

    # secondary workloads: warm up until the clocks have ramped, then time
    # about 20 ms of launches
    ramp = dict(warm_seconds=0.05, timed_seconds=0.02)

    def fwd_kind(w):
        """(kernel, dtype label, peak TFLOP/s, bound) of a forward workload."""
        if w.fp8_scales is not None:
            return "fwd_fp8", "fp8_e4m3", PEAK_FP8_FWD_TFLOPS, "mfma"
        if w.q.dtype == torch.bfloat16:
            return "fwd_bf16", "bf16", PEAK_BF16_TFLOPS, "mfma"
        return "fwd_f32", "f32", PEAK_FP32_TFLOPS, "alu"

    def fwd_entry(name, w, steps, warmup, sets, **warm):
        r = bench_fwd(torch, ga, w, steps, warmup, sets, singles=20, **warm)
        tf = r["flops"] / (r["avg_ms"] * 1e-3) / 1e12
        kernel, _, peak, _ = fwd_kind(w)
        return r, {"workload": w.name, "kernel": kernel, "tflops": round(tf, 2),
                   "peak": round(peak, 1), "frac_peak": round(tf / peak, 4),
                   "ms_per_launch": round(r["avg_ms"], 5),
                   "ms_per_launch_median": round(r["med_ms"], 5),
                   "ms_per_launch_min": round(r["min_ms"], 5),
                   "gflop": round(r["flops"] / 1e9, 3)}

    loaders = {
        "bert_base_encoder": gqa_inputs.bert_base_encoder,
        "llama31_8b_prefill": gqa_inputs.llama31_8b_prefill,
        "varlen_packed_causal": gqa_inputs.varlen_packed_causal_48_12,
        "tiny_causal_gqa_fp32": gqa_inputs.tiny_causal_gqa_fp32,
        "llama31_8b_decode": gqa_inputs.llama31_8b_decode,
        "llama31_8b_prefill_fp8": gqa_inputs.llama31_8b_prefill_fp8,
        "bert_base_encoder_fp8": gqa_inputs.bert_base_encoder_fp8,
    }
    sets_for = {"bert_base_encoder": 3, "bert_base_encoder_fp8": 3, "llama31_8b_decode": 2}

    def cache_entry(wc, ns, steps, warmup, **warm):
        rc = bench_decode_ex(torch, ga, wc, ns, steps, warmup, **warm)
        gbs = rc["bytes"] / (rc["avg_ms"] * 1e-3) / 1e9
        kern = "decode_bf16" + ("+combine" if ns > 1 else "")
        return rc, {"workload": wc.name, "kernel": kern, "num_splits": ns,
                    "kv_gbs": round(gbs, 1), "frac_peak": round(gbs / PEAK_HBM_GBS, 4),
                    "ms_per_call": round(rc["avg_ms"], 5), "kv_bytes": rc["bytes"]}

    if args.pass_ == "backward":
        w = loaders[args.workload]()
        if w.decode or w.q.dtype != torch.bfloat16 or w.fp8_scales is not None:
            print("the backward pass is timed on the bf16 forward workloads", file=sys.stderr)
            sys.exit(2)
        r = bench_bwd(torch, ga, w, args.steps, args.warmup)
        tf = r["flops"] / (r["avg_ms"] * 1e-3) / 1e12
        line = {"metric": METRIC, "value": round(r["flops"] * args.steps / r["wall"] / 1e12, 3),
                "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": round(r["wall"] * 1e3 / args.steps, 5), "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                "config": {"workload": w.name, "pass": "backward",
                           "gflop_per_step": round(r["flops"] / 1e9, 3)},
                "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                             "traffic": None, "kernel": "bwd (dq + dkdv)",
                             "launch_ms": round(r["avg_ms"], 5)}}
        print(json.dumps(line))
        return

    if args.workload in gqa_inputs.CACHE_NAMED:
        w = gqa_inputs.CACHE_NAMED[args.workload]()
        r, e = cache_entry(w, args.num_splits, args.steps, args.warmup,
                           warm_seconds=args.warm_ms * 1e-3)
        gbs = e["kv_gbs"]
        line = {"metric": METRIC, "value": round(r["bytes"] * args.steps / r["wall"] / 1e9, 3),
                "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": round(r["wall"] * 1e3 / args.steps, 5),
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                "dtype": "fp8_e4m3" if w.fp8 else "bf16", "data": "synthetic",
                "config": {"workload": w.name, "B": w.batch, "Hq": w.q.shape[1],
                           "Hkv": w.k_cache.shape[2], "d": w.q.shape[2],
                           "block_size": w.block_size, "window_left": w.window_left,
                           "num_splits": args.num_splits, "kv_bytes": r["bytes"]},
                "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                             "traffic": measured_traffic("decode_bf16", w.name),
                             "kernel": e["kernel"], "launch_ms": e["ms_per_call"]}}
        print(json.dumps(line))
        return

    w = loaders[args.workload]()
    sets = sets_for.get(args.workload, 1)
    if w.decode:
        r = bench_decode(torch, ga, w, args.num_splits, args.steps, args.warmup, sets,
                         singles=args.singles, warm_seconds=args.warm_ms * 1e-3)
        gbs = r["bytes"] / (r["avg_ms"] * 1e-3) / 1e9
        value = r["bytes"] * args.steps / r["wall"] / 1e9
        unit, dtype_s = "GB/s", "bf16"
        kernel = "decode_bf16"
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
        traffic = measured_traffic(kernel, w.name)
        config = {"workload": w.name, "B": w.q.shape[0], "Hq": w.q.shape[1], "Hkv": w.k.shape[2],
                  "Sk": w.k.shape[1], "d": w.q.shape[2], "num_splits": args.num_splits,
                  "kv_bytes": r["bytes"], "input_sets_rotated": sets}
    else:
        r = bench_fwd(torch, ga, w, args.steps, args.warmup, sets, singles=args.singles,
                      warm_seconds=args.warm_ms * 1e-3)
        tf = r["flops"] / (r["avg_ms"] * 1e-3) / 1e12
        value = r["flops"] * args.steps / r["wall"] / 1e12
        unit = "TFLOP/s"
        kernel, dtype_s, peak, bound = fwd_kind(w)
        roof = {"bound": bound, "achieved": round(tf, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(tf / peak, 4)}
        traffic = measured_traffic(kernel, w.name) if bound == "mfma" else None
        if w.varlen:
            config = {"workload": w.name, "sequences": len(w.cu_seqlens_q) - 1,
                      "total_tokens": w.q.shape[0], "Hq": w.q.shape[1], "Hkv": w.k.shape[1],
                      "d": w.q.shape[2], "causal": w.causal}
        else:
            config = {"workload": w.name, "B": w.q.shape[0], "Sq": w.q.shape[1],
                      "Sk": w.k.shape[1], "Hq": w.q.shape[2], "Hkv": w.k.shape[2],
                      "d": w.q.shape[3], "causal": w.causal}
        config["gflop_per_step"] = round(r["flops"] / 1e9, 3)
        config["input_sets_rotated"] = sets
    roof["traffic"] = traffic
    roof["kernel"] = kernel
    roof["launch_ms"] = round(r["avg_ms"], 5)
    if r.get("med_ms"):
        roof["launch_ms_median"] = round(r["med_ms"], 5)
        roof["launch_ms_min"] = round(r["min_ms"], 5)
        roof["single_launches"] = args.singles
    roof["warmup_gpu_ms"] = args.warm_ms

    line = {"metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(r["wall"] * 1e3 / args.steps, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype_s, "data": "synthetic",
            "config": config, "roofline": roof}

    if not args.no_extra:
        extra = []
        for name in ["llama31_8b_prefill", "varlen_packed_causal", "tiny_causal_gqa_fp32",
                     "bert_base_encoder", "llama31_8b_prefill_fp8", "bert_base_encoder_fp8"]:
            if name == args.workload:
                continue
            wx = loaders[name]()
            _, e = fwd_entry(name, wx, 20, 3, sets_for.get(name, 1), **ramp)
            extra.append(e)
            del wx
        if args.workload != "llama31_8b_decode":
            wd = loaders["llama31_8b_decode"]()
            for ns in (1, 2, 4, 8):
                rd = bench_decode(torch, ga, wd, ns, 20, 3, 2, **ramp)
                gbs = rd["bytes"] / (rd["avg_ms"] * 1e-3) / 1e9
                extra.append({"workload": wd.name, "kernel": "decode_bf16+combine" if ns > 1
                              else "decode_bf16", "num_splits": ns, "kv_gbs": round(gbs, 1),
                              "frac_peak": round(gbs / PEAK_HBM_GBS, 4),
                              "ms_per_call": round(rd["avg_ms"], 5)})
            del wd
        for name in ["bert_base_encoder", "llama31_8b_prefill", "varlen_packed_causal"]:
            wb = loaders[name]()
            rb = bench_bwd(torch, ga, wb, 10, 2, **ramp)
            tf = rb["flops"] / (rb["avg_ms"] * 1e-3) / 1e12
            extra.append({"workload": wb.name, "kernel": "bwd (dq + dkdv)",
                          "pass": "backward", "tflops": round(tf, 2),
                          "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                          "ms_per_call": round(rb["avg_ms"], 5),
                          "gflop": round(rb["flops"] / 1e9, 3)})
            del wb
            torch.cuda.empty_cache()
        for cname in sorted(gqa_inputs.CACHE_NAMED):
            wc = gqa_inputs.CACHE_NAMED[cname]()
            rec = ga.decode_num_splits(wc.batch, wc.q.shape[1], wc.k_cache.shape[2],
                                       wc.q.shape[2], wc.max_seqlen_k, wc.window_left,
                                       ragged=wc.seqlens is not None)
            for ns in (1, 2, 4, 8):
                _, e = cache_entry(wc, ns, 20, 3, **ramp)
                e["recommended_num_splits"] = rec
                extra.append(e)
            del wc
            torch.cuda.empty_cache()
        line["extra"] = extra

    if not args.no_cpu_baseline and not w.decode:
        line["cpu_baseline"] = cpu_baseline(w)
        line["cpu_baseline"]["gpu_speedup"] = round(roof["achieved"] / line["cpu_baseline"]["value"], 1)
    elif not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        nb = 0
        while nb < w.q.shape[0] and time.perf_counter() - t0 < 15.0:
            oracle.decode(w.q[nb:nb + 1], w.k[nb:nb + 1], w.v[nb:nb + 1], w.scale)
            nb += 1
        el = time.perf_counter() - t0
        kvb = 2 * w.k[:nb].numel() * w.k.element_size()
        line["cpu_baseline"] = {"value": kvb / el / 1e9, "unit": "GB/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"{nb} of {w.q.shape[0]} sequences, fp64 NumPy, {el:.1f} s"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
