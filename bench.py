#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * prefill: attn_fwd, bf16, B=2, Hq=32, Hkv=8, Sq=Sk=2048, D=128, causal,
    scale 1/sqrt(128) -- causal-effective TFLOP/s (4 * D * admissible pairs);
  * decode: attn_paged_decode, bf16, B=64, Hq=32, Hkv=8, D=128, context
    lengths uniform on [512, 8192], 64-token blocks randomly permuted in one
    pool, num_splits 8 (the split form: 512 (sequence, KV head) groups x 8
    key ranges = 4096 items over persistent per-wave workers, then the merge
    kernel) -- HBM GB/s over the live K/V bytes plus Q, out and the
    block-table entries read.

Inputs are generated (seeded) and resident in device memory before the timed
region.  Kernel durations come from HIP events recorded on the stream the
kernels run on, around each launch inside the timed steps.  ``value`` is the
prefill TFLOP/s; the decode figures ride along under ``decode``.  The CPU
oracle is timed on a bounded sample of the same prefill workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --mode profile [--launches N]   # the bench's steps, for rocprofv3
    python bench.py --mode profile_prefill          # launches for the MFMA counter pass
    python bench.py --mode profile_backward         # backward launches for rocprofv3
    python bench.py --summarize DIR [--last N]      # kernel-trace summary (last N dispatches)
    python bench.py --traffic FETCH WRITE           # HBM bytes per launch from two counter runs
    python bench.py --mfma-util DIR --launches N    # MFMA busy per prefill workload
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOPS (bf16 causal prefill) + paged-decode HBM GB/s, % of roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
KERNEL_SOURCES = ["scaled_dot_product_amd/csrc/fwd_mfma.hip",
                  "scaled_dot_product_amd/csrc/decode.hip",
                  "scaled_dot_product_amd/csrc/device_common.h"]


# ---------------------------------------------------------------- work counts

def admissible_pairs(Sq, Sk, causal, window_left=None, window_right=None) -> int:
    """(query, key) pairs one head may attend to, counted per row from the
    admissible interval [max(0, i'-left), min(Sk-1, i', i'+right)], with the
    bottom-right aligned position i' = i + Sk - Sq."""
    ip = np.arange(Sq, dtype=np.int64) + (Sk - Sq)
    lo = np.zeros(Sq, dtype=np.int64) if window_left is None else np.maximum(0, ip - window_left)
    hi = np.full(Sq, Sk - 1, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, ip)
    if window_right is not None:
        hi = np.minimum(hi, ip + window_right)
    return int(np.maximum(hi - lo + 1, 0).sum())


def prefill_flops(w) -> int:
    return 4 * w.D * w.B * w.Hq * admissible_pairs(w.Sq, w.Sk, w.causal, w.window_left,
                                                   w.window_right)


def decode_bytes(w, lens) -> int:
    """Algorithmic HBM bytes of one decode: live K and V rows once, Q and the
    output once, each live block-table entry once per KV head, the lengths."""
    lens = np.asarray(lens, dtype=np.int64)
    es = 2
    kv = int(lens.sum()) * w.Hkv * w.D * es * 2
    qo = 2 * w.B * w.Hq * w.D * es
    pages = int(((lens + w.block_size - 1) // w.block_size).sum())
    return kv + qo + pages * 4 * w.Hkv + w.B * 4


def sources_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """Per-launch HBM bytes measured with rocprofv3 counters, if they were
    taken on the current kernel sources; {} otherwise."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    vals = {}
    for line in open(TRAFFIC_FILE):
        line = line.strip()
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("sources_sha256_16") != sources_digest():
        return {}
    out = {}
    for key in ("prefill_bytes", "decode_bytes"):
        if key in vals:
            out[key] = float(vals[key])
    return out


# ---------------------------------------------------------------- GPU setup

def setup(torch, sdpa, W, dev):
    wp, wd = W.GQA_CAUSAL_2K, W.PAGED_DECODE
    q, k, v, _ = W.dense_inputs(wp)
    pre = dict(q=q.to(dev), k=k.to(dev), v=v.to(dev))
    pre["out"] = torch.empty_like(pre["q"])
    dq, kp, vp, table, lens, _ = W.paged_inputs(wd)
    dec = dict(q=dq.to(dev), k_pool=kp.to(dev), v_pool=vp.to(dev), block_table=table.to(dev),
               seq_lens=lens.to(dev))
    dec["out"] = torch.empty_like(dec["q"])
    p = sdpa.attn_paged_params(tuple(dq.shape), tuple(kp.shape), table.shape[1], dq.dtype,
                               num_splits=wd.num_splits)
    dec["workspace"] = torch.empty(sdpa.attn_paged_decode_workspace_size(p), dtype=torch.uint8,
                                   device=dev)
    del kp, vp
    return wp, wd, pre, dec, lens.numpy()


def run_dense(sdpa, w, t, alibi, stream):
    sdpa.attn_fwd(t["q"], t["k"], t["v"], alibi, t["out"], softmax_scale=w.scale, causal=w.causal,
                  window_left=w.window_left, window_right=w.window_right, softcap=w.softcap,
                  stream=stream)


def time_launches(torch, run, stream, launches, warm=3):
    """Median per-launch time (seconds) of ``run`` from HIP events recorded
    on ``stream`` around each launch, after ``warm`` untimed launches."""
    for _ in range(warm):
        run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(launches)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e-3


def extra_prefill(torch, sdpa, W, dev, stream, launches=10):
    """The other prefill workloads, timed on their own after the timed steps
    (not part of a step): the long masked 8k prefill (causal + window 4096,
    softcap 50, ALiBi) and the f16 chunked prefill with Sq != Sk."""
    out = {}
    for w in (W.LONG_MASKED_8K, W.CHUNKED_PREFILL):
        q, k, v, alibi = W.dense_inputs(w)
        t = dict(q=q.to(dev), k=k.to(dev), v=v.to(dev))
        t["out"] = torch.empty_like(t["q"])
        al = alibi.to(dev) if alibi is not None else None
        sec = time_launches(torch, lambda: run_dense(sdpa, w, t, al, stream), stream, launches)
        tf = prefill_flops(w) / sec / 1e12
        out[w.name] = {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                       "frac": tf / PEAK_BF16_TFLOPS, "dtype": w.dtype, "work_per_launch": prefill_flops(w),
                       "ms_per_launch": sec * 1e3, "launches": launches}
        del t
    return out


def extra_paged_prefill(torch, sdpa, W, dev, stream, launches=10, block_size=64):
    """The chunked f16 prefill workload run through the paged pool: the same
    q, k, v, with K/V scattered over 64-token blocks in a randomly permuted
    pool, the queries packed with a prefix sum; timed like the other
    workloads, after the timed steps."""
    w = W.CHUNKED_PREFILL
    q, k, v, _ = W.dense_inputs(w)
    nb_seq = (w.Sk + block_size - 1) // block_size
    rng = np.random.default_rng(w.seed + 77)
    perm = torch.from_numpy(rng.permutation(w.B * nb_seq).astype(np.int64))
    table = perm.reshape(w.B, nb_seq).to(torch.int32)
    # pool[block, slot, kv head, d]: block table[b, n] holds keys n*bs .. of sequence b
    kk = k.permute(0, 2, 1, 3).reshape(w.B, nb_seq, block_size, w.Hkv, w.D)
    vv = v.permute(0, 2, 1, 3).reshape(w.B, nb_seq, block_size, w.Hkv, w.D)
    kp = torch.empty((w.B * nb_seq, block_size, w.Hkv, w.D), dtype=k.dtype)
    vp = torch.empty_like(kp)
    kp[perm] = kk.reshape(-1, block_size, w.Hkv, w.D)
    vp[perm] = vv.reshape(-1, block_size, w.Hkv, w.D)
    qp = q.permute(0, 2, 1, 3).reshape(w.B * w.Sq, w.Hq, w.D).contiguous()
    cu = torch.arange(0, (w.B + 1) * w.Sq, w.Sq, dtype=torch.int32)
    lens = torch.full((w.B,), w.Sk, dtype=torch.int32)
    t = dict(q=qp.to(dev), kp=kp.to(dev), vp=vp.to(dev), table=table.to(dev), lens=lens.to(dev),
             cu=cu.to(dev))
    t["out"] = torch.empty_like(t["q"])

    def run():
        sdpa.attn_paged_prefill(t["q"], t["kp"], t["vp"], t["table"], t["lens"], t["cu"], None,
                                t["out"], max_seqlen_q=w.Sq, softmax_scale=w.scale, causal=True,
                                stream=stream)
    sec = time_launches(torch, run, stream, launches)
    tf = prefill_flops(w) / sec / 1e12
    return {w.name + " over the paged pool (64-token blocks)": {
        "bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": tf / PEAK_BF16_TFLOPS, "dtype": w.dtype, "work_per_launch": prefill_flops(w),
        "ms_per_launch": sec * 1e3, "launches": launches}}


def backward_flops(w) -> int:
    """Algorithmic work of the backward: the five matmuls per admissible
    (query, key) pair (S = Q K^T, dP = dO V^T, dV, dQ, dK), 2 D FLOP each."""
    return 10 * w.D * w.B * w.Hq * admissible_pairs(w.Sq, w.Sk, w.causal, w.window_left,
                                                    w.window_right)


def extra_backward(torch, sdpa, W, dev, stream, launches=10):
    """The backward on the 2048-token causal GQA workload, timed on its own
    after the timed steps: attn_bwd (the forward's row statistics recomputed,
    dK/dV, dQ) and attn_bwd_lse (row statistics from a saved forward's output
    and LSE, then the same dK/dV and dQ)."""
    w = W.GQA_CAUSAL_2K
    q, k, v, _ = W.dense_inputs(w)
    do = W.random_dense(w.dtype, w.B, w.Hq, w.Hkv, w.Sq, 1, w.D, 4242, 1.0)[0]
    t = dict(q=q.to(dev), k=k.to(dev), v=v.to(dev), do=do.to(dev))
    t["dq"], t["dk"], t["dv"] = (torch.empty_like(t["q"]), torch.empty_like(t["k"]),
                                 torch.empty_like(t["v"]))
    p = sdpa.attn_fwd_params(tuple(q.shape), tuple(k.shape), q.dtype, softmax_scale=w.scale,
                             causal=True)
    ws = torch.empty(sdpa.attn_bwd_workspace_size(p), dtype=torch.uint8, device=dev)
    t["out"], t["lse"] = sdpa.attn_fwd_lse(t["q"], t["k"], t["v"], None, softmax_scale=w.scale,
                                           causal=True, stream=stream)

    def recompute():
        sdpa.attn_bwd(t["q"], t["k"], t["v"], t["do"], None, softmax_scale=w.scale, causal=True,
                      dq=t["dq"], dk=t["dk"], dv=t["dv"], workspace=ws, stream=stream)

    def saved():
        sdpa.attn_bwd_lse(t["q"], t["k"], t["v"], t["out"], t["lse"], t["do"], None,
                          softmax_scale=w.scale, causal=True, dq=t["dq"], dk=t["dk"], dv=t["dv"],
                          workspace=ws, stream=stream)

    out = {}
    for label, run, kernels in (
            (w.name, recompute, "forward statistics + bwd_dkdv_kernel + bwd_dq_kernel"),
            (w.name + " (from the saved forward)", saved,
             "bwd_rowstats_kernel + bwd_dkdv_kernel + bwd_dq_kernel")):
        sec = time_launches(torch, run, stream, launches)
        tf = backward_flops(w) / sec / 1e12
        out[label] = {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                      "frac": tf / PEAK_BF16_TFLOPS, "dtype": w.dtype,
                      "work_per_launch": backward_flops(w), "ms_per_launch": sec * 1e3,
                      "launches": launches, "kernels": kernels}
    return out


def run_prefill(sdpa, wp, pre, stream):
    sdpa.attn_fwd(pre["q"], pre["k"], pre["v"], None, pre["out"], softmax_scale=wp.scale,
                  causal=wp.causal, stream=stream)


def run_decode(sdpa, wd, dec, stream):
    sdpa.attn_paged_decode(dec["q"], dec["k_pool"], dec["v_pool"], dec["block_table"],
                           dec["seq_lens"], None, dec["out"], softmax_scale=wd.scale,
                           num_splits=wd.num_splits, workspace=dec["workspace"], stream=stream)


DECODE_SPLIT_USED = ("split form: each (sequence, KV head) group in 8 key ranges, the 4096 items "
                     "streamed by persistent per-wave workers, the partials combined by the merge kernel")


def clock_warm(torch, step, seconds):
    """Runs ``step`` untimed until ``seconds`` of wall time have passed (at
    least once), so that the timed steps see the sustained clock rather than
    the ramp from idle; returns (seconds spent, steps run)."""
    if seconds <= 0:
        return 0.0, 0
    t0, n = time.perf_counter(), 0
    while True:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return time.perf_counter() - t0, n


def host_overhead(torch, sdpa, W, dev, wd, dec, calls=200):
    """Per-call cost of a launch that the caller waits for, in three modes:
    eager (the binding marshals the arguments and launches, host + kernel),
    HIP graph replay of the same call (kernel only, no host marshalling) and
    the binding's prepared plan (one C call), all as
    wall time per call with a synchronisation after each call; and the
    kernel's own median event time.  For the paged decode workload, the
    chunked f16 prefill (512 queries, a short prefill), and a small decode
    (4 sequences of 1024 tokens, the same heads and pool layout) whose kernel
    is short enough for the host cost to matter."""
    w = W.CHUNKED_PREFILL
    q, k, v, _ = W.dense_inputs(w)
    t = dict(q=q.to(dev), k=k.to(dev), v=v.to(dev))
    t["out"] = torch.empty_like(t["q"])
    ws = W.Paged("paged_decode_bf16_b4_h32x8_d128_ctx1024_bs64", "bf16", 4, 32, 8, 128, 64, 1024, 1024,
                 8, 16, seed=1006)
    sq, skp, svp, stab, slens, _ = W.paged_inputs(ws)
    small = dict(q=sq.to(dev), k_pool=skp.to(dev), v_pool=svp.to(dev), block_table=stab.to(dev),
                 seq_lens=slens.to(dev))
    small["out"] = torch.empty_like(small["q"])
    sp = sdpa.attn_paged_params(tuple(sq.shape), tuple(skp.shape), stab.shape[1], sq.dtype,
                                num_splits=ws.num_splits)
    small["workspace"] = torch.empty(max(1, sdpa.attn_paged_decode_workspace_size(sp)), dtype=torch.uint8,
                                     device=dev)
    def decode_plan(wk, d, s):
        return sdpa.PagedDecodePlan(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"],
                                    None, d["out"], softmax_scale=wk.scale, num_splits=wk.num_splits,
                                    workspace=d["workspace"], stream=s)
    cases = {
        W.PAGED_DECODE.name: (lambda s: run_decode(sdpa, wd, dec, s), lambda s: decode_plan(wd, dec, s)),
        w.name: (lambda s: run_dense(sdpa, w, t, None, s),
                 lambda s: sdpa.AttnFwdPlan(t["q"], t["k"], t["v"], None, t["out"], softmax_scale=w.scale,
                                            causal=w.causal, stream=s)),
        ws.name: (lambda s: run_decode(sdpa, ws, small, s), lambda s: decode_plan(ws, small, s)),
    }
    res = {}
    for name, (fn, make_plan) in cases.items():
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                fn(side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(torch.cuda.current_stream())
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        kern = []
        for _ in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(stream)
            e1.record(stream)
            torch.cuda.synchronize()
            kern.append(e0.elapsed_time(e1) * 1e3)
        plan = make_plan(stream)
        modes = {}
        for mode, call in (("eager", lambda: fn(stream)), ("graph", g.replay), ("plan", plan.run)):
            for _ in range(10):
                call()
                torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(calls):
                call()
                torch.cuda.synchronize()
            modes[mode] = (time.perf_counter() - t0) / calls * 1e6
        res[name] = {"kernel_us": float(np.median(kern)), "eager_us_per_call": modes["eager"],
                     "graph_us_per_call": modes["graph"], "plan_us_per_call": modes["plan"],
                     "note": "wall time per call with a synchronisation after each call; plan = the "
                             "binding's prepared call (checks and marshalling done once)"}
        del g, plan
    del t, small
    return res


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(W, budget_s: float):
    """The oracle, as it stands, on whole (batch, head) slices of the prefill
    workload, cycling over them until about ``budget_s`` seconds of CPU work
    have been spent (at least one slice)."""
    import oracle
    affinity = len(os.sched_getaffinity(0))
    # the host cores this process may use, capped by the thread count the
    # environment grants it (a shared host sets OMP_NUM_THREADS to its share)
    threads = min(affinity, int(os.environ.get("OMP_NUM_THREADS", affinity) or affinity))
    limiter = None
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=threads)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass
    w = W.GQA_CAUSAL_2K
    q, k, v, _ = W.dense_inputs(w)
    q64, k64, v64 = W.to_f64(q), W.to_f64(k), W.to_f64(v)
    pairs = admissible_pairs(w.Sq, w.Sk, w.causal)
    heads, t0 = 0, time.perf_counter()
    order = [(b, h) for h in range(w.Hq) for b in range(w.B)]
    while True:
        b, h = order[heads % len(order)]
        g = oracle.kv_head_of(h, w.Hq, w.Hkv)
        oracle.sdpa_naive_f64(q64[b:b + 1, h:h + 1], k64[b:b + 1, g:g + 1], v64[b:b + 1, g:g + 1],
                              scale=w.scale, causal=True)
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister()
    flops = 4 * w.D * pairs * heads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "affinity_cpus": affinity, "kind": "oracle",
            "sample": f"{heads} (batch, head) slices of the prefill workload, cycling over its "
                      f"{len(order)} (all {w.Sq} rows each), float64 NumPy, {dt:.1f} s"}


# ---------------------------------------------------------------- modes

def bench(args):
    import torch
    import scaled_dot_product_amd as sdpa
    import workloads as W
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU (cuda:0)")
    dev = torch.device("cuda:0")
    sdpa.library()
    wp, wd, pre, dec, lens = setup(torch, sdpa, W, dev)
    stream = torch.cuda.current_stream(dev)
    warm_s, warm_steps = clock_warm(torch, lambda: (run_prefill(sdpa, wp, pre, stream),
                                                    run_decode(sdpa, wd, dec, stream)), args.clock_warm)
    for _ in range(args.warmup):
        run_prefill(sdpa, wp, pre, stream)
        run_decode(sdpa, wd, dec, stream)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        run_prefill(sdpa, wp, pre, stream)
        ev[i][1].record(stream)
        run_decode(sdpa, wd, dec, stream)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # median of the per-launch event times (kernel time on the launch stream)
    t_pre = float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
    t_dec = float(np.median([e[1].elapsed_time(e[2]) for e in ev])) * 1e-3

    flops = prefill_flops(wp)
    nbytes = decode_bytes(wd, lens)
    tflops = flops / t_pre / 1e12
    gbs = nbytes / t_dec / 1e9
    traffic = read_traffic()
    roof_pre = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / PEAK_BF16_TFLOPS, "traffic": traffic.get("prefill_bytes"),
                "kernel": "fwd_mfma_kernel<bf16, D=128, causal>",
                "work_per_launch": flops, "ms_per_launch": t_pre * 1e3}
    roof_dec = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS, "traffic": traffic.get("decode_bytes"),
                "kernel": "decode_stream_kernel<bf16, D=128, split form> + decode_merge_kernel "
                          "(4096 items: 512 groups x 8 splits)",
                "work_per_launch": nbytes, "ms_per_launch": t_dec * 1e3}
    dominant = roof_pre if t_pre >= t_dec else roof_dec
    result = {
        "metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 inputs; uniform context lengths)",
        "config": {"workload": f"{wp.name} + {wd.name}",
                   "prefill": {"B": wp.B, "Hq": wp.Hq, "Hkv": wp.Hkv, "Sq": wp.Sq, "Sk": wp.Sk,
                               "D": wp.D, "causal": wp.causal},
                   "decode": {"B": wd.B, "Hq": wd.Hq, "Hkv": wd.Hkv, "D": wd.D,
                              "block_size": wd.block_size, "ctx": [wd.ctx_lo, wd.ctx_hi],
                              "num_splits_arg": wd.num_splits, "split_used": DECODE_SPLIT_USED,
                              "live_tokens": int(lens.sum())}},
        "timing": {"statistic": "median of per-launch HIP event times on the launch stream",
                   "clock_warm_s": round(warm_s, 3), "clock_warm_steps": warm_steps},
        "decode": {"value": gbs, "unit": "GB/s", "frac_of_hbm_peak": gbs / PEAK_HBM_GBS,
                   "ms": t_dec * 1e3},
        "roofline": dominant,
        "rooflines": {"prefill": roof_pre, "decode": roof_dec},
    }
    if not args.no_extra:
        result["host_overhead"] = host_overhead(torch, sdpa, W, dev, wd, dec)
        result["other_prefill"] = extra_prefill(torch, sdpa, W, dev, stream)
        result["other_prefill"].update(extra_paged_prefill(torch, sdpa, W, dev, stream))
        result["backward"] = extra_backward(torch, sdpa, W, dev, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(W, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def profile(args):
    """Fixed launches for rocprofv3 in the bench's own order: the same clock
    warm-up and warm-up steps, then ``--launches`` steps of (prefill, paged
    decode), then a plain 256 MiB float32 copy kernel (read N, write N) that
    calibrates the HBM byte counters.  ``--summarize DIR --last N`` averages
    only the last N dispatches of each kernel, i.e. the timed steps."""
    import torch
    import scaled_dot_product_amd as sdpa
    import workloads as W
    dev = torch.device("cuda:0")
    wp, wd, pre, dec, lens = setup(torch, sdpa, W, dev)
    stream = torch.cuda.current_stream(dev)
    src = torch.randn(64 * 1024 * 1024, device=dev)
    dst = torch.empty_like(src)

    def step():
        run_prefill(sdpa, wp, pre, stream)
        run_decode(sdpa, wd, dec, stream)
    warm_s, warm_steps = clock_warm(torch, step, args.clock_warm)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for _ in range(args.launches):
        step()
    for _ in range(args.launches):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"profile_launches": args.launches, "clock_warm_steps": warm_steps,
                      "warmup_steps": args.warmup, "prefill_flops": prefill_flops(wp),
                      "decode_bytes": decode_bytes(wd, lens), "copy_bytes_each_way": src.numel() * 4,
                      "sources_sha256_16": sources_digest()}), flush=True)


def profile_backward(args):
    """Fixed launches on the 2048-token causal GQA workload for rocprofv3:
    attn_bwd (the forward's row statistics, dK/dV, dQ), then one attn_fwd_lse
    and attn_bwd_lse from its saved output (row statistics kernel, dK/dV, dQ)."""
    import torch
    import scaled_dot_product_amd as sdpa
    import workloads as W
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    w = W.GQA_CAUSAL_2K
    q, k, v, _ = W.dense_inputs(w)
    do = W.random_dense(w.dtype, w.B, w.Hq, w.Hkv, w.Sq, 1, w.D, 4242, 1.0)[0]
    q, k, v, do = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    for _ in range(2 + args.launches):
        sdpa.attn_bwd(q, k, v, do, None, softmax_scale=w.scale, causal=True, stream=stream)
    out, lse = sdpa.attn_fwd_lse(q, k, v, None, softmax_scale=w.scale, causal=True, stream=stream)
    for _ in range(2 + args.launches):
        sdpa.attn_bwd_lse(q, k, v, out, lse, do, None, softmax_scale=w.scale, causal=True,
                          stream=stream)
    torch.cuda.synchronize()
    print(json.dumps({"profile_launches": args.launches, "backward_flops": backward_flops(w)}),
          flush=True)


PREFILL_CONFIGS = ("GQA_CAUSAL_2K", "LONG_MASKED_8K", "CHUNKED_PREFILL")


def profile_prefill(args):
    """Fixed launches for the MFMA-utilisation counter pass: the 2048-token
    causal GQA prefill as the bench times it (clock warm-up, then
    ``--launches`` steps of prefill + paged decode), then 2 + ``--launches``
    launches each of the long masked 8192-token prefill and the chunked f16
    prefill."""
    import torch
    import scaled_dot_product_amd as sdpa
    import workloads as W
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    wp, wd, pre, dec, lens = setup(torch, sdpa, W, dev)

    def step():
        run_prefill(sdpa, wp, pre, stream)
        run_decode(sdpa, wd, dec, stream)
    clock_warm(torch, step, args.clock_warm)
    torch.cuda.synchronize()
    for _ in range(args.launches):
        step()
    torch.cuda.synchronize()
    del pre, dec
    for name in PREFILL_CONFIGS[1:]:
        w = getattr(W, name)
        q, k, v, alibi = W.dense_inputs(w)
        t = dict(q=q.to(dev), k=k.to(dev), v=v.to(dev))
        t["out"] = torch.empty_like(t["q"])
        al = alibi.to(dev) if alibi is not None else None
        for _ in range(2 + args.launches):
            run_dense(sdpa, w, t, al, stream)
        torch.cuda.synchronize()
        del t
    print(json.dumps({"profile_launches": args.launches, "workloads": list(PREFILL_CONFIGS)}), flush=True)


def mfma_util(path, launches):
    """MFMA utilisation of each prefill launch class from a rocprofv3 counter
    run of --mode profile_prefill with SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES
    and GRBM_GUI_ACTIVE: busy cycles per SIMD over the kernel's GPU cycles (per
    XCD), and the clock the GPU ran at (GPU cycles over the dispatch time).
    Dispatches are taken from the end of the run: the last 2 + L of the
    chunked prefill, the 2 + L before them of the long masked prefill (the
    first 2 of each skipped as warm-up), and the L timed bench steps' prefills
    before those (L = ``launches``)."""
    import workloads as W
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        sys.exit(f"no rocprofv3 counter output under {path}")
    rows = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if "fwd_mfma_kernel" not in r["Kernel_Name"]:
                    continue
                d = rows.setdefault(int(r["Dispatch_Id"]), {"t": (int(r["End_Timestamp"]) -
                                                                  int(r["Start_Timestamp"])) * 1e-9})
                d[r["Counter_Name"]] = float(r["Counter_Value"])
    ids = sorted(rows)
    L = launches
    n_other = 2 + L
    if len(ids) < L + 2 * n_other:
        sys.exit(f"expected at least {L + 2 * n_other} prefill dispatches, found {len(ids)}")
    groups = {PREFILL_CONFIGS[2]: ids[-n_other:][2:],
              PREFILL_CONFIGS[1]: ids[-2 * n_other:-n_other][2:],
              PREFILL_CONFIGS[0]: ids[-2 * n_other - L:-2 * n_other]}
    simds, xcds = 1024, 8
    print("# commands (from the repository root, on one MI355X; cd /tmp && export TMPDIR=/tmp first, "
          "then back to the repository root):")
    print(f"#   rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv "
          f"-d {path.rstrip('/')} -- python bench.py --mode profile_prefill --launches {L}")
    print(f"#   python bench.py --mfma-util {path.rstrip('/')} --launches {L} > profiles/mfma_util_prefill.txt")
    print("# MFMA utilisation per prefill workload (rocprofv3 counters, one pass).  The 2048-token prefill "
          "is measured as the bench times it:")
    print("# after a 1 s clock warm-up, each launch right after a paged decode; the other two run back to "
          "back, their first 2 launches skipped")
    print("# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8 XCDs); "
          "clock = GPU cycles per XCD / dispatch time")
    for name in PREFILL_CONFIGS:
        w = getattr(W, name)
        sel = [rows[k] for k in groups[name]]
        busy = sum(d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) for d in sel) / simds
        gpu = sum(d.get("GRBM_GUI_ACTIVE", 0) for d in sel) / xcds
        t = sum(d["t"] for d in sel)
        flops = prefill_flops(w) * len(sel)
        print(f"{w.name}: launches={len(sel)} mfma_busy={busy / gpu:.3f} clock_ghz={gpu / t / 1e9:.2f} "
              f"avg_us={t / len(sel) * 1e6:.1f} tflops={flops / t / 1e12:.1f}")


def summarize(path, last=None):
    """Print the per-kernel duration table of a rocprofv3 kernel-trace run
    (its SQLite database, or the CSV stats when it wrote those).  With
    ``last`` (database only), each kernel's figures cover only its last
    ``last`` dispatches, i.e. the timed launches after the warm-up."""
    dbs = glob.glob(os.path.join(path, "**", "*.db"), recursive=True)
    csvs = glob.glob(os.path.join(path, "**", "*kernel_stats.csv"), recursive=True)
    if not dbs and not csvs:
        sys.exit(f"no rocprofv3 output under {path}")
    print(f"{'calls':>6} {'avg_us':>10} {'median_us':>10} {'min_us':>10} {'max_us':>10}  kernel")
    for fn in dbs:
        import sqlite3
        con = sqlite3.connect(fn)
        cur = con.execute("select * from kernels limit 1")
        cols = [c[0] for c in cur.description]
        start = next((c for c in ("start", "start_ns", "begin", "timestamp") if c in cols), None)
        order = f" order by {start}" if start else ""
        per = {}
        for name, dur in con.execute(f"select name, duration from kernels{order}"):
            per.setdefault(name, []).append(dur)
        table = []
        for name, durs in per.items():
            if last:
                durs = durs[-last:]
            table.append((sum(durs), name, durs))
        for _, name, durs in sorted(table, reverse=True):
            a = np.asarray(durs, dtype=np.float64) / 1e3
            print(f"{len(a):>6} {a.mean():>10.2f} {np.median(a):>10.2f} {a.min():>10.2f} {a.max():>10.2f}  "
                  f"{name[:160]}")
    for fn in csvs:
        with open(fn) as f:
            for r in csv.DictReader(f):
                print(f"{int(r.get('Calls', 0)):>6} {float(r.get('AverageNs', 0)) / 1e3:>10.2f} {'-':>10} "
                      f"{float(r.get('MinNs', 0)) / 1e3:>10.2f} "
                      f"{float(r.get('MaxNs', 0)) / 1e3:>10.2f}  {r.get('Name', '?')[:160]}")


def _counter_means(path, counter):
    """Mean per-dispatch value of one rocprofv3 counter, by kernel class."""
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        sys.exit(f"no rocprofv3 counter output under {path}")
    vals = {"prefill": [], "decode_main": [], "decode_merge": [], "copy": []}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                n = r["Kernel_Name"]
                key = ("prefill" if "fwd_mfma_kernel" in n
                       else "decode_main" if ("decode_partial" in n or "decode_stream" in n)
                       else "decode_merge" if "decode_merge" in n else "copy" if "neg_kernel" in n else None)
                if key:
                    vals[key].append(float(r["Counter_Value"]))
    # a kernel class with no dispatch contributes nothing (the copy is required)
    return {k: (sum(v) / len(v) if v else (float("nan") if k == "copy" else 0.0))
            for k, v in vals.items()}


def traffic(fetch_dir, write_dir, copy_bytes=64 * 1024 * 1024 * 4):
    """Per-launch HBM bytes from a FETCH_SIZE run and a WRITE_SIZE run of
    ``--mode profile`` (KiB per dispatch), each scaled by what the same
    counter reads for the copy kernel of known size; prints the traffic file."""
    fe, wr = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    f_fac = copy_bytes / 1024.0 / fe["copy"]
    w_fac = copy_bytes / 1024.0 / wr["copy"]
    pre = (fe["prefill"] * f_fac + wr["prefill"] * w_fac) * 1024.0
    dec_f = (fe["decode_main"] + fe["decode_merge"]) * f_fac * 1024.0
    dec_w = (wr["decode_main"] + wr["decode_merge"]) * w_fac * 1024.0
    print("# commands (from the repository root, on one MI355X; cd /tmp && export TMPDIR=/tmp first, "
          "then back to the repository root):")
    for ctr, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        print(f"#   rocprofv3 --pmc {ctr} --output-format csv -d {d.rstrip('/')} "
              "-- python bench.py --mode profile")
    print(f"#   python bench.py --traffic {fetch_dir.rstrip('/')} {write_dir.rstrip('/')} > profiles/hbm_traffic.txt")
    print("# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch),")
    print("# each scaled by the factor that makes the copy kernel (torch.neg over 256 MiB float32,")
    print("# 256 MiB read + 256 MiB written) read its known size.")
    print(f"fetch_calibration = {f_fac:.4f}")
    print(f"write_calibration = {w_fac:.4f}")
    print(f"copy_fetch_kib_raw = {fe['copy']:.1f}")
    print(f"copy_write_kib_raw = {wr['copy']:.1f}")
    print(f"prefill_fetch_kib_raw = {fe['prefill']:.1f}")
    print(f"prefill_write_kib_raw = {wr['prefill']:.1f}")
    print(f"decode_fetch_kib_raw = {fe['decode_main']:.1f} + {fe['decode_merge']:.1f} (decode + merge kernel, if any)")
    print(f"decode_write_kib_raw = {wr['decode_main']:.1f} + {wr['decode_merge']:.1f} (decode + merge kernel, if any)")
    print(f"prefill_bytes = {pre:.0f}")
    print(f"decode_bytes = {dec_f + dec_w:.0f}")
    print(f"decode_read_bytes = {dec_f:.0f}")
    print(f"decode_write_bytes = {dec_w:.0f}")
    print(f"sources_sha256_16 = {sources_digest()}")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--mode", choices=["bench", "profile", "profile_backward", "profile_prefill"],
                    default="bench")
    ap.add_argument("--launches", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip timing the other prefill workloads and the backward")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--clock-warm", type=float, default=1.0,
                    help="seconds of untimed steps before the warm-up steps, so that the GPU "
                         "clocks have ramped to their sustained level")
    ap.add_argument("--summarize", metavar="DIR")
    ap.add_argument("--last", type=int, default=None,
                    help="with --summarize: average only each kernel's last N dispatches")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--mfma-util", metavar="DIR")
    args = ap.parse_args()
    if args.summarize:
        return summarize(args.summarize, args.last)
    if args.traffic:
        return traffic(*args.traffic)
    if args.mfma_util:
        return mfma_util(args.mfma_util, args.launches)
    if args.gpus != 1:
        sys.exit(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}): the attention "
                 "kernels here run on one GPU and the library has no multi-GPU path")
    if args.mode == "profile":
        return profile(args)
    if args.mode == "profile_backward":
        return profile_backward(args)
    if args.mode == "profile_prefill":
        return profile_prefill(args)
    return bench(args)


if __name__ == "__main__":
    main()
