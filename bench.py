#!/usr/bin/env python3
"""Benchmark of the paged decode-attention hot path on one MI355X.

One step = pa_kv_append of every sequence's new token + pa_decode over the whole batch (one
decode step of one attention layer).  The headline workload is the largest single-GPU one, the
70B-style GQA layer: 64 sequences of 128..8192 tokens (uniform), 64 query / 8 KV heads,
head_dim 128, bf16, 16-token blocks scattered over a pool twice the needed size (1.16 GB of
K/V, tables, queries and outputs per call).  Every other decode workload is timed the same way
in the same run and reported under "configs".  Inputs are seeded synthetic data, resident in
HBM before the timed region; the pool is replicated `rotations` times and the steps cycle
through the copies so that no step finds its K/V in the 256 MB last-level cache.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved HBM GB/s (% of peak) and decode tokens/s"
PEAK_GBS = 8000.0           # MI355X HBM3E
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}   # MI355X dense MFMA
BLOCK_TOKENS = 16
DEFAULT_WORKLOAD = "gqa_b64_h64kv8_d128_bf16_l128to8192"
# decode workloads timed beside the headline (reported under "configs"), smallest first
CONFIG_WORKLOADS = ("tiny_b4_h8kv2_d64_bf16", "mha_b16_h32_d128_f16_l2048",
                    "gqa_b64_h64kv8_d128_bf16_l128to8192",
                    "mixed_b256_h32kv8_d128_bf16_lognorm600_prefix1024",
                    "long_b4_h64kv8_d128_fp8_l32768_split512")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(wl, decode_bytes_fn, append_bytes, min_s: float = 10.0,
                 max_s: float = 25.0) -> dict:
    """The fp64 oracle, as it stands, on one thread: repeated passes of append + decode over the
    workload until about min_s seconds have run (a pass stops early past max_s)."""
    from threadpoolctl import threadpool_limits

    import oracle

    s = wl.spec
    nbytes, seqs, appends = 0, 0, 0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        while True:
            k, v = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, wl.slot_mapping)
            nbytes += append_bytes
            appends += 1
            for b in range(wl.batch):
                sl = slice(b, b + 1)
                oracle.decode(wl.q[sl], k, v, wl.block_tables[sl], wl.context_lens[sl], wl.scale,
                              s.q_dtype, s.kv_dtype, wl.k_scale, wl.v_scale)
                nbytes += decode_bytes_fn(wl.context_lens[sl])
                seqs += 1
                if time.perf_counter() - t0 > max_s:
                    break
            secs = time.perf_counter() - t0
            if secs >= min_s:
                break
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{appends} append(s) of {wl.batch} tokens + {seqs} sequence decodes "
                      f"({seqs / wl.batch:.2f} passes over the batch) in {secs:.1f} s, numpy "
                      f"float64 on 1 thread; same byte model as the GPU figure"}


DECODE_SOURCES = ("decode.hip", "stepper.hpp", "device_common.hpp", "pa_internal.hpp")
MULTI_SOURCES = ("multi.hip", "multi_split.hip", "stepper.hpp", "device_common.hpp",
                 "pa_internal.hpp")


def traffic_record(workload: str, sources=DECODE_SOURCES):
    """HBM bytes per call measured with rocprofv3 PMC counters (profiles/), reported only while
    the kernel sources still hash to what they were when the counters were taken."""
    import glob
    import hashlib
    import re

    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, "paged_kv_cache_31_amd", "csrc", f), "rb").read())
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}.md"))):
        m = re.search(r"<!-- traffic-record (\{.*?\}) -->", open(path).read())
        if not m:
            continue
        rec = json.loads(m.group(1))
        if rec.get("workload") == workload and h.hexdigest() == rec.get("kernel_source_sha256"):
            return rec.get("traffic_bytes_per_launch")
    return None


def copy_probe(dev) -> int:
    """A plain device copy of 1 GiB, five times: its HBM byte counters per dispatch, compared
    with the 1 GiB read and 1 GiB written, give the scale factor for FETCH_SIZE / WRITE_SIZE."""
    import torch

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n}), flush=True)
    return 0


def multi_cpu_baseline(mw, unit_of, min_s: float = 10.0, max_s: float = 25.0) -> dict:
    """The fp64 oracle, as it stands, on one thread: oracle.decode_multi one sequence at a time
    over the workload until about min_s seconds have run."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    wl, s = mw.wl, mw.wl.spec
    amount, seqs = 0.0, 0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        while True:
            for b in range(wl.batch):
                qs = mw.query_start
                sub = np.array([0, qs[b + 1] - qs[b]], dtype=np.int32)
                oracle.decode_multi(mw.q[qs[b]:qs[b + 1]], sub, wl.k_cache, wl.v_cache,
                                    wl.block_tables[b:b + 1], wl.context_lens[b:b + 1], wl.scale,
                                    s.q_dtype, s.kv_dtype, wl.k_scale, wl.v_scale)
                amount += unit_of(b)
                seqs += 1
                if time.perf_counter() - t0 > max_s:
                    break
            secs = time.perf_counter() - t0
            if secs >= min_s:
                break
    return {"value": amount / secs, "cores": 1, "kind": "oracle",
            "sample": f"{seqs} sequences' multi-query attention ({seqs / wl.batch:.2f} passes "
                      f"over the batch) in {secs:.1f} s, numpy float64 on 1 thread; same "
                      f"byte/flop model as the GPU figure"}


def bench_multi(args, dev) -> int:
    """Several query tokens per sequence: one step = pa_kv_append of the new tokens +
    pa_decode_multi.  HBM-bound shapes report GB/s, MFMA-bound ones TFLOP/s."""
    import numpy as np
    import torch

    import paged_kv_cache_31_amd as pa
    import workloads

    t0 = time.perf_counter()
    mw = workloads.make_multi(args.workload)
    wl, s = mw.wl, mw.wl.spec
    B, Hq, Hkv, D = s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim
    N, maxT = int(mw.query_start[-1]), int(mw.query_lens.max())
    log(f"workload {args.workload}: generated in {time.perf_counter() - t0:.1f} s")
    nbytes = workloads.multi_bytes(wl.context_lens, mw.query_lens, Hq, Hkv, D, s.q_dtype,
                                   s.kv_dtype)
    flops = workloads.multi_flops(wl.context_lens, mw.query_lens, Hq, D)
    bytes_append = workloads.append_bytes(N, Hkv, D, s.kv_dtype)
    mfma = flops / nbytes > PEAK_TFLOPS[s.q_dtype] * 1e12 / (PEAK_GBS * 1e9)
    pool_bytes = wl.k_cache.nbytes + wl.v_cache.nbytes
    R = args.rotations or max(2, math.ceil(2 * 2**30 / nbytes))
    R = max(1, min(R, 64, int(48 * 2**30 // pool_bytes)))

    def to_dev(bits, dtype):
        a = np.ascontiguousarray(bits)
        if dtype == "fp8_e4m3":
            return torch.from_numpy(a).to(dev)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
        return torch.from_numpy(a.view(np.int16)).view(tdt).to(dev)

    base = {"q": to_dev(mw.q, s.q_dtype), "k": to_dev(wl.k_cache, s.kv_dtype),
            "v": to_dev(wl.v_cache, s.kv_dtype), "k_new": to_dev(mw.k_new, s.kv_dtype),
            "v_new": to_dev(mw.v_new, s.kv_dtype)}
    qs = torch.from_numpy(mw.query_start).to(dev)
    slots = torch.from_numpy(mw.slot_mapping).to(dev)
    tables = torch.from_numpy(wl.block_tables).to(dev)
    lens = torch.from_numpy(wl.context_lens).to(dev)
    k_scale = None if wl.k_scale is None else torch.from_numpy(wl.k_scale).to(dev)
    v_scale = None if wl.v_scale is None else torch.from_numpy(wl.v_scale).to(dev)
    rots = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(R - 1)]
    for r in rots:
        r["out"] = torch.empty_like(r["q"])
    P = args.partition or 0
    desc = pa.multi_desc(base["q"], base["k"], tables, maxT, wl.max_context_len, P)
    ws_bytes = pa.pa_decode_multi_workspace_size(desc)
    workspace = pa.new_workspace(max(ws_bytes, 1), dev)
    torch.cuda.synchronize()
    log(f"uploaded: {R} pool copies of {pool_bytes / 2**30:.2f} GiB; workspace {ws_bytes} B")

    appends = [pa.AppendCall(x["k_new"], x["v_new"], slots, x["k"], x["v"]) for x in rots]
    calls = [pa.MultiCall(x["q"], qs, x["k"], x["v"], tables, lens, float(wl.scale), x["out"],
                          maxT, k_scale=k_scale, v_scale=v_scale,
                          max_context_len=wl.max_context_len, partition_tokens=P,
                          workspace=workspace)
             for x in rots]

    def step(r):
        appends[r]()
        calls[r]()

    for i in range(args.warmup):
        step(i % R)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i % R)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step")

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        calls[i % R]()
    e1.record()
    torch.cuda.synchronize()
    launch_s = e0.elapsed_time(e1) / 1e3 / args.steps
    log(f"{args.steps} back-to-back pa_decode_multi calls: {launch_s * 1e6:.1f} us each")

    # the library's choice (pa_internal.hpp multi_plan): without a fixed partition, heads of one
    # to four row tiles take the balanced split kernel, larger ones the LDS-staged chunk kernel
    tiles = (maxT * (Hq // Hkv) + 15) // 16
    if P == 0 and tiles <= 4:
        kernel = "multi_split_kernel"
    else:
        kernel = "chunk_kernel" if P == 0 and tiles > 1 else "multi_kernel"
        if ws_bytes > 0:
            kernel += "+multi_merge_kernel"
    step_s = ms_per_step / 1e3
    if mfma:
        peak, unit = PEAK_TFLOPS[s.q_dtype], "TFLOP/s"
        metric = "paged multi-query attention (chunked prefill): achieved TFLOP/s"
        value = flops / step_s / 1e12
        achieved = flops / launch_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic_record(args.workload,
                                                                              MULTI_SOURCES),
                "kernel": kernel, "flops_per_launch": flops,
                "duration_us": round(launch_s * 1e6, 2)}
    else:
        unit = "GB/s"
        metric = "paged multi-query attention (speculative verification): achieved HBM GB/s"
        value = (nbytes + bytes_append) / step_s / 1e9
        achieved = nbytes / launch_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_GBS, "unit": unit,
                "frac": round(achieved / PEAK_GBS, 4),
                "traffic": traffic_record(args.workload, MULTI_SOURCES), "kernel": kernel,
                "bytes_per_launch": nbytes, "duration_us": round(launch_s * 1e6, 2)}
    result = {
        "metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": s.kv_dtype if s.kv_dtype == s.q_dtype else f"{s.q_dtype}+{s.kv_dtype}",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_dim": D, "block_size": 16, "q_dtype": s.q_dtype, "kv_dtype": s.kv_dtype,
            "query_tokens": N, "max_query_len": maxT,
            "context_len_min": int(wl.context_lens.min()),
            "context_len_max": int(wl.context_lens.max()),
            "partition_tokens": P or "auto", "rotations": R,
            "step": "pa_kv_append (the new tokens) + pa_decode_multi",
        },
        "query_tokens_per_s": round(N / launch_s, 1),
        "us_per_call": round(launch_s * 1e6, 2),
        "bytes_per_call": nbytes, "flops_per_call": flops,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (cpu_baseline)")
        if mfma:
            def unit_of(b):
                return workloads.multi_flops(wl.context_lens[b:b + 1], mw.query_lens[b:b + 1],
                                             Hq, D) / 1e12
        else:
            def unit_of(b):
                return workloads.multi_bytes(wl.context_lens[b:b + 1], mw.query_lens[b:b + 1],
                                             Hq, Hkv, D, s.q_dtype, s.kv_dtype) / 1e9
        cb = multi_cpu_baseline(mw, unit_of)
        cb["value"] = round(cb["value"], 6)
        cb["unit"] = unit
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)
    return 0


def graph_timing(args, rots, tables, lens, scale, k_scale, v_scale, mcl, P, share, ws_bytes,
                 dev) -> dict:
    """A step of K layers (pa_decode_append on K pool copies, one per layer) timed eagerly and
    as one HIP graph replay, both on one non-default stream, synchronised around `steps` steps."""
    import torch

    import paged_kv_cache_31_amd as pa

    K = args.graph_layers
    stream = torch.cuda.Stream(device=dev)
    calls = [pa.DecodeCall(x["q"], x["k"], x["v"], tables, lens, scale, x["out"],
                           k_scale=k_scale, v_scale=v_scale, max_context_len=mcl,
                           partition_tokens=P, shared_prefixes=share, k_new=x["k_new"],
                           v_new=x["v_new"], stream=stream,
                           workspace=pa.new_workspace(ws_bytes, dev))
             for x in rots[:K]]

    def eager():
        for c in calls:
            c()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        stream.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        stream.synchronize()
        return (time.perf_counter() - t0) * 1e6 / args.steps

    def unprepared():
        # the convenience function: descriptor, checks and argument marshalling on every call
        for x in rots[:K]:
            pa.pa_decode_append(x["q"], x["k_new"], x["v_new"], x["k"], x["v"], tables, lens,
                                scale, x["out"], k_scale=k_scale, v_scale=v_scale,
                                max_context_len=mcl, partition_tokens=P, workspace=ws0,
                                stream=stream, shared_prefixes=share)

    ws0 = pa.new_workspace(ws_bytes, dev)
    eager()
    stream.synchronize()
    graph = pa.StepGraph(calls, stream)
    t_eager = timed(eager)
    t_unprep = timed(unprepared)
    t_graph = timed(graph)
    launches = K * (2 if share else 1)
    log(f"{K}-layer step: eager {t_eager:.1f} us, unprepared {t_unprep:.1f} us, "
        f"graph {t_graph:.1f} us")
    return {"layers": K, "eager_us_per_step": round(t_eager, 2),
            "eager_unprepared_us_per_step": round(t_unprep, 2),
            "graph_us_per_step": round(t_graph, 2), "kernel_launches_per_step": launches,
            "us_saved_per_launch": round((t_eager - t_graph) / launches, 3)}


def bench_copy(args, dev) -> int:
    """Copy-on-write copies: pa_copy_blocks of N random (source, target) pairs over the
    workload's pool (targets distinct and never sources), HBM-bound: each pair reads and writes
    the K and V tiles of every KV head.  Also times the host pool's pa_pool_slot_for."""
    import numpy as np
    import torch

    import paged_kv_cache_31_amd as pa
    import workloads

    wl = workloads.make(args.workload, poison=False)
    s = wl.spec
    Hkv, D = s.num_kv_heads, s.head_dim
    e = 1 if s.kv_dtype == "fp8_e4m3" else 2
    NB = wl.num_blocks
    n = min(args.cow_pairs, NB // 2)
    rng = np.random.default_rng(1)
    perm = rng.permutation(NB)
    pairs_np = np.stack([perm[:n], perm[n:2 * n]], axis=1).astype(np.int32)
    tile = BLOCK_TOKENS * D * e
    nbytes = n * Hkv * (2 * 2 * tile + (16 if e == 1 else 0)) + n * 8

    def to_dev(bits, dtype):
        a = np.ascontiguousarray(bits)
        if dtype == "fp8_e4m3":
            return torch.from_numpy(a).to(dev)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
        return torch.from_numpy(a.view(np.int16)).view(tdt).to(dev)

    k, v = to_dev(wl.k_cache, s.kv_dtype), to_dev(wl.v_cache, s.kv_dtype)
    ks = None if wl.k_scale is None else torch.from_numpy(wl.k_scale).to(dev)
    vs = None if wl.v_scale is None else torch.from_numpy(wl.v_scale).to(dev)
    pairs = torch.from_numpy(pairs_np).to(dev)
    for _ in range(args.warmup):
        pa.pa_copy_blocks(pairs, k, v, ks, vs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        pa.pa_copy_blocks(pairs, k, v, ks, vs)
    e1.record()
    torch.cuda.synchronize()
    launch_s = e0.elapsed_time(e1) / 1e3 / args.steps
    achieved = nbytes / launch_s / 1e9
    log(f"pa_copy_blocks of {n} pairs: {launch_s * 1e6:.1f} us, {achieved:.0f} GB/s")

    # host bookkeeping: a decode step of 256 sequences, each forked once, every sequence asks
    # for the slot of its next token (a copy for the first writer of each shared block)
    pool = pa.BlockPool(1 << 16)
    tables, lens = [], []
    for i in range(128):
        t = pool.alloc(8)
        tables += [t, list(t)]
        pool.share(t)
        lens += [8 * 16 - 5, 8 * 16 - 5]
    t0 = time.perf_counter()
    calls = 0
    while time.perf_counter() - t0 < 0.5:
        for b in range(len(tables)):
            pool.slot_for(tables[b], lens[b], 64)
            lens[b] += 1
            calls += 1
    host_rate = calls / (time.perf_counter() - t0)

    result = {
        "metric": "copy-on-write block copy: achieved HBM GB/s", "value": round(achieved, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(launch_s * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u8" if e == 1 else "u16", "data": "synthetic",
        "config": {"workload": f"copy_blocks_{n}pairs_{args.workload}", "pairs": n,
                   "num_kv_heads": Hkv, "head_dim": D, "kv_dtype": s.kv_dtype,
                   "num_blocks": NB},
        "us_per_call": round(launch_s * 1e6, 2),
        "host_slot_for_calls_per_s": round(host_rate, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4), "traffic": None,
                     "kernel": "copy_blocks_kernel", "bytes_per_launch": nbytes,
                     "duration_us": round(launch_s * 1e6, 2)},
    }
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        done = 0
        sub = max(1, n // 16)
        while time.perf_counter() - t0 < 10.0:
            oracle.copy_blocks(wl.k_cache, wl.v_cache, wl.k_scale, wl.v_scale, pairs_np[:sub])
            done += sub
        secs = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(done / n * nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"oracle.copy_blocks of {done} pairs in batches of {sub} in {secs:.1f} s "
                      f"(each call copies the whole pool first, as the oracle returns new arrays)"}
    print(json.dumps(result), flush=True)
    return 0


def bench_decode(args, dev, name: str, headline: bool) -> dict:
    """One decode workload: a step is pa_decode_append (the append of token L-1 fused into the
    decode) unless --separate-append; the per-launch duration of the decode call alone is timed
    back to back between HIP events on the launching stream.  headline=False: the compact record
    reported under "configs" (no graph timing, no CPU baseline)."""
    import numpy as np
    import torch

    import paged_kv_cache_31_amd as pa
    import workloads

    t0 = time.perf_counter()
    wl = workloads.make(name, poison=False)
    s = wl.spec
    B, Hq, Hkv, D = s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim
    log(f"workload {name}: generated in {time.perf_counter() - t0:.1f} s")

    def dbytes(lens, unique=None):
        return workloads.decode_bytes(lens, Hq, Hkv, D, s.q_dtype, s.kv_dtype, unique)

    bytes_decode = dbytes(wl.context_lens, wl.unique_tokens)
    bytes_decode_logical = dbytes(wl.context_lens)
    bytes_append = workloads.append_bytes(B, Hkv, D, s.kv_dtype)
    pool_bytes = wl.k_cache.nbytes + wl.v_cache.nbytes
    R = args.rotations or max(2, math.ceil(2 * 2**30 / bytes_decode))
    R = max(1, min(R, 64, int(48 * 2**30 // pool_bytes)))
    if headline and args.graph_layers:
        R = max(R, args.graph_layers)

    def to_dev(bits, dtype):
        a = np.ascontiguousarray(bits)
        if dtype == "fp8_e4m3":
            return torch.from_numpy(a).to(dev)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
        return torch.from_numpy(a.view(np.int16)).view(tdt).to(dev)

    base = {
        "q": to_dev(wl.q, s.q_dtype), "k": to_dev(wl.k_cache, s.kv_dtype),
        "v": to_dev(wl.v_cache, s.kv_dtype),
        "k_new": to_dev(wl.k_new, s.kv_dtype), "v_new": to_dev(wl.v_new, s.kv_dtype),
    }
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    tables = torch.from_numpy(wl.block_tables).to(dev)
    lens = torch.from_numpy(wl.context_lens).to(dev)
    k_scale = None if wl.k_scale is None else torch.from_numpy(wl.k_scale).to(dev)
    v_scale = None if wl.v_scale is None else torch.from_numpy(wl.v_scale).to(dev)
    rots = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(R - 1)]
    for r in rots:
        r["out"] = torch.empty_like(r["q"])
    torch.cuda.synchronize()
    log(f"uploaded: {R} pool copies of {pool_bytes / 2**30:.2f} GiB")

    P = s.partition_tokens if args.partition is None else args.partition
    # a batch whose sequences share a prefix is decoded with the shared-prefix plan
    share = s.prefix is not None and not args.no_shared_prefixes
    desc = pa.decode_desc(base["q"], base["k"], tables, wl.max_context_len, P, share)
    ws_bytes = pa.pa_decode_workspace_size(desc)
    workspace = pa.new_workspace(ws_bytes, dev)
    scale = float(wl.scale)
    mcl = wl.max_context_len

    decodes = [pa.DecodeCall(x["q"], x["k"], x["v"], tables, lens, scale, x["out"],
                             k_scale=k_scale, v_scale=v_scale, max_context_len=mcl,
                             partition_tokens=P, workspace=workspace, shared_prefixes=share)
               for x in rots]
    if args.separate_append:
        appends = [pa.AppendCall(x["k_new"], x["v_new"], slots, x["k"], x["v"]) for x in rots]

        def step(r):
            appends[r]()
            decodes[r]()
    else:
        # the whole step in one launch: the append of token L-1 fused into the decode
        fused = [pa.DecodeCall(x["q"], x["k"], x["v"], tables, lens, scale, x["out"],
                               k_scale=k_scale, v_scale=v_scale, max_context_len=mcl,
                               partition_tokens=P, workspace=workspace, shared_prefixes=share,
                               k_new=x["k_new"], v_new=x["v_new"])
                 for x in rots]

        def step(r):
            fused[r]()

    for i in range(args.warmup):
        step(i % R)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i % R)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step")

    # Per-launch duration of the decode kernel: the same decode calls back to back on the same
    # stream between two events (per-call events above also count the dispatch latency).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        decodes[i % R]()
    e1.record()
    torch.cuda.synchronize()
    launch_s = e0.elapsed_time(e1) / 1e3 / args.steps
    log(f"{args.steps} back-to-back decode launches: {launch_s * 1e6:.1f} us each")

    achieved = bytes_decode / launch_s / 1e9
    value = (bytes_decode + bytes_append) / (ms_per_step / 1e3) / 1e9
    # the decode call is one kernel, or the prefix and decode kernels with shared prefixes
    kernel = "prefix_kernel+decode_kernel" if share else "decode_kernel"
    lens_np = wl.context_lens
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.kv_dtype if s.kv_dtype == s.q_dtype else f"{s.q_dtype}+{s.kv_dtype}",
        "data": "synthetic",
        "config": {
            "workload": name, "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_dim": D, "block_size": 16, "q_dtype": s.q_dtype, "kv_dtype": s.kv_dtype,
            "context_len_min": int(lens_np.min()), "context_len_max": int(lens_np.max()),
            "context_tokens": int(lens_np.sum()), "unique_tokens": int(wl.unique_tokens),
            "num_blocks": wl.num_blocks, "partition_tokens": P or "balanced", "rotations": R,
            "shared_prefixes": share,
            "step": ("pa_kv_append (1 token per sequence) + pa_decode" if args.separate_append
                     else "pa_decode_append (append of 1 token per sequence fused into the decode)"),
        },
        "pct_of_peak": round(100 * value / PEAK_GBS, 2),
        "decode_tokens_per_s": round(B / launch_s, 1),
        "step_tokens_per_s": round(B / (ms_per_step / 1e3), 1),
        "us_per_decode_launch": round(launch_s * 1e6, 2),
        "bytes_per_step": {"decode": bytes_decode, "decode_logical": bytes_decode_logical,
                           "append": bytes_append},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": traffic_record(name),
                     "kernel": kernel, "bytes_per_launch": bytes_decode,
                     "duration_us": round(launch_s * 1e6, 2)},
    }
    if share:
        # After a planning call, the other layers of the step and later steps while the batch
        # keeps its sequences may reuse its grouping (shared_prefixes 2; the reusing call checks
        # it against its tables and lengths).  Reported beside the planning call, with the
        # average over a step of 32 layers that plans once.
        reuse = [pa.DecodeCall(x["q"], x["k"], x["v"], tables, lens, scale, x["out"],
                               k_scale=k_scale, v_scale=v_scale, max_context_len=mcl,
                               partition_tokens=P, workspace=workspace, shared_prefixes=2)
                 for x in rots]
        decodes[0]()
        for i in range(args.warmup):
            reuse[i % R]()
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            reuse[i % R]()
        e1.record()
        torch.cuda.synchronize()
        reuse_s = e0.elapsed_time(e1) / 1e3 / args.steps
        log(f"{args.steps} back-to-back decode launches reusing the plan: "
            f"{reuse_s * 1e6:.1f} us each")
        layer_s = (launch_s + 31 * reuse_s) / 32
        result["reusing_the_plan"] = {
            "what": "pa_decode with shared_prefixes 2: the grouping of a planning call reused "
                    "(checked against the call's tables and lengths) by the other layers of "
                    "the step and by later steps",
            "us_per_decode_launch": round(reuse_s * 1e6, 2),
            "achieved": round(bytes_decode / reuse_s / 1e9, 2), "unit": "GB/s",
            "frac": round(bytes_decode / reuse_s / 1e9 / PEAK_GBS, 4),
            "step_of_32_layers_planning_once": {
                "us_per_decode_launch": round(layer_s * 1e6, 2),
                "frac": round(bytes_decode / layer_s / 1e9 / PEAK_GBS, 4)}}
    if headline and args.graph_layers:
        result["graph"] = graph_timing(args, rots, tables, lens, scale, k_scale, v_scale, mcl, P,
                                       share, ws_bytes, dev)
    if headline and not args.no_cpu_baseline:
        log("timing the oracle on the host (cpu_baseline)")
        result["cpu_baseline"] = cpu_baseline(wl, dbytes, bytes_append)
    record = {
        "workload": name, "kernel": kernel, "bytes_per_launch": bytes_decode,
        "us_per_decode_launch": round(launch_s * 1e6, 2),
        "achieved_GBps": round(achieved, 2), "frac": round(achieved / PEAK_GBS, 4),
        "decode_tokens_per_s": round(B / launch_s, 1),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "step": "pa_kv_append + pa_decode" if args.separate_append else "pa_decode_append",
    }
    if "reusing_the_plan" in result:
        record["reusing_the_plan"] = {k: result["reusing_the_plan"][k] for k in
                                      ("us_per_decode_launch", "achieved", "frac",
                                       "step_of_32_layers_planning_once")}
    if not headline:
        return record
    result["this_config"] = record
    return result



def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="a single-query workload (default) or a multi-query one: "
                         "verify_b64_h64kv8_d128_bf16_l128to8192_t4, "
                         "verify_b4_h64kv8_d128_fp8_l32768_t4, "
                         "prefill_b4_h32kv8_d128_bf16_l4608_chunk512")
    ap.add_argument("--partition", type=int, default=None,
                    help="key-partition tokens (default: the workload's, else the library's)")
    ap.add_argument("--rotations", type=int, default=0, help="pool copies cycled (0: auto)")
    ap.add_argument("--separate-append", action="store_true",
                    help="time a step as pa_kv_append + pa_decode instead of pa_decode_append")
    ap.add_argument("--no-shared-prefixes", action="store_true",
                    help="decode a workload with a shared prefix without the prefix plan")
    ap.add_argument("--graph-layers", type=int, default=0,
                    help="also time a step of this many layers (one pool copy each) eagerly "
                         "and as one HIP graph replay")
    ap.add_argument("--cow-pairs", type=int, default=0,
                    help="instead: time pa_copy_blocks of this many (source, target) block pairs "
                         "on the workload's pool, and the host pool's slot bookkeeping")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the chosen workload, not every decode workload beside it")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs on one GPU; no multi-GPU path is built, so "
              f"--gpus {args.gpus} is not supported (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import paged_kv_cache_31_amd as pa
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.copy_probe:
        return copy_probe(dev)
    pa.lib()
    if args.workload in workloads.MULTI_SPECS:
        return bench_multi(args, dev)
    if args.cow_pairs:
        return bench_copy(args, dev)

    result = bench_decode(args, dev, args.workload, headline=True)
    if not args.no_configs:
        # every decode workload, timed the same way in this run (the headline's own included)
        result["configs"] = []
        for name in CONFIG_WORKLOADS:
            gc.collect()
            torch.cuda.empty_cache()                  # the previous workload's pool copies
            if name == args.workload:
                result["configs"].append(result["this_config"])
            else:
                result["configs"].append(bench_decode(args, dev, name, headline=False))
    result.pop("this_config", None)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
