#!/usr/bin/env python3
"""Benchmark one decode step of paged attention on one MI355X.

A step is the whole hot path over one batch: pa_cache_write of the step's
new tokens (one per sequence) into the paged caches, then pa_decode of every
sequence over its cached context. Inputs are seeded synthetic data already
resident in HBM when the timed region starts.

    python bench.py [--steps K] [--warmup W] [--workload llama70b_gqa] [--kv bf16|fp8]

Prints progress on stderr and ONE JSON line on stdout:
  value      algorithmic bytes of the step (decode + cache write) / step time, GB/s
  roofline   the decode kernel alone: algorithmic bytes per launch / average
             launch time (HIP events on the launch stream) against 8 TB/s
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same
             workload, same byte model, on this host's cores
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_bytes(w, kv_bytes: int) -> int:
    """Algorithmic bytes of one decode launch: each sequence reads its K and V
    rows once (2 * ctx * Hkv * D * e), its q row and writes its output
    (2 * Hq * D * 2), reads its block-table entries (4 per block) and its
    context length (4)."""
    s = w.spec
    ctx = w.context_lens.astype(np.int64)
    nblk = (ctx + s.block_size - 1) // s.block_size
    kv = 2 * ctx * s.num_kv_heads * s.head_dim * kv_bytes
    return int(kv.sum() + s.num_seqs * (2 * s.num_q_heads * s.head_dim * 2 + 4) + 4 * nblk.sum())


def write_bytes(w, kv_bytes: int) -> int:
    """Cache write: read new K and V (bf16), write them (kv_bytes each), read 8-byte slots."""
    s = w.spec
    T = len(w.slot_mapping)
    return int(T * s.num_kv_heads * s.head_dim * (2 * 2 + 2 * kv_bytes) + 8 * T)


def load_traffic(workload: str, kv: str, plan: dict, layout: str = "page", partition_tokens: int = 0):
    """HBM traffic per decode launch from the committed rocprofv3 counter
    summary of this configuration, if it was taken on the current kernel
    sources with the same launch plan."""
    from paged_kv_decode_mapping_amd.profiling import kernel_source_hash, traffic_file
    p = traffic_file(workload, kv, layout, partition_tokens or 0)
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("kernel_source_hash") != kernel_source_hash(plan) or d.get("plan") != plan:
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(w, kv: str, kq=None, vq=None, min_s: float = 10.0, budget_s: float = 30.0) -> dict:
    """Time the oracle on a bounded sample of (sequence, KV head) units: chunks
    of a fixed random order of all units, cycling through it again when one
    pass takes less than min_s, and stopping at min_s (at most budget_s)."""
    import oracle
    s = w.spec
    units_all = np.random.default_rng(5).permutation(s.num_seqs * s.num_kv_heads)
    kvd = oracle.KV_BF16 if kv == "bf16" else oracle.KV_FP8_E4M3FN
    ks, vs = w.fp8_scales if kv == "fp8" else (1.0, 1.0)
    kc = w.k_cache if kv == "bf16" else kq
    vc = w.v_cache if kv == "bf16" else vq
    e = 2 if kv == "bf16" else 1
    done, nbytes, t_total = 0, 0, 0.0
    chunk = max(1, min(64, len(units_all)))
    while t_total < min(min_s, budget_s):
        i = done % len(units_all)
        u = units_all[i:i + chunk]
        t0 = time.perf_counter()
        oracle.decode_workload(w, units=u, kv_dtype=kvd, k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs)
        t_total += time.perf_counter() - t0
        seqs = u // s.num_kv_heads
        ctx = w.context_lens[seqs].astype(np.int64)
        nbytes += int((2 * ctx * s.head_dim * e + 2 * s.group * s.head_dim * 2 + 4 * ((ctx + s.block_size - 1) // s.block_size)).sum())
        done += len(u)
    return {"value": round(nbytes / t_total / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{done} (sequence, KV head) unit decodes ({done / len(units_all):.2f} passes over the "
                      f"{len(units_all)} units), {t_total:.1f} s, float64 gather + softmax(qK^T)V, same byte model"}


def stream_read_gbps(dev, nbytes: int, iters: int, nontemporal: bool = True) -> float:
    """Read rate of the library's streaming-read probe over nbytes (one pass,
    16-byte loads), averaged over iters timed launches after two untimed."""
    import torch
    import paged_kv_decode_mapping_amd as pa
    x = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        pa.pa_probe_stream_read(x, sink, nontemporal)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record(stream)
        pa.pa_probe_stream_read(x, sink, nontemporal)
        b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    del x
    return nbytes / (ms.mean() * 1e-3) / 1e9


def bench_stream(args, dev) -> int:
    """Streaming-read reference on the same GPU: the library's probe kernel
    reads a 4 GiB buffer once with 16-byte loads, with the default cache
    policy and with the non-temporal one the decode kernels use."""
    import torch
    import paged_kv_decode_mapping_amd as pa
    nbytes = 4 << 30
    x = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    rates = {}
    for nt in (False, True):
        for _ in range(max(args.warmup, 1)):
            pa.pa_probe_stream_read(x, sink, nt)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in ev:
            a.record(stream)
            pa.pa_probe_stream_read(x, sink, nt)
            b.record(stream)
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in ev])
        rates["nontemporal" if nt else "default"] = nbytes / (ms.mean() * 1e-3) / 1e9
        log(f"stream read ({'non-temporal' if nt else 'default'} loads): {nbytes} B, avg {ms.mean() * 1e3:.1f} us "
            f"= {rates['nontemporal' if nt else 'default']:.0f} GB/s")
    best = max(rates.values())
    res = {"metric": "streaming read of 4 GiB by pa_probe_stream_read (the practical read ceiling)",
           "value": round(best, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(nbytes / best / 1e6, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "u8", "data": "synthetic",
           "config": {"workload": "one read of a 4 GiB buffer, 16-byte loads"},
           "rates_gbps": {k: round(v, 1) for k, v in rates.items()},
           "roofline": {"bound": "hbm", "achieved": round(best, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(best / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": "pa_probe_read_kernel"},
           "cpu_baseline": None}
    print(json.dumps(res), flush=True)
    return 0


def bench_graph(args, w, q, k_cache, v_cache, tables, ctx, new_k, new_v, slots, k_scale, v_scale, plan,
                kv_b: int) -> int:
    """Time the step (cache write + decode) captured once in a HIP graph and
    replayed, next to the same step launched eagerly through the binding."""
    import torch
    import paged_kv_decode_mapping_amd as pa
    s = w.spec
    dev = q.device
    ws = torch.empty(max(plan["workspace_bytes"], 256), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)

    def step():
        pa.pa_cache_write(new_k, new_v, slots, k_cache, v_cache, k_scale, v_scale)
        pa.pa_decode(q, k_cache, v_cache, tables, ctx, w.scale, out, k_scale=k_scale, v_scale=v_scale,
                     workspace=ws, partition_tokens=args.partition, variant=args.variant, waves=args.waves,
                     prefetch=args.prefetch, schedule=args.schedule, heads_per_tile=args.heads_per_tile)

    def timed(fn, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(max(args.warmup, 1)):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    eager = timed(step, args.steps)
    replay = timed(graph.replay, args.steps)
    dec_b = decode_bytes(w, kv_b)
    wr_b = write_bytes(w, kv_b)
    log(f"graph: eager step {eager * 1e6:.1f} us, replay {replay * 1e6:.1f} us")
    res = {
        "metric": "paged decode step (cache write + decode) from a HIP graph: achieved HBM GB/s",
        "value": round((dec_b + wr_b) / replay / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(replay * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.kv, "data": "synthetic",
        "config": {"workload": f"{s.name}: {s.description}", "num_seqs": s.num_seqs, "plan": plan},
        "eager_us_per_step": round(eager * 1e6, 2), "graph_us_per_step": round(replay * 1e6, 2),
        "decode_tokens_per_s": round(s.num_seqs / replay, 1),
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)
    return 0


def bench_multi(args, w, k_cache, v_cache, tables, ctx, kv_b: int, k_scale: float, v_scale: float,
                kq=None, vq=None) -> int:
    """Time pa_decode_multi: the last --qlen cached tokens of every sequence are
    its queries (speculative verification of qlen - 1 draft tokens)."""
    import torch
    import paged_kv_decode_mapping_amd as pa
    from paged_kv_decode_mapping_amd import workloads as W
    s = w.spec
    qlens = np.minimum(np.full(s.num_seqs, args.qlen), w.context_lens)
    mq = W.make_multi_query(w, qlens)
    dev = k_cache.device
    q = torch.from_numpy(mq.q.view(np.int16)).view(torch.bfloat16).to(dev)
    qs = torch.from_numpy(mq.query_start).to(dev)
    maxq = int(qlens.max())
    kvd = pa.PA_KV_BF16 if kv_b == 2 else pa.PA_KV_FP8_E4M3FN
    need = pa.pa_decode_multi_workspace_size(q, k_cache, tables, maxq, args.partition)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)

    def run():
        pa.pa_decode_multi(q, k_cache, v_cache, tables, ctx, qs, w.scale, maxq, out, k_scale=k_scale,
                           v_scale=v_scale, workspace=ws, partition_tokens=args.partition)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        run()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    avg = float(ms.mean())
    cl = w.context_lens.astype(np.int64)
    nblk = (cl + s.block_size - 1) // s.block_size
    # K and V of every context once, q in and out for every query row, tables and offsets
    nbytes = int((2 * cl * s.num_kv_heads * s.head_dim * kv_b).sum() + 2 * mq.num_tokens * s.num_q_heads * s.head_dim * 2
                 + 4 * nblk.sum() + 4 * s.num_seqs + 4 * (s.num_seqs + 1))
    achieved = nbytes / (avg * 1e-3) / 1e9
    log(f"multi: {mq.num_tokens} query tokens (qlen {args.qlen}), avg {avg * 1e3:.1f} us = {achieved:.0f} GB/s")
    base = None
    if not args.no_cpu_baseline:
        import oracle
        kvd_o = oracle.KV_BF16 if kv_b == 2 else oracle.KV_FP8_E4M3FN
        kc = w.k_cache if kq is None else kq
        vc = w.v_cache if vq is None else vq
        units_all = np.random.default_rng(5).permutation(s.num_seqs * s.num_kv_heads)
        done, t_total, ob = 0, 0.0, 0
        while done < len(units_all) and t_total < 12.0:
            u = units_all[done:done + 64]
            t1 = time.perf_counter()
            oracle.multi_decode(mq.q, kc, vc, w.block_tables, w.context_lens, mq.query_start, w.scale, units=u,
                                kv_dtype=kvd_o, k_scale=k_scale, v_scale=v_scale)
            t_total += time.perf_counter() - t1
            seqs = u // s.num_kv_heads
            ob += int((2 * cl[seqs] * s.head_dim * kv_b + 4 * qlens[seqs] * s.group * s.head_dim).sum())
            done += len(u)
        base = {"value": round(ob / t_total / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
                "kind": "oracle", "sample": f"{done} of {len(units_all)} (sequence, KV head) units, {t_total:.1f} s"}
        log(f"cpu baseline {base}")
    res = {
        "metric": "multi-token paged attention achieved HBM GB/s + query tokens/s",
        "value": round(nbytes * args.steps / wall / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.kv, "data": "synthetic",
        "config": {"workload": f"{s.name} with {args.qlen} query tokens per sequence", "num_seqs": s.num_seqs,
                   "query_tokens": mq.num_tokens, "num_q_heads": s.num_q_heads, "num_kv_heads": s.num_kv_heads,
                   "head_dim": s.head_dim, "block_size": s.block_size, "layout": args.layout},
        "query_tokens_per_s": round(mq.num_tokens / (avg * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": "pa_decode_multi"},
        "cpu_baseline": base,
    }
    print(json.dumps(res), flush=True)
    return 0


def bench_cascade(args, w, k_cache, v_cache, kv_b: int, k_scale: float, v_scale: float, kq=None, vq=None) -> int:
    """Time pa_decode_cascade on a workload whose sequences share a prefix (the
    mixed batch): the batch reordered with its sharers first (one group), the
    shared prefix attended once for the group. pa_decode on the same batch is
    timed beside it."""
    import torch
    import paged_kv_decode_mapping_amd as pa
    from paged_kv_decode_mapping_amd import workloads as W
    s = w.spec
    b = W.cascade_batch(w)
    if b.num_groups == 0:
        log(f"{s.name} has no shared prefix: nothing to cascade")
        return 2
    dev = k_cache.device
    q = torch.from_numpy(b.q.view(np.int16)).view(torch.bfloat16).to(dev)
    tables = torch.from_numpy(b.block_tables).to(dev)
    ctx = torch.from_numpy(b.context_lens).to(dev)
    ptab = torch.from_numpy(b.prefix_tables).to(dev)
    plen = torch.from_numpy(b.prefix_lens).to(dev)
    gst = torch.from_numpy(b.group_start).to(dev)
    kvd = pa.PA_KV_BF16 if kv_b == 2 else pa.PA_KV_FP8_E4M3FN
    need = pa.pa_decode_cascade_workspace_size(q, k_cache, tables, ptab, b.max_group_size,
                                               partition_tokens=args.partition)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    plan = pa.pa_decode_get_plan(q, k_cache, tables, partition_tokens=args.partition)
    ws_d = torch.empty(max(plan["workspace_bytes"], 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    out_d = torch.empty_like(q)

    def cascade():
        pa.pa_decode_cascade(q, k_cache, v_cache, tables, ctx, ptab, plen, gst, w.scale, out,
                             max_group_size=b.max_group_size, k_scale=k_scale, v_scale=v_scale, workspace=ws,
                             partition_tokens=args.partition)

    def plain():
        pa.pa_decode(q, k_cache, v_cache, tables, ctx, w.scale, out_d, k_scale=k_scale, v_scale=v_scale,
                     workspace=ws_d, partition_tokens=args.partition)

    stream = torch.cuda.current_stream()
    # In serving, every other layer's KV passes through the caches between two
    # steps of one layer: a scratch write before each timed call (outside its
    # events) evicts the 256 MB Infinity Cache, so no call starts warm.
    scratch = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for i in range(args.steps):
            scratch.add_(1)
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(e) for a, e in ev])

    cas_ms = timed(cascade)
    dec_ms = timed(plain)
    cl = b.context_lens.astype(np.int64)
    n_sh = int(b.group_start[1])
    shared = np.zeros_like(cl)
    shared[:n_sh] = np.minimum(cl[:n_sh], int(b.prefix_lens[0]))
    row = s.num_kv_heads * s.head_dim * kv_b
    logical = decode_bytes(w, kv_b)
    # the cascade must read the prefix once (as far as its longest member
    # goes) and each sequence's tokens after it; q, out and tables as before
    unique = logical - int(2 * shared.sum() * row) + int(2 * shared.max() * row)
    avg = float(cas_ms.mean())
    avg_d = float(dec_ms.mean())
    log(f"cascade avg {avg * 1e3:.1f} us (p10 {np.percentile(cas_ms, 10) * 1e3:.1f}, p90 "
        f"{np.percentile(cas_ms, 90) * 1e3:.1f}); pa_decode on the same batch {avg_d * 1e3:.1f} us; "
        f"logical {logical / (avg * 1e-3) / 1e9:.0f} GB/s, unique {unique / (avg * 1e-3) / 1e9:.0f} GB/s")
    base = None
    if not args.no_cpu_baseline:
        import oracle
        kvd_o = oracle.KV_BF16 if kv_b == 2 else oracle.KV_FP8_E4M3FN
        kc = w.k_cache if kq is None else kq
        vc = w.v_cache if vq is None else vq
        units_all = np.random.default_rng(5).permutation(s.num_seqs * s.num_kv_heads)
        done, t_total, ob = 0, 0.0, 0
        while done < len(units_all) and t_total < 12.0:
            u = units_all[done:done + 64]
            t1 = time.perf_counter()
            oracle.cascade_decode(b.q, kc, vc, b.block_tables, b.context_lens, b.prefix_tables, b.prefix_lens,
                                  b.group_start, w.scale, max_group_size=b.max_group_size, units=u,
                                  kv_dtype=kvd_o, k_scale=k_scale, v_scale=v_scale)
            t_total += time.perf_counter() - t1
            seqs = u // s.num_kv_heads
            ob += int((2 * cl[seqs] * s.head_dim * kv_b + 4 * s.group * s.head_dim).sum())
            done += len(u)
        base = {"value": round(ob / t_total / 1e9, 3), "unit": "GB/s (logical)", "cores": oracle.num_threads(),
                "kind": "oracle", "sample": f"{done} of {len(units_all)} (sequence, KV head) units, "
                                            f"{t_total:.1f} s, float64, gather through the composed table"}
        log(f"cpu baseline {base}")
    achieved = unique / (avg * 1e-3) / 1e9
    res = {
        "metric": "shared-prefix (cascade) decode: logical GB/s (bytes a plain decode reads for the same outputs)",
        "value": round(logical / (avg * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(avg, 5),
        "timing": "HIP events around each call, caches evicted before each (512 MiB scratch write)",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.kv, "data": "synthetic",
        "config": {"workload": f"{s.name} reordered, {n_sh} sequences sharing a {int(b.prefix_lens[0])}-token "
                               f"prefix as one group", "num_seqs": s.num_seqs, "num_q_heads": s.num_q_heads,
                   "num_kv_heads": s.num_kv_heads, "head_dim": s.head_dim, "block_size": s.block_size},
        "cascade_us": {"avg": round(avg * 1e3, 2), "p10": round(float(np.percentile(cas_ms, 10)) * 1e3, 2),
                       "p90": round(float(np.percentile(cas_ms, 90)) * 1e3, 2)},
        "pa_decode_us": round(avg_d * 1e3, 2),
        "speedup_vs_pa_decode": round(avg_d / avg, 3),
        "bytes": {"logical": logical, "unique": unique},
        "decode_tokens_per_s_kernel": round(s.num_seqs / (avg * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "pa_decode_cascade (schedule + prefix pass + decode + merge), unique bytes"},
        "cpu_baseline": base,
    }
    print(json.dumps(res), flush=True)
    return 0


def bench_copy_blocks(args, w, k_cache, v_cache, kv_b: int, kq=None, vq=None) -> int:
    """Time pa_copy_blocks: each call copies --pairs whole blocks of K and V
    (src and dst drawn without replacement from a fresh permutation of the
    pool per call, so no call finds its blocks in a cache)."""
    import torch
    import paged_kv_decode_mapping_amd as pa
    s = w.spec
    n = args.pairs
    N = w.num_blocks
    if 2 * n > N:
        raise SystemExit(f"--pairs {n} needs a pool of at least {2 * n} blocks (have {N})")
    rng = np.random.default_rng(77)
    calls = args.warmup + args.steps
    maps = [torch.from_numpy(np.ascontiguousarray(rng.permutation(N)[:2 * n].reshape(2, n).T)).to(k_cache.device)
            for _ in range(calls)]
    block_bytes = s.block_size * s.num_kv_heads * s.head_dim * kv_b
    moved = 4 * n * block_bytes  # K and V, read once and written once
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        pa.pa_copy_blocks(k_cache, v_cache, maps[i])
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        pa.pa_copy_blocks(k_cache, v_cache, maps[args.warmup + i])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    avg = float(ms.mean())
    achieved = moved / (avg * 1e-3) / 1e9
    log(f"copy_blocks: {n} pairs x {block_bytes} B, avg {avg * 1e3:.1f} us = {achieved:.0f} GB/s")
    base = None
    if not args.no_cpu_baseline:
        import oracle
        kc = w.k_cache if kq is None else kq
        vc = w.v_cache if vq is None else vq
        kc, vc = np.array(kc), np.array(vc)  # private copies: the oracle copies in place
        pairs = maps[0].cpu().numpy()[: min(n, 256)]
        t1 = time.perf_counter()
        oracle.copy_blocks(kc, vc, pairs)
        dt = time.perf_counter() - t1
        base = {"value": round(4 * len(pairs) * block_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                "kind": "oracle", "sample": f"{len(pairs)} of {n} pairs of one call, {dt:.2f} s, element-wise copy"}
        log(f"cpu baseline {base}")
    res = {
        "metric": "paged KV block copy achieved HBM GB/s (read + write)",
        "value": round(moved * args.steps / wall / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.kv, "data": "synthetic",
        "config": {"workload": f"{s.name} pool: {n} block pairs per call, {block_bytes} B per block and cache",
                   "num_blocks": N, "block_size": s.block_size, "num_kv_heads": s.num_kv_heads,
                   "head_dim": s.head_dim, "pairs": n},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": "pa_copy_blocks"},
        "cpu_baseline": base,
    }
    print(json.dumps(res), flush=True)
    return 0


# The other named configurations, measured in the same run after the
# headline one (decode alone, HIP events per launch): the 7B-shaped MHA
# batch, the long-context batch at its stated 512-token partitions and at
# the library's own plan, the mixed continuous batch with bf16 and fp8
# caches, and the 70B-shaped batch with fp8 caches.
PER_CONFIG = [
    ("llama7b_mha", "bf16", 0),
    ("long_splitk", "bf16", 512),
    ("long_splitk", "bf16", 0),
    ("mixed_batch", "bf16", 0),
    ("mixed_batch", "fp8", 0),
    ("long_splitk", "fp8", 0),
    ("llama70b_gqa", "fp8", 0),
]
EVICT_BELOW_BYTES = 1 << 30  # KV smaller than this could stay in the 256 MB Infinity Cache between steps
MIN_WARMUP_S = 0.2           # clocks ramp during the first ~10 ms of GPU work after host-side set-up


class DeviceBatch:
    """One workload's inputs resident on the device: q, the two caches (bf16,
    or fp8 codes written by the library's own quantising cache write) in the
    requested layout, tables, lengths, and the step's new tokens."""

    def __init__(self, w, kv: str, layout: str, dev, host_codes: bool = False):
        import torch
        import paged_kv_decode_mapping_amd as pa
        s = w.spec
        self.w, self.kv, self.layout = w, kv, layout
        self.kv_b = 2 if kv == "bf16" else 1

        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        self.q = bf16(w.q)
        k_cache, v_cache = bf16(w.k_cache), bf16(w.v_cache)
        self.tables = torch.from_numpy(w.block_tables).to(dev)
        self.ctx = torch.from_numpy(w.context_lens).to(dev)
        self.new_k, self.new_v = bf16(w.new_k), bf16(w.new_v)
        self.slots = torch.from_numpy(w.slot_mapping).to(dev)
        self.k_scale = self.v_scale = 1.0
        self.kq = self.vq = None
        if kv == "fp8":
            self.k_scale, self.v_scale = w.fp8_scales
            rows = w.num_blocks * s.block_size
            all_slots = torch.arange(rows, dtype=torch.int64, device=dev)
            kc8 = torch.empty((w.num_blocks, s.block_size, s.num_kv_heads, s.head_dim), dtype=torch.uint8,
                              device=dev)
            vc8 = torch.empty_like(kc8)
            pa.pa_cache_write(k_cache.view(rows, s.num_kv_heads, s.head_dim),
                              v_cache.view(rows, s.num_kv_heads, s.head_dim), all_slots, kc8, vc8,
                              self.k_scale, self.v_scale)
            torch.cuda.synchronize()
            del k_cache, v_cache
            k_cache, v_cache = kc8, vc8
            if host_codes:
                self.kq, self.vq = kc8.cpu().numpy(), vc8.cpu().numpy()
        if layout == "head_major":
            # the same logical pool stored [N, Hkv, bs, D]: each (block, KV
            # head) tile is one contiguous run; passed as the permuted view
            def to_head_major(t):
                hm = torch.empty((t.shape[0], t.shape[2], t.shape[1], t.shape[3]), dtype=t.dtype, device=dev)
                hm.copy_(t.permute(0, 2, 1, 3))
                return hm.permute(0, 2, 1, 3)
            k_cache, v_cache = to_head_major(k_cache), to_head_major(v_cache)
            torch.cuda.synchronize()
        self.k_cache, self.v_cache = k_cache, v_cache

    def unique_kv_bytes(self) -> int:
        w = self.w
        return 2 * w.unique_blocks * w.spec.block_size * w.spec.num_kv_heads * w.spec.head_dim * self.kv_b


def time_decode(b: "DeviceBatch", opts: dict, steps: int, warmup: int, evict: bool):
    """Per-launch decode times (ms, HIP events on the launch stream) after a
    warm-up of at least `warmup` launches and MIN_WARMUP_S seconds. With
    evict, a 512 MiB scratch write before each timed launch (outside its
    events) clears the Infinity Cache, as every other layer's KV would."""
    import torch
    import paged_kv_decode_mapping_amd as pa
    plan = pa.pa_decode_get_plan(b.q, b.k_cache, b.tables, **opts)
    ws = torch.empty(max(plan["workspace_bytes"], 1), dtype=torch.uint8, device=b.q.device)
    out = torch.empty_like(b.q)
    stream = torch.cuda.current_stream()

    def run():
        pa.pa_decode(b.q, b.k_cache, b.v_cache, b.tables, b.ctx, b.w.scale, out, k_scale=b.k_scale,
                     v_scale=b.v_scale, workspace=ws, **opts)

    warm_up(run, warmup)
    scratch = torch.zeros(512 << 20, dtype=torch.uint8, device=b.q.device) if evict else None
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, e in ev:
        if scratch is not None:
            scratch.add_(1)
        a.record(stream)
        run()
        e.record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(e) for a, e in ev]), plan, out


def warm_up(fn, n: int) -> None:
    import torch
    t0 = time.perf_counter()
    i = 0
    while i < n or time.perf_counter() - t0 < MIN_WARMUP_S:
        fn()
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def fp8_accuracy(b: "DeviceBatch", out, n_units: int = 24) -> dict:
    """The fp8-KV decode against the float64 oracle on the values before
    quantisation (the bf16 caches), and against the oracle on the same codes,
    on sampled (sequence, KV head) units: max and mean absolute error."""
    import oracle
    w, s = b.w, b.w.spec
    rng = np.random.default_rng(9)
    units = np.unique(np.concatenate([rng.choice(s.num_seqs * s.num_kv_heads, min(n_units, s.num_seqs * s.num_kv_heads),
                                                 replace=False),
                                      [int(np.argmax(w.context_lens)) * s.num_kv_heads]]))
    bits = out.cpu().view(__import__("torch").int16).numpy().view(np.uint16)
    g = s.group
    got = np.stack([bits[u // s.num_kv_heads, (u % s.num_kv_heads) * g:(u % s.num_kv_heads + 1) * g] for u in units])
    got = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref_v = oracle.decode_workload(w, units=units)
    ref_c = oracle.decode_workload(w, units=units, kv_dtype=oracle.KV_FP8_E4M3FN, k_cache=b.kq, v_cache=b.vq,
                                   k_scale=b.k_scale, v_scale=b.v_scale)
    e_v, e_c = np.abs(got - ref_v), np.abs(got - ref_c)
    return {"units": int(len(units)), "vs_bf16_values": {"max": round(float(e_v.max()), 6),
                                                         "mean": round(float(e_v.mean()), 7)},
            "vs_fp8_codes": {"max": round(float(e_c.max()), 6), "mean": round(float(e_c.mean()), 7)}}


def per_config(args, dev, skip) -> list:
    """Decode of every other named configuration in this run, in both pool
    layouts (the page's [block, row, KV head, d] order and head-major)."""
    import torch
    from paged_kv_decode_mapping_amd import workloads as W
    res = []
    for name, kv, part in PER_CONFIG:
        if (name, kv, part) == skip:
            continue
        t0 = time.time()
        w = W.make_workload(name)
        nbytes = decode_bytes(w, 2 if kv == "bf16" else 1)
        entry = {"workload": f"{name}: {w.spec.description}", "kv_cache": kv, "partition_tokens_asked": part,
                 "bytes": nbytes, "layouts": {}}
        for layout in ("page", "head_major"):
            b = DeviceBatch(w, kv, layout, dev, host_codes=(kv == "fp8"))
            evict = b.unique_kv_bytes() < EVICT_BELOW_BYTES
            ms, plan, out = time_decode(b, dict(partition_tokens=part), max(args.steps, 20), args.warmup, evict)
            avg = float(ms.mean())
            gbps = nbytes / (avg * 1e-3) / 1e9
            entry["layouts"][layout] = {
                "plan": plan,
                "decode_us": {"avg": round(avg * 1e3, 2), "p10": round(float(np.percentile(ms, 10)) * 1e3, 2),
                              "p90": round(float(np.percentile(ms, 90)) * 1e3, 2)},
                "achieved_gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                "decode_tokens_per_s": round(w.spec.num_seqs / (avg * 1e-3), 1),
                "cache_evicted_between_launches": evict,
                "traffic": load_traffic(name, kv, plan, layout, part)}
            if kv == "fp8" and layout == "page":
                entry["fp8_accuracy"] = fp8_accuracy(b, out)
            if not args.no_cpu_baseline and layout == "page":
                entry["cpu_baseline"] = cpu_baseline(w, kv, b.kq, b.vq, min_s=2.0, budget_s=4.0)
            log(f"per-config {name} {kv} P={part} {layout}: {avg * 1e3:.1f} us, {gbps:.0f} GB/s = "
                f"{gbps / HBM_PEAK_GBPS:.1%}")
            del b, out
            torch.cuda.empty_cache()
        best = max(entry["layouts"], key=lambda k: entry["layouts"][k]["frac"])
        entry["best_layout"] = best
        entry["best_frac"] = entry["layouts"][best]["frac"]
        log(f"per-config {name} {kv} P={part}: best {best} ({time.time() - t0:.1f} s)")
        res.append(entry)
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50,
                    help="warm-up steps (at least; warm-up also lasts at least 0.2 s)")
    ap.add_argument("--workload", default="llama70b_gqa")
    ap.add_argument("--kv", choices=["bf16", "fp8"], default="bf16")
    ap.add_argument("--layout", choices=["page", "head_major"], default="page",
                    help="pool layout: the page's [block, row, KV head, d] order, or head-major "
                         "[block, KV head, row, d] passed through strides")
    ap.add_argument("--variant", default="auto")
    ap.add_argument("--partition", type=int, default=None,
                    help="tokens per split-K partition (default: the partition the workload names, "
                         "else the library's plan; -1 = never split)")
    ap.add_argument("--waves", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true", help="skip the other configurations")
    ap.add_argument("--prefetch", type=int, default=0)
    ap.add_argument("--schedule", type=int, default=0)
    ap.add_argument("--heads-per-tile", type=int, default=0, help="KV heads per MFMA tile (0 = the plan's choice)")
    ap.add_argument("--op", choices=["step", "copy_blocks", "multi", "graph", "stream", "cascade"], default="step",
                    help="step: cache write + decode (the default measurement); copy_blocks: time "
                         "pa_copy_blocks on the workload's pool; multi: time pa_decode_multi with "
                         "--qlen query tokens per sequence; graph: the step captured in a HIP graph, "
                         "replayed (eager step time reported beside it); stream: the streaming-read "
                         "reference: the library's probe kernel reading 4 GiB once, the practical read ceiling; "
                         "cascade: pa_decode_cascade on a workload with a shared prefix (mixed_batch), its "
                         "sharers as one group, pa_decode timed beside it")
    ap.add_argument("--qlen", type=int, default=4, help="query tokens per sequence for --op multi")
    ap.add_argument("--pairs", type=int, default=1024, help="block pairs per pa_copy_blocks call")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before timing, copy this many MiB device-to-device once (a plain copy kernel "
                         "of known size, the reference for hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the decode path runs on a single MI355X "
              "(no multi-GPU path is built); run it with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import paged_kv_decode_mapping_amd as pa
    from paged_kv_decode_mapping_amd import workloads as W

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    pa.load_library()
    dev = torch.device("cuda:0")
    if args.op == "stream":
        return bench_stream(args, dev)
    if args.partition is None:
        args.partition = W.SPECS[args.workload].partition_tokens if args.workload in W.SPECS else 0
    log(f"generating workload {args.workload} ({args.kv} KV, {args.layout} layout)")
    t0 = time.time()
    w = W.make_workload(args.workload)
    s = w.spec
    log(f"generated in {time.time() - t0:.1f} s: {s.num_seqs} seqs, pool {w.num_blocks} blocks, "
        f"{w.k_cache.nbytes / 1e9:.2f} GB per cache")
    b = DeviceBatch(w, args.kv, args.layout, dev, host_codes=(args.kv == "fp8"))
    q, k_cache, v_cache, tables, ctx = b.q, b.k_cache, b.v_cache, b.tables, b.ctx
    new_k, new_v, slots, k_scale, v_scale, kq, vq = b.new_k, b.new_v, b.slots, b.k_scale, b.v_scale, b.kq, b.vq
    kv_b = b.kv_b
    if args.op == "copy_blocks":
        return bench_copy_blocks(args, w, k_cache, v_cache, kv_b, kq, vq)
    if args.op == "multi":
        return bench_multi(args, w, k_cache, v_cache, tables, ctx, kv_b, k_scale, v_scale, kq, vq)
    if args.op == "cascade":
        return bench_cascade(args, w, k_cache, v_cache, kv_b, k_scale, v_scale, kq, vq)
    opts = dict(partition_tokens=args.partition, variant=args.variant, waves=args.waves, prefetch=args.prefetch,
                schedule=args.schedule, heads_per_tile=args.heads_per_tile)
    plan = pa.pa_decode_get_plan(q, k_cache, tables, **opts)
    log(f"plan {plan}")
    ws = torch.empty(max(plan["workspace_bytes"], 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    if args.op == "graph":
        return bench_graph(args, w, q, k_cache, v_cache, tables, ctx, new_k, new_v, slots, k_scale, v_scale,
                           plan, kv_b)

    def step(ev=None, mark_write=True):
        if ev is not None and mark_write:
            ev[0].record(stream)
        pa.pa_cache_write(new_k, new_v, slots, k_cache, v_cache, k_scale, v_scale)
        if ev is not None:
            ev[1].record(stream)
        pa.pa_decode(q, k_cache, v_cache, tables, ctx, w.scale, out, k_scale=k_scale, v_scale=v_scale,
                     workspace=ws, **opts)
        if ev is not None:
            ev[2].record(stream)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1, out=dst)  # an elementwise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        log(f"copy probe: {n} bytes read, {n} bytes written")
        del src, dst

    # the practical read ceiling on this GPU: the library's streaming-read
    # probe over 2 GiB with the decode kernels' non-temporal loads; run
    # first, it also brings the clocks up before the warm-up
    stream_gbps = stream_read_gbps(dev, 2 << 30, 10)
    log(f"streaming read {stream_gbps:.0f} GB/s")

    t_w = time.perf_counter()
    warm_up(step, args.warmup)
    warm_s = time.perf_counter() - t_w
    evict = b.unique_kv_bytes() < EVICT_BELOW_BYTES
    scratch = torch.zeros(512 << 20, dtype=torch.uint8, device=dev) if evict else None
    log(f"warm-up done ({warm_s * 1e3:.0f} ms); timing {args.steps} steps"
        + (" (caches evicted between steps)" if evict else ""))
    # The timed steps carry the decode's own events (its average launch time
    # is the roofline figure). Each event is a marker the GPU processes
    # between kernels (measured on the 70B batch: 3 markers a step 334 us,
    # 2 markers 329 us, none 322 us), so the write gets a leading marker only
    # when an eviction kernel runs before it and must be kept out of the
    # step; otherwise the step is the wall time and the write is timed in a
    # loop of its own afterwards.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        if scratch is not None:
            scratch.add_(1)
        step(events[i], mark_write=scratch is not None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    decode_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    if scratch is not None:  # the scratch writes are not part of the step
        write_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
        wall = float((write_ms + decode_ms).sum()) * 1e-3
    ms_per_step = wall * 1e3 / args.steps
    # after the timed steps, without eviction only: the write's own events,
    # and the step with no markers at all (reported beside the result)
    plain_us = None
    if scratch is None:
        wev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            step(wev[i])
        torch.cuda.synchronize()
        write_ms = np.array([e[0].elapsed_time(e[1]) for e in wev])
        t_plain = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        plain_us = round((time.perf_counter() - t_plain) * 1e6 / args.steps, 1)
    dec_b = decode_bytes(w, kv_b)
    wr_b = write_bytes(w, kv_b)
    dec_avg = float(decode_ms.mean())
    achieved = dec_b / (dec_avg * 1e-3) / 1e9
    step_gbps = (dec_b + wr_b) / (ms_per_step * 1e-3) / 1e9
    log(f"decode avg {dec_avg * 1e3:.1f} us (p10 {np.percentile(decode_ms, 10) * 1e3:.1f}, "
        f"p90 {np.percentile(decode_ms, 90) * 1e3:.1f}), write avg {write_ms.mean() * 1e3:.1f} us, "
        f"step {ms_per_step * 1e3:.1f} us, decode {achieved:.0f} GB/s = {achieved / HBM_PEAK_GBPS:.1%} of peak, "
        f"{achieved / stream_gbps:.1%} of the streaming read")

    acc = fp8_accuracy(b, out) if args.kv == "fp8" else None
    if acc:
        log(f"fp8 accuracy {acc}")
    base = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        base = cpu_baseline(w, args.kv, kq, vq)
        log(f"cpu baseline {base}")
    traffic = load_traffic(args.workload, args.kv, plan, args.layout, args.partition)
    tok_s = s.num_seqs / (ms_per_step * 1e-3)
    head = dict(workload=args.workload, kv=args.kv, part=args.partition)
    del b, q, k_cache, v_cache, out, ws
    torch.cuda.empty_cache()
    others = [] if args.no_per_config else per_config(args, dev, (head["workload"], head["kv"], head["part"]))
    res = {
        "metric": "paged decode attention achieved HBM GB/s (% of peak) + decode tokens/s",
        "value": round(step_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_ms": round(warm_s * 1e3, 1),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.kv,
        "data": "synthetic",
        "config": {
            "workload": f"{s.name}: {s.description}",
            "kv_cache": args.kv, "layout": args.layout,
            "num_seqs": s.num_seqs, "num_q_heads": s.num_q_heads, "num_kv_heads": s.num_kv_heads,
            "head_dim": s.head_dim, "block_size": s.block_size,
            "context_tokens": int(w.context_lens.sum()), "new_tokens": int(len(w.slot_mapping)),
            "plan": plan,
        },
        "pct_of_peak": round(step_gbps / HBM_PEAK_GBPS, 4),
        "decode_tokens_per_s": round(tok_s, 1),
        "decode_tokens_per_s_kernel": round(s.num_seqs / (dec_avg * 1e-3), 1),
        "decode_us": {"avg": round(dec_avg * 1e3, 2), "p10": round(float(np.percentile(decode_ms, 10)) * 1e3, 2),
                      "p90": round(float(np.percentile(decode_ms, 90)) * 1e3, 2)},
        "cache_write_us": round(float(write_ms.mean()) * 1e3, 2),
        "step_us_without_events": plain_us,
        "cache_evicted_between_steps": evict,
        "stream_read_gbps": round(stream_gbps, 1),
        "decode_frac_of_stream_read": round(achieved / stream_gbps, 4),
        "bytes": {"decode": dec_b, "cache_write": wr_b},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "pa_decode (decode kernel%s)" % (" + merge" if plan["num_partitions"] > 1 else "")},
        "fp8_accuracy": acc,
        "cpu_baseline": base,
        "per_config": others,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
