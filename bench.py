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


def load_traffic(workload: str, kv: str):
    """HBM traffic per decode launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", f"traffic_decode_{workload}_{kv}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    from paged_kv_decode_mapping_amd.profiling import kernel_source_hash
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(w, kv: str, kq=None, vq=None, budget_s: float = 12.0) -> dict:
    """Time the oracle on a bounded sample of (sequence, KV head) units."""
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
    while done < len(units_all) and t_total < budget_s:
        u = units_all[done:done + chunk]
        t0 = time.perf_counter()
        oracle.decode_workload(w, units=u, kv_dtype=kvd, k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs)
        t_total += time.perf_counter() - t0
        seqs = u // s.num_kv_heads
        ctx = w.context_lens[seqs].astype(np.int64)
        nbytes += int((2 * ctx * s.head_dim * e + 2 * s.group * s.head_dim * 2 + 4 * ((ctx + s.block_size - 1) // s.block_size)).sum())
        done += len(u)
    return {"value": round(nbytes / t_total / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{done} of {len(units_all)} (sequence, KV head) units, {t_total:.1f} s, "
                      f"float64 gather + softmax(qK^T)V, same byte model"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama70b_gqa")
    ap.add_argument("--kv", choices=["bf16", "fp8"], default="bf16")
    ap.add_argument("--variant", default="auto")
    ap.add_argument("--partition", type=int, default=0)
    ap.add_argument("--waves", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--check", action="store_true", help="compare sampled outputs with the oracle")
    ap.add_argument("--prefetch", type=int, default=0)
    ap.add_argument("--schedule", type=int, default=0)
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
    log(f"generating workload {args.workload} ({args.kv} KV)")
    t0 = time.time()
    w = W.make_workload(args.workload)
    s = w.spec
    log(f"generated in {time.time() - t0:.1f} s: {s.num_seqs} seqs, pool {w.num_blocks} blocks, "
        f"{w.k_cache.nbytes / 1e9:.2f} GB per cache")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q = bf16(w.q)
    k_cache = bf16(w.k_cache)
    v_cache = bf16(w.v_cache)
    tables = torch.from_numpy(w.block_tables).to(dev)
    ctx = torch.from_numpy(w.context_lens).to(dev)
    new_k, new_v = bf16(w.new_k), bf16(w.new_v)
    slots = torch.from_numpy(w.slot_mapping).to(dev)
    k_scale = v_scale = 1.0
    kq = vq = None
    if args.kv == "fp8":
        k_scale, v_scale = w.fp8_scales
        # quantise the whole pool on the GPU with the product's own cache write
        rows = w.num_blocks * s.block_size
        all_slots = torch.arange(rows, dtype=torch.int64, device=dev)
        kc8 = torch.empty((w.num_blocks, s.block_size, s.num_kv_heads, s.head_dim), dtype=torch.uint8, device=dev)
        vc8 = torch.empty_like(kc8)
        pa.pa_cache_write(k_cache.view(rows, s.num_kv_heads, s.head_dim), v_cache.view(rows, s.num_kv_heads, s.head_dim),
                          all_slots, kc8, vc8, k_scale, v_scale)
        torch.cuda.synchronize()
        del k_cache, v_cache
        k_cache, v_cache = kc8, vc8
        if not args.no_cpu_baseline:
            kq, vq = kc8.cpu().numpy(), vc8.cpu().numpy()
    kv_b = 2 if args.kv == "bf16" else 1
    plan = pa.pa_decode_get_plan(s.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim, s.block_size,
                                 w.max_blocks_per_seq, pa.PA_KV_BF16 if args.kv == "bf16" else pa.PA_KV_FP8_E4M3FN,
                                 partition_tokens=args.partition, variant=args.variant, waves=args.waves,
                                 prefetch=args.prefetch, schedule=args.schedule)
    log(f"plan {plan}")
    ws = torch.empty(max(plan["workspace_bytes"], 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        pa.pa_cache_write(new_k, new_v, slots, k_cache, v_cache, k_scale, v_scale)
        if ev is not None:
            ev[1].record(stream)
        pa.pa_decode(q, k_cache, v_cache, tables, ctx, w.scale, out, k_scale=k_scale, v_scale=v_scale,
                     workspace=ws, partition_tokens=args.partition, variant=args.variant, waves=args.waves,
                     prefetch=args.prefetch, schedule=args.schedule)
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    write_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    decode_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    ms_per_step = wall * 1e3 / args.steps
    dec_b = decode_bytes(w, kv_b)
    wr_b = write_bytes(w, kv_b)
    dec_avg = float(decode_ms.mean())
    achieved = dec_b / (dec_avg * 1e-3) / 1e9
    step_gbps = (dec_b + wr_b) / (ms_per_step * 1e-3) / 1e9
    log(f"decode avg {dec_avg * 1e3:.1f} us (p10 {np.percentile(decode_ms, 10) * 1e3:.1f}, "
        f"p90 {np.percentile(decode_ms, 90) * 1e3:.1f}), write avg {write_ms.mean() * 1e3:.1f} us, "
        f"step {ms_per_step * 1e3:.1f} us, decode {achieved:.0f} GB/s = {achieved / HBM_PEAK_GBPS:.1%} of peak")

    check = None
    if args.check:
        import oracle
        units = np.random.default_rng(9).choice(s.num_seqs * s.num_kv_heads, 32, replace=False)
        pa.pa_decode(q, k_cache, v_cache, tables, ctx, w.scale, out, k_scale=k_scale, v_scale=v_scale,
                     workspace=ws, partition_tokens=args.partition, variant=args.variant, waves=args.waves,
                     prefetch=args.prefetch, schedule=args.schedule)
        got = out.cpu().view(torch.int16).numpy().view(np.uint16)
        kvd = oracle.KV_BF16 if args.kv == "bf16" else oracle.KV_FP8_E4M3FN
        if args.kv == "fp8" and kq is None:
            kq, vq = k_cache.cpu().numpy(), v_cache.cpu().numpy()
        ref = oracle.decode_workload(w, units=units, kv_dtype=kvd, k_cache=kq, v_cache=vq,
                                     k_scale=k_scale, v_scale=v_scale)
        g = s.group
        errs = []
        for n, u in enumerate(units):
            i, kh = divmod(int(u), s.num_kv_heads)
            gv = (got[i, kh * g:(kh + 1) * g].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            errs.append(np.abs(gv - ref[n]))
        errs = np.stack(errs)
        check = {"units": len(units), "max_abs": float(errs.max()), "mean_abs": float(errs.mean())}
        log(f"check vs oracle on {len(units)} units: {check}")

    base = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        base = cpu_baseline(w, args.kv, kq, vq)
        log(f"cpu baseline {base}")

    traffic = load_traffic(args.workload, args.kv)
    tok_s = s.num_seqs / (ms_per_step * 1e-3)
    res = {
        "metric": "paged decode attention achieved HBM GB/s (% of peak) + decode tokens/s",
        "value": round(step_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.kv,
        "data": "synthetic",
        "config": {
            "workload": f"{s.name}: {s.description}",
            "kv_cache": args.kv,
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
        "bytes": {"decode": dec_b, "cache_write": wr_b},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "pa_decode (decode kernel%s)" % (" + merge" if plan["num_partitions"] > 1 else "")},
        "cpu_baseline": base,
    }
    if check is not None:
        res["check"] = check
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
