"""Turn rocprofv3 output into the short text summaries kept under profiles/.

    python -m paged_kv_decode_mapping_amd.profiling stats  <rocprof dir> <out.md> --cmd "<command>"
    python -m paged_kv_decode_mapping_amd.profiling traffic <fetch dir> <write dir> <out.json> \
        --workload NAME --kv bf16 [--layout head_major] [--partition P] --copy-bytes N --cmd "<commands>"

`stats` reads the kernel statistics CSV of a `rocprofv3 --kernel-trace
--stats --output-format csv` run. `traffic` reads the counter-collection CSVs
of two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of the same
command (which starts with a device copy of `copy-bytes` bytes), scales each
counter by what it reads for that copy (bytes moved / counter value), and
writes the HBM bytes per decode launch, tagged with a hash of the kernel
sources so that a stale figure is not reported after the kernels change.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict
from typing import Optional

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# What decides the decode kernels' traffic: their sources, the headers they
# include, and the argument blocks they receive. The launch plan (waves,
# tiles in flight, partitions) is stored next to the figure and compared
# separately, so host-side changes elsewhere do not invalidate it. With a
# plan, only the kernels it launches count: the work-list builder when it
# uses a device-built list, the merge when it splits contexts.
COMMON_SOURCES = ("pa_epilogue.h", "pa_device.h")
KERNEL_SOURCES = {"mfma": "decode_mfma.hip", "valu": "decode_valu.hip"}
COMMON_STRUCTS = ("DecodeArgs", "LaunchShape")


def _struct_text(src: str, name: str) -> str:
    i = src.index("struct " + name + " {")
    return src[i:src.index("};", i) + 2]


def kernel_source_hash(plan: Optional[dict] = None) -> str:
    """Hash of what the decode launches of `plan` run (every decode kernel,
    the builder and the merge when no plan is given)."""
    files = list(COMMON_SOURCES)
    structs = list(COMMON_STRUCTS)
    variants = [plan["variant"]] if plan else sorted(KERNEL_SOURCES)
    files += [KERNEL_SOURCES[v] for v in variants]
    if plan is None or (plan.get("scheduled") and not plan.get("self_scheduled")):
        files += ["schedule.hip", "pa_cascade.h"]
        structs.append("ScheduleArgs")
    if plan is None or plan.get("num_partitions", 1) > 1:
        files += ["merge.hip", "pa_merge.h", "pa_cascade.h"]
        structs.append("MergeArgs")
    files = list(dict.fromkeys(files))
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_decode_mapping_amd", "csrc")
    for f in files:
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    internal = open(os.path.join(csrc, "pa_internal.h")).read()
    for name in structs:
        h.update(_struct_text(internal, name).encode())
    return h.hexdigest()[:16]


def decode_plan(workload: str, kv: str, layout: str = "page", partition_tokens: int = 0) -> dict:
    """The launch plan pa_decode uses for a named workload on this GPU, with
    the page's pool layout or the head-major one, and the default partition
    choice or a given partition size."""
    import paged_kv_decode_mapping_amd as pa
    from paged_kv_decode_mapping_amd import workloads as W
    s = W.SPECS[workload]
    ctx = s.context
    cap = {"const": lambda: ctx[1], "uniform": lambda: ctx[2], "lognormal": lambda: ctx[4],
           "list": lambda: max(ctx[1])}[ctx[0]]()
    mb = -(-int(cap) // s.block_size)
    specs = pa.decode_specs(s.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim, s.block_size, mb,
                            pa.PA_KV_BF16 if kv == "bf16" else pa.PA_KV_FP8_E4M3FN,
                            head_major=(layout == "head_major"))
    return pa.pa_decode_get_plan(*specs, partition_tokens=partition_tokens)


def traffic_file(workload: str, kv: str, layout: str = "page", partition_tokens: int = 0) -> str:
    """Name of the committed traffic summary of a decode configuration."""
    tag = ("" if layout == "page" else "_" + layout) + ("" if partition_tokens == 0 else f"_p{partition_tokens}")
    return os.path.join(ROOT, "profiles", f"traffic_decode_{workload}_{kv}{tag}.json")


def _plan_or_none(workload: str, kv: str, layout: str = "page", partition_tokens: int = 0):
    try:
        return decode_plan(workload, kv, layout, partition_tokens)
    except Exception:  # unknown workload, or no GPU to plan for: the figure is then never reported
        return None


def _plan_from_log(path: str):
    """The launch plan a profiled bench.py run printed in its JSON line."""
    for line in reversed(open(path).read().splitlines()):
        if line.startswith("{"):
            return json.loads(line).get("config", {}).get("plan")
    return None


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[-1]


def _short(name: str) -> str:
    n = name
    for p in ("void ", "(anonymous namespace)::", "pa::"):
        n = n.replace(p, "")
    return n.split("(")[0].strip()


def stats(d: str) -> list:
    rows = []
    with open(_find(d, "kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append({"name": r.get("Name", ""), "calls": int(float(r.get("Calls", 0))),
                         "total_ns": float(r.get("TotalDurationNs", 0)), "avg_ns": float(r.get("AverageNs", 0)),
                         "min_ns": float(r.get("MinNs", 0)), "max_ns": float(r.get("MaxNs", 0)),
                         "pct": float(r.get("Percentage", 0))})
    rows.sort(key=lambda r: -r["total_ns"])
    return rows


def last_dispatches(d: str, n: int) -> list:
    """Per kernel, statistics over its last n dispatches (in dispatch order)
    from the kernel trace CSV: the timed steps of a benchmark run, without
    its warm-up."""
    per = defaultdict(list)
    with open(_find(d, "kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            per[r["Kernel_Name"]].append((int(r["Dispatch_Id"]),
                                          float(r["End_Timestamp"]) - float(r["Start_Timestamp"])))
    rows = []
    for name, ds in per.items():
        ds.sort()
        t = [x for _, x in ds[-n:]]
        rows.append({"name": name, "calls": len(t), "total_ns": sum(t), "avg_ns": sum(t) / len(t),
                     "min_ns": min(t), "max_ns": max(t)})
    total = sum(r["total_ns"] for r in rows) or 1.0
    for r in rows:
        r["pct"] = 100.0 * r["total_ns"] / total
    rows.sort(key=lambda r: -r["total_ns"])
    return rows


def counters(d: str) -> dict:
    """{kernel name: {counter: [value per dispatch]}}"""
    out = defaultdict(lambda: defaultdict(list))
    with open(_find(d, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            out[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return out


def cmd_stats(a) -> None:
    last = getattr(a, "last", 0) or 0
    rows = last_dispatches(a.dir, last) if last > 0 else stats(a.dir)
    head = ([f"Last {last} dispatches of each kernel (the timed steps), from the per-dispatch kernel trace.", ""]
            if last > 0 else [])
    lines = [f"# {a.title}", "", "Command:", "", "```", a.cmd, "```", ""] + head + [
             "| kernel | calls | avg µs | min µs | max µs | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{_short(r['name'])}` | {r['calls']} | {r['avg_ns'] / 1e3:.2f} | {r['min_ns'] / 1e3:.2f} | "
                     f"{r['max_ns'] / 1e3:.2f} | {r['pct']:.1f} |")
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_traffic(a) -> None:
    fetch = counters(a.fetch_dir)
    write = counters(a.write_dir)

    def pick(cs, key_sub, counter):
        for k, v in cs.items():
            if key_sub in k and counter in v:
                return k, v[counter]
        raise KeyError(f"{key_sub} / {counter} not in the counter CSV: {list(cs)}")

    # the copy kernel: of the kernels outside the library, the one that reads
    # the most (the 1 GiB copy; fills read nothing, index helpers little)
    others = [k for k in fetch if "pa_" not in k and "FETCH_SIZE" in fetch[k] and k in write]
    copy_name = max(others, key=lambda k: fetch[k]["FETCH_SIZE"][0])
    cf = fetch[copy_name]["FETCH_SIZE"][0]
    cw = write[copy_name]["WRITE_SIZE"][0]
    f_scale = a.copy_bytes / cf
    w_scale = a.copy_bytes / cw
    dname, dfetch = pick(fetch, "pa_decode_", "FETCH_SIZE")
    _, dwrite = pick(write, "pa_decode_", "WRITE_SIZE")
    fb = sorted(dfetch)[len(dfetch) // 2] * f_scale
    wb = sorted(dwrite)[len(dwrite) // 2] * w_scale
    res = {"workload": a.workload, "kv": a.kv, "kernel": _short(dname),
           "copy_kernel": _short(copy_name), "copy_bytes": a.copy_bytes,
           "fetch_counter_per_copy_byte": cf / a.copy_bytes, "write_counter_per_copy_byte": cw / a.copy_bytes,
           "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb, "bytes_per_launch": fb + wb,
           "dispatches": len(dfetch)}
    plan = _plan_from_log(a.bench_log) if a.bench_log else _plan_or_none(a.workload, a.kv, a.layout, a.partition)
    res.update({"layout": a.layout, "partition_tokens_asked": a.partition,
                "kernel_source_hash": kernel_source_hash(plan), "plan": plan, "command": a.cmd})
    json.dump(res, open(a.out, "w"), indent=1)
    print(json.dumps(res, indent=1))


def main() -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("out")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="rocprofv3 kernel statistics")
    s.add_argument("--last", type=int, default=0,
                   help="summarise each kernel's last N dispatches only (the timed steps)")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("out")
    t.add_argument("--workload", required=True)
    t.add_argument("--kv", default="bf16")
    t.add_argument("--layout", choices=["page", "head_major"], default="page")
    t.add_argument("--partition", type=int, default=0, help="partition size asked for (0 = the plan's choice)")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--bench-log", default="",
                   help="output of one of the profiled bench.py runs: its plan is the one recorded "
                        "(else the plan is asked of the library on this machine)")
    t.add_argument("--cmd", required=True)
    a = ap.parse_args()
    cmd_stats(a) if a.what == "stats" else cmd_traffic(a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
