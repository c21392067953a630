"""The rocprofv3 summary tool on small synthetic CSVs (no GPU)."""
import json
import os

from paged_kv_decode_mapping_amd import profiling


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(f'"{x}"' if isinstance(x, str) else str(x) for x in r) + "\n")


def test_stats_summary(tmp_path):
    d = tmp_path / "prof"
    _write(str(d / "host" / "123" / "x_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
           [["void pa::(anonymous namespace)::pa_decode_mfma_kernel<128, false, 3>(pa::DecodeArgs)", 20, 7600000, 380000, 97.0, 370000, 390000, 1.0],
            ["void pa::(anonymous namespace)::pa_cache_write_kernel<false>(pa::CacheWriteArgs)", 20, 140000, 7000, 3.0, 6000, 8000, 1.0]])
    out = tmp_path / "s.md"
    rows = profiling.stats(str(d))
    assert rows[0]["calls"] == 20 and rows[0]["avg_ns"] == 380000
    class A:  # argparse stand-in
        dir, cmd, title = str(d), "rocprofv3 ... -- python bench.py", "t"
    A.out = str(out)
    profiling.cmd_stats(A)
    text = out.read_text()
    assert "pa_decode_mfma_kernel<128, false, 3>" in text and "380.00" in text


def test_traffic_scaling(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    copy = "void at::native::elementwise_kernel<...>(int)"
    dec = "void pa::(anonymous namespace)::pa_decode_mfma_kernel<128, false, 3>(pa::DecodeArgs)"
    # counters read in KiB: the copy of 1 MiB reads 1024 KiB and writes 1024 KiB
    idx = "void at::native::elementwise_kernel_with_index<int, arange>(int)"  # a small helper kernel first
    _write(str(tmp_path / "f" / "a_counter_collection.csv"), hdr,
           [[0, idx, "FETCH_SIZE", 3.0], [1, copy, "FETCH_SIZE", 1024.0], [2, dec, "FETCH_SIZE", 2000.0],
            [3, dec, "FETCH_SIZE", 2100.0]])
    _write(str(tmp_path / "w" / "a_counter_collection.csv"), hdr,
           [[0, idx, "WRITE_SIZE", 8.0], [1, copy, "WRITE_SIZE", 1024.0], [2, dec, "WRITE_SIZE", 10.0],
            [3, dec, "WRITE_SIZE", 12.0]])
    class A:
        fetch_dir, write_dir = str(tmp_path / "f"), str(tmp_path / "w")
        out = str(tmp_path / "t.json")
        workload, kv, copy_bytes, cmd = "w", "bf16", 1 << 20, "c"
        layout, partition, bench_log = "head_major", 0, ""
    profiling.cmd_traffic(A)
    r = json.load(open(A.out))
    assert r["fetch_bytes_per_launch"] == 2100.0 * 1024
    assert r["write_bytes_per_launch"] == 12.0 * 1024
    assert r["kernel_source_hash"] == profiling.kernel_source_hash()
    assert r["plan"] is None  # unknown workload: no plan, so bench.py never reports this figure
    assert r["layout"] == "head_major"
    assert profiling.traffic_file("w", "fp8", "head_major", 512).endswith("traffic_decode_w_fp8_head_major_p512.json")
    assert profiling.traffic_file("w", "bf16").endswith("traffic_decode_w_bf16.json")


def test_source_hash_follows_the_plan():
    """A plan's hash covers the kernels it launches: the work-list builder
    only when scheduled, the merge only when split, one decode kernel."""
    base = {"variant": "mfma", "scheduled": False, "num_partitions": 1}
    h = profiling.kernel_source_hash(base)
    assert h == profiling.kernel_source_hash(dict(base))
    assert h != profiling.kernel_source_hash(dict(base, variant="valu"))
    assert h != profiling.kernel_source_hash(dict(base, scheduled=True))
    assert h != profiling.kernel_source_hash(dict(base, num_partitions=2))
    assert profiling.kernel_source_hash() not in (h, profiling.kernel_source_hash(dict(base, scheduled=True)))
