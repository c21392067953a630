"""GPU parity of multi-token paged attention (pa_decode_multi) and of
pa_decode with more than 16 query heads per KV head (MQA), against the
float64 oracle, through the C ABI. Tolerances as for decode: max |err|
1e-2, mean 1e-3 with bf16 KV; 5e-2 / 5e-3 with fp8 KV (same cache codes).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_mapping_amd as pa
from paged_kv_decode_mapping_amd import workloads as W

from _gpu_util import DeviceWorkload, bf16_to_f64, compare, host_bits, note

pytestmark = pytest.mark.gpu

BF16_TOL = (1e-2, 1e-3)
FP8_TOL = (5e-2, 5e-3)


@pytest.fixture(scope="module")
def lib(gpu):
    return pa.load_library()


CASES = {
    # name: (workload kwargs, query lengths)
    "tiny_mixed_lengths": ("tiny", dict(), [1, 5, 16, 4]),
    "spec_verify_70b": ("llama70b_gqa", dict(num_seqs=3, context=("list", [4096, 1234, 17])), [4, 4, 4]),
    "spec_verify_mixed": ("mixed_batch", dict(num_seqs=6, context=("list", [16, 100, 511, 900, 3000, 77])),
                          [8, 1, 8, 5, 8, 0]),
    "chunk_prefill": ("mixed_batch", dict(num_seqs=3, context=("list", [600, 1500, 100])), [100, 37, 100]),
    "long_bs128": ("long_splitk", dict(num_seqs=2, context=("list", [5000, 2049])), [16, 3]),
    "mha_multi": ("llama7b_mha", dict(num_seqs=3, context=("list", [512, 1000, 33])), [6, 2, 33]),
    # 128 rows per KV head: one workgroup of 4 waves x 32 rows
    "verify16_70b": ("llama70b_gqa", dict(num_seqs=2, context=("list", [300, 2000])), [16, 9]),
    # groups and block sizes the named workloads do not have
    "g3_bs32": ("tiny", dict(num_seqs=3, context=("list", [40, 300, 1000]), num_q_heads=12, num_kv_heads=4,
                             head_dim=128, block_size=32), [3, 7, 16]),
    "g12_bs1024": ("long_splitk", dict(num_seqs=2, context=("list", [1100, 2500]), num_q_heads=96, block_size=1024),
                   [5, 16]),
    "g6_d64_bs64": ("tiny", dict(num_seqs=3, context=("list", [64, 65, 500]), num_q_heads=12, num_kv_heads=2,
                                 block_size=64), [1, 11, 4]),
}


def _run(name, partition=0, kv="bf16"):
    base, kw, qlens = CASES[name]
    w = W.make_workload(base, **kw)
    mq = W.make_multi_query(w, qlens)
    kc, vc, ks, vs = w.k_cache, w.v_cache, 1.0, 1.0
    kvd = oracle.KV_BF16
    if kv == "fp8":
        ks, vs = w.fp8_scales
        kc, vc = oracle.quantize_pool(kc, ks), oracle.quantize_pool(vc, vs)
        kvd = oracle.KV_FP8_E4M3FN
    ref = oracle.multi_decode(mq.q, kc, vc, w.block_tables, w.context_lens, mq.query_start, w.scale,
                              kv_dtype=kvd, k_scale=ks, v_scale=vs)
    d = DeviceWorkload(w, kc, vc)
    q = torch.from_numpy(mq.q.view(np.int16)).view(torch.bfloat16).cuda()
    qs = torch.from_numpy(mq.query_start).cuda()
    note(f"multi {name} kv={kv} partition={partition} qlens={qlens}")
    out = pa.pa_decode_multi(q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, qs, w.scale,
                             int(max(qlens)), k_scale=ks, v_scale=vs, partition_tokens=partition)
    torch.cuda.synchronize()
    return host_bits(out), ref


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("partition", [0, -1, 512])
def test_multi_matches_oracle(lib, name, partition):
    got, ref = _run(name, partition)
    compare(got, ref, *BF16_TOL)


@pytest.mark.parametrize("name", ["spec_verify_mixed", "long_bs128", "verify16_70b", "chunk_prefill",
                                  "g3_bs32", "g12_bs1024", "g6_d64_bs64"])
def test_multi_fp8_matches_oracle(lib, name):
    got, ref = _run(name, 0, "fp8")
    compare(got, ref, *FP8_TOL)


def test_multi_small_partitions_and_ragged_tiles(lib):
    """Partitions of one tile: every query row merges many partials, rows
    whose position ends inside a tile mask the rest of it."""
    got, ref = _run("tiny_mixed_lengths", 16)
    compare(got, ref, *BF16_TOL)
    got, ref = _run("chunk_prefill", 48)
    compare(got, ref, *BF16_TOL)
    got, ref = _run("long_bs128", 16)  # more than a hundred partitions per row: the widest merge
    compare(got, ref, *BF16_TOL)


def test_multi_one_token_equals_decode_oracle(lib):
    """With one query token per sequence the operation is decode."""
    w = W.make_workload("mixed_batch", num_seqs=5, context=("list", [1, 16, 17, 700, 2049]))
    mq = W.make_multi_query(w, [1] * 5)
    d = DeviceWorkload(w)
    q = torch.from_numpy(mq.q.view(np.int16)).view(torch.bfloat16).cuda()
    note("multi n=1")
    out = pa.pa_decode_multi(q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                             torch.from_numpy(mq.query_start).cuda(), w.scale, 1)
    ref = oracle.decode(mq.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale)
    compare(host_bits(out), ref, *BF16_TOL)


def test_multi_last_row_of_full_context_equals_decode_bits(lib):
    """Query r = n - 1 sees the whole context; r = 0 with n = L sees one
    token, so its output is that token's V row exactly."""
    w = W.make_workload("tiny")
    L = w.context_lens.astype(int)
    mq = W.make_multi_query(w, L.tolist())  # every cached token is a query
    d = DeviceWorkload(w)
    q = torch.from_numpy(mq.q.view(np.int16)).view(torch.bfloat16).cuda()
    note("multi n=L")
    got = host_bits(pa.pa_decode_multi(q, d.k_cache, d.v_cache, d.block_tables, d.context_lens,
                                       torch.from_numpy(mq.query_start).cuda(), w.scale, int(L.max())))
    torch.cuda.synchronize()
    g = w.spec.group
    for i in range(w.spec.num_seqs):
        row0 = int(mq.query_start[i])
        b = w.block_tables[i, 0]
        for h in range(w.spec.num_q_heads):
            assert np.array_equal(got[row0, h], w.v_cache[b, 0, h // g])
    ref = oracle.multi_decode(mq.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, mq.query_start, w.scale)
    compare(got, ref, *BF16_TOL)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 1, 128), (64, 1, 64), (64, 2, 128), (48, 2, 128)])
@pytest.mark.parametrize("partition", [0, -1, 256])
def test_decode_mqa_wide_groups(lib, Hq, Hkv, D, partition):
    """pa_decode with g > 16 (MQA): routed to the multi-row kernel."""
    w = W.make_workload("mixed_batch", num_seqs=5, context=("list", [1, 16, 300, 1000, 2100]),
                        num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D)
    ref = oracle.decode_workload(w)
    d = DeviceWorkload(w)
    note(f"mqa Hq={Hq} Hkv={Hkv} D={D} partition={partition}")
    plan = pa.pa_decode_get_plan(d.q, d.k_cache, d.block_tables, partition_tokens=partition)
    assert plan["variant"] == "mfma"
    got = host_bits(d.decode(partition_tokens=partition))
    torch.cuda.synchronize()
    compare(got, ref, *BF16_TOL)
    if plan["num_partitions"] > 1:
        # the builder's list, the workgroups' own ranking and the direct grid: the same bits
        for schedule in (1, 2, -1):
            assert np.array_equal(host_bits(d.decode(partition_tokens=partition, schedule=schedule)), got)


@pytest.mark.parametrize("shape", ["rows128", "mqa"])
@pytest.mark.parametrize("scale", [0.0, 1.0, 8.0, 64.0, -8.0])
def test_multi_extreme_logits_and_a_moving_max(lib, shape, scale):
    """The multi-row kernel's online softmax under stress. In every sequence
    the keys of each KV head are aligned with the query of the head's first
    row and grow with the position, so that row's running maximum climbs on
    every tile: across a 32-token step by less than the kernel's lazy-rescale
    slack on the long contexts (probabilities above 1 against an older
    reference) and by more on the short ones (a rescale every step); scale 64
    makes the softmax nearly one-hot, scale 0 gives the mean of V, scale -8
    favours the smallest scores (the earliest tokens for those rows). 128 rows
    per KV head (waves of two row tiles) through pa_decode_multi, and MQA
    (64 heads on one KV head) through pa_decode; unsplit and split.

    V is the workload's scaled by 1/4 (exact in bf16): a nearly one-hot row
    returns about one V element, and for |x| >= 4 one rounding to bf16
    alone can miss x by up to 1/64 > 1e-2, so full-size V would test the
    output format rather than the softmax."""
    ctx = [40, 300, 1000, 2100]
    if shape == "rows128":
        w = W.make_workload("llama70b_gqa", num_seqs=len(ctx), context=("list", ctx))
        qlens = [16, 16, 9, 16]
    else:
        w = W.make_workload("mixed_batch", num_seqs=len(ctx), context=("list", ctx), num_q_heads=64,
                            num_kv_heads=1)
        qlens = [1] * len(ctx)
    mq = W.make_multi_query(w, qlens)
    q32 = W.bf16_bits_to_f32(mq.q)
    g, bs = w.spec.group, w.spec.block_size
    kc = w.k_cache.copy()
    for i, L in enumerate(ctx):
        js = np.arange(L)
        blocks, offs = w.block_tables[i, js // bs], js % bs
        f = (np.float32(0.5) * (js + 1) / L).astype(np.float32)
        for h in range(w.spec.num_kv_heads):
            kc[blocks, offs, h] = W._to_bf16_bits(q32[mq.query_start[i], h * g][None, :] * f[:, None])
    vc = W._to_bf16_bits(W.bf16_bits_to_f32(w.v_cache) * np.float32(0.25))
    ref = oracle.multi_decode(mq.q, kc, vc, w.block_tables, w.context_lens, mq.query_start, scale)
    d = DeviceWorkload(w, kc, vc)
    q = torch.from_numpy(mq.q.view(np.int16)).view(torch.bfloat16).cuda()
    qs = torch.from_numpy(mq.query_start).cuda()
    for part in (-1, 64):
        note(f"multi extreme logits {shape} scale={scale} partition={part}")
        if shape == "rows128":
            out = pa.pa_decode_multi(q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, qs, scale,
                                     int(max(qlens)), partition_tokens=part)
        else:
            out = pa.pa_decode(q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, scale,
                               partition_tokens=part)
        torch.cuda.synchronize()
        compare(host_bits(out), ref, *BF16_TOL)


@pytest.mark.parametrize("layout", ["dense", "sparse"])
def test_multi_split_merge_grids(lib, layout):
    """The split merge of pa_decode_multi, both grids: rows that see partition
    0 only are finished by the kernel, the others merged. With queries on
    every sequence ("dense": 24 sequences x 8 queries x 32 heads, D 128) the
    merge walks (sequence, head, block of 8 rows): 24 * 32 * 1 blocks against
    192 * 32 * 32 / 256 by rows. With queries on 2 of 64 sequences
    ("sparse") that grid would be 64 * 32 * 2 blocks against 32 * 32 * 32 /
    256, so the merge walks the rows. 512-token partitions over contexts of
    17 to 3000 tokens: rows see 1 to 6 partitions, few enough for the flat
    merge (one thread per float4 column of a row)."""
    rng = np.random.default_rng(11)
    if layout == "dense":
        S = 24
        ctx = rng.integers(17, 3000, size=S)
        qlens = [8] * S
    else:
        S = 64
        ctx = rng.integers(17, 3000, size=S)
        qlens = [0] * S
        qlens[5], qlens[40] = 16, 16
    w = W.make_workload("mixed_batch", num_seqs=S, context=("list", [int(x) for x in ctx]))
    mq = W.make_multi_query(w, qlens)
    ref = oracle.multi_decode(mq.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, mq.query_start, w.scale)
    d = DeviceWorkload(w)
    q = torch.from_numpy(mq.q.view(np.int16)).view(torch.bfloat16).cuda()
    qs = torch.from_numpy(mq.query_start).cuda()
    note(f"multi split merge {layout}")
    out = pa.pa_decode_multi(q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, qs, w.scale,
                             int(max(qlens)), partition_tokens=512)
    torch.cuda.synchronize()
    compare(host_bits(out), ref, *BF16_TOL)


@pytest.mark.parametrize("S", [256, 300])
def test_multi_rows_ordered_by_the_workgroups_or_the_list(lib, S):
    """Split multi-row items, longest first: ranked by each workgroup itself
    up to 256 sequences (with MQA heads through pa_decode, schedule = 2), by
    the builder's list beyond (300) or when asked (schedule = 1); ragged
    and zero lengths; the same bits as the direct grid and the oracle."""
    rng = np.random.default_rng(S)
    ctx = [int(x) for x in rng.integers(0, 700, size=S)]
    ctx[0], ctx[1] = 0, 699
    w = W.make_workload("mixed_batch", num_seqs=S, context=("list", ctx), num_q_heads=32, num_kv_heads=1,
                        head_dim=64, shared_prefix_tokens=0)
    ref = oracle.decode_workload(w)
    d = DeviceWorkload(w)
    outs = {}
    for schedule in (0, 1, 2, -1):
        plan = pa.pa_decode_get_plan(d.q, d.k_cache, d.block_tables, partition_tokens=64, schedule=schedule)
        assert plan["num_partitions"] > 1
        if schedule == 0:
            assert plan["self_scheduled"] == (S <= 256 and S * plan["num_partitions"] <= 1024)
        if schedule == 2:
            assert plan["self_scheduled"] == (S <= 256)
        note(f"multi-row order S={S} schedule={schedule} plan={plan}")
        outs[schedule] = host_bits(d.decode(partition_tokens=64, schedule=schedule))
    compare(outs[0], ref, *BF16_TOL)
    for schedule in (1, 2, -1):
        assert np.array_equal(outs[schedule], outs[0])
    # pa_decode_multi (several query tokens) on the same batch, with its own plan
    qlens = [min(int(x), c) for x, c in zip(rng.integers(0, 4, size=S), ctx)]
    mq = W.make_multi_query(w, qlens)
    q = torch.from_numpy(mq.q.view(np.int16)).view(torch.bfloat16).cuda()
    qs = torch.from_numpy(mq.query_start).cuda()
    note(f"multi-row order S={S} pa_decode_multi")
    got = host_bits(pa.pa_decode_multi(q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, qs, w.scale,
                                       int(max(qlens)), partition_tokens=64))
    mref = oracle.multi_decode(mq.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, mq.query_start, w.scale)
    compare(got, mref, *BF16_TOL)


def _sampled_units(w, n, seed):
    """n random (sequence, KV head) units plus every unit of the longest and
    the shortest context."""
    s = w.spec
    rng = np.random.default_rng(seed)
    extra = [int(np.argmax(w.context_lens)), int(np.argmin(w.context_lens))]
    units = rng.choice(s.num_seqs * s.num_kv_heads, n, replace=False).tolist()
    units += [i * s.num_kv_heads + k for i in extra for k in range(s.num_kv_heads)]
    return np.unique(np.asarray(units, dtype=np.int64))


@pytest.mark.parametrize("name,qlen", [("llama70b_gqa", 16), ("mixed_batch", 32), ("llama70b_gqa", 4)])
def test_full_size_multi_sampled(lib, name, qlen):
    """pa_decode_multi at the full size and in the launch configuration the
    benchmark times (the last qlen cached tokens of every sequence are its
    queries; the library's own plan), checked on sampled (sequence, KV
    head) units, the longest and the shortest context included, that the
    oracle computes one by one."""
    w = W.make_workload(name)
    qlens = np.minimum(np.full(w.spec.num_seqs, qlen), w.context_lens)
    mq = W.make_multi_query(w, qlens)
    d = DeviceWorkload(w)
    q = torch.from_numpy(mq.q.view(np.int16)).view(torch.bfloat16).cuda()
    qs = torch.from_numpy(mq.query_start).cuda()
    plan = pa.pa_decode_get_plan(d.q, d.k_cache, d.block_tables)
    note(f"full-size multi {name} qlen={qlen} decode plan={plan}")
    got = bf16_to_f64(host_bits(pa.pa_decode_multi(q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, qs,
                                                    w.scale, int(qlens.max()))))
    torch.cuda.synchronize()
    units = _sampled_units(w, 12, qlen)
    ref = oracle.multi_decode(mq.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, mq.query_start, w.scale,
                              units=units)
    mask = ~np.isnan(ref)
    assert mask.sum() > 0
    err = np.abs(got[mask] - ref[mask])
    assert np.all(np.isfinite(got[mask]))
    assert err.max() <= BF16_TOL[0] and err.mean() <= BF16_TOL[1], (err.max(), err.mean())


def test_full_size_mqa_sampled(lib):
    """The MQA batch (128 sequences of 4096 tokens, 64 query heads on one KV
    head) through pa_decode's multi-row route, at full size with the
    library's own plan, on sampled sequences the oracle computes one by
    one."""
    w = W.make_workload("mqa_70b")
    d = DeviceWorkload(w)
    plan = pa.pa_decode_get_plan(d.q, d.k_cache, d.block_tables)
    note(f"full-size mqa plan={plan}")
    out = host_bits(d.decode())
    torch.cuda.synchronize()
    units = _sampled_units(w, 10, 5)
    ref = oracle.decode_workload(w, units=units)  # [n_units, g, D]
    g = w.spec.num_q_heads // w.spec.num_kv_heads
    got = np.stack([out[u // w.spec.num_kv_heads, (u % w.spec.num_kv_heads) * g:(u % w.spec.num_kv_heads + 1) * g]
                    for u in units])
    compare(got, ref, *BF16_TOL)
