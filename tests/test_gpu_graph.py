"""GPU tests: the write + decode step captured in a HIP graph (through
torch.cuda.CUDAGraph) at a bucketed batch size, replayed with new inputs.

The library calls allocate nothing and never synchronise, so a caller can
capture them. Batches smaller than the bucket are padded: padding sequences
have context length 0 (zero output) and slot -1 (nothing written). Every
replay is checked against the same step run eagerly on a second copy of the
caches (bit-identical outputs and caches), with eager work and
synchronisations between the replays, and one replay against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_mapping_amd as pa
from paged_kv_decode_mapping_amd import workloads as W

from _gpu_util import compare, dev_bf16, host_bits, note

pytestmark = pytest.mark.gpu

BUCKET = 16


@pytest.fixture(scope="module")
def lib(gpu):
    return pa.load_library()


def _step_inputs(w, n_real, step):
    """Padded inputs of one decode step for the first n_real sequences of w:
    contexts shortened by a step-dependent amount, new tokens to fresh slots."""
    s = w.spec
    S = BUCKET
    ctx = np.zeros(S, np.int32)
    ctx[:n_real] = np.maximum(w.context_lens[:n_real] - step * 7, 0)
    tables = np.full((S, w.max_blocks_per_seq), w.poison_block, np.int32)
    tables[:n_real] = w.block_tables[:n_real]
    q = np.zeros((S, s.num_q_heads, s.head_dim), np.uint16)
    q[:n_real] = W.make_multi_query(w, [1] * s.num_seqs, seed=500 + step).q[:n_real]
    slots = np.full(S, -1, np.int64)
    slots[:n_real] = w.slot_mapping[:n_real] + step  # stays in the fresh blocks
    nk = np.zeros((S, s.num_kv_heads, s.head_dim), np.uint16)
    nv = np.zeros_like(nk)
    nk[:n_real] = np.roll(w.new_k, step, axis=0)[:n_real]
    nv[:n_real] = np.roll(w.new_v, -step, axis=0)[:n_real]
    return ctx, tables, q, slots, nk, nv


@pytest.mark.parametrize("partition,schedule", [(-1, 0), (64, 2), (64, 1)])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_captured_step_replays_match_eager(lib, partition, schedule, kv):
    """Split plans are captured both with the items ranked by each
    workgroup from the context lengths (schedule 2) and with the builder's
    list (schedule 1): either way the order is found on the device at every
    replay, from the lengths that replay's inputs hold."""
    w = W.make_workload("mixed_batch", num_seqs=12,
                        context=("list", [16, 100, 511, 512, 513, 900, 1000, 40, 2000, 77, 300, 1]))
    s = w.spec
    n_real = 10
    dev = torch.device("cuda")
    ks = vs = 1.0
    kc0, vc0 = w.k_cache, w.v_cache
    if kv == "fp8":
        ks, vs = w.fp8_scales
        kc0, vc0 = oracle.quantize_pool(kc0, ks), oracle.quantize_pool(vc0, vs)

    def dev_cache(a):
        return torch.from_numpy(a).cuda() if kv == "fp8" else dev_bf16(a)

    kc_g, vc_g = dev_cache(kc0), dev_cache(vc0)   # the graph's caches
    kc_e, vc_e = kc_g.clone(), vc_g.clone()                 # the eager reference's caches
    S, MB = BUCKET, w.max_blocks_per_seq
    st_q = torch.zeros((S, s.num_q_heads, s.head_dim), dtype=torch.bfloat16, device=dev)
    st_ctx = torch.zeros(S, dtype=torch.int32, device=dev)
    st_tab = torch.zeros((S, MB), dtype=torch.int32, device=dev)
    st_slots = torch.full((S,), -1, dtype=torch.int64, device=dev)
    st_nk = torch.zeros((S, s.num_kv_heads, s.head_dim), dtype=torch.bfloat16, device=dev)
    st_nv = torch.zeros_like(st_nk)
    st_out = torch.zeros_like(st_q)
    need = pa.pa_decode_workspace_size(st_q, kc_g, st_tab, partition_tokens=partition, schedule=schedule)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def load(step):
        ctx, tables, q, slots, nk, nv = _step_inputs(w, n_real, step)
        st_ctx.copy_(torch.from_numpy(ctx))
        st_tab.copy_(torch.from_numpy(tables))
        st_q.copy_(dev_bf16(q))
        st_slots.copy_(torch.from_numpy(slots))
        st_nk.copy_(dev_bf16(nk))
        st_nv.copy_(dev_bf16(nv))
        return ctx, tables, q, slots, nk, nv

    def step_on(kc, vc, out):
        pa.pa_cache_write(st_nk, st_nv, st_slots, kc, vc, ks, vs)
        pa.pa_decode(st_q, kc, vc, st_tab, st_ctx, w.scale, out, workspace=ws, partition_tokens=partition,
                     schedule=schedule, k_scale=ks, v_scale=vs)

    # warm up on a side stream (as torch asks before capture), on scratch caches
    load(0)
    kc_w, vc_w = kc_g.clone(), vc_g.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_on(kc_w, vc_w, torch.empty_like(st_out))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del kc_w, vc_w

    plan = pa.pa_decode_get_plan(st_q, kc_g, st_tab, partition_tokens=partition, schedule=schedule)
    if partition > 0:
        assert plan["scheduled"] and plan["self_scheduled"] == (schedule == 2)
    note(f"graph capture partition={partition} schedule={schedule}")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step_on(kc_g, vc_g, st_out)
    torch.cuda.synchronize()

    for step in range(4):
        ctx, tables, q, slots, nk, nv = load(step)
        note(f"graph replay {step} partition={partition}")
        graph.replay()
        torch.cuda.synchronize()
        got = host_bits(st_out)
        # the same step eagerly, on the reference caches
        out_e = torch.empty_like(st_out)
        step_on(kc_e, vc_e, out_e)
        torch.cuda.synchronize()
        assert np.array_equal(got, host_bits(out_e)), f"replay {step}"
        assert torch.equal(kc_g.view(torch.int16), kc_e.view(torch.int16))
        assert torch.equal(vc_g.view(torch.int16), vc_e.view(torch.int16))
        assert np.all(got[n_real:] == 0)  # padding sequences
        if step == 2:
            if kv == "fp8":
                kh, vh = kc_g.cpu().numpy(), vc_g.cpu().numpy()
                ref = oracle.decode(q, kh, vh, tables, ctx, w.scale, kv_dtype=oracle.KV_FP8_E4M3FN,
                                    k_scale=ks, v_scale=vs)
                compare(got, ref, 5e-2, 5e-3)
            else:
                kh, vh = host_bits(kc_g), host_bits(vc_g)
                ref = oracle.decode(q, kh, vh, tables, ctx, w.scale)
                compare(got, ref, 1e-2, 1e-3)


BUCKETS = (16, 64, 128)


def _padded_inputs(w, seqs, S, step):
    """Inputs of one step for the batch of sequences `seqs` of w, padded to
    bucket size S (context 0, poison table rows, slot -1), new tokens to
    fresh slots of their sequences."""
    s = w.spec
    n = len(seqs)
    ctx = np.zeros(S, np.int32)
    ctx[:n] = np.maximum(w.context_lens[seqs] - step, 0)
    tables = np.full((S, w.max_blocks_per_seq), w.poison_block, np.int32)
    tables[:n] = w.block_tables[seqs]
    q = np.zeros((S, s.num_q_heads, s.head_dim), np.uint16)
    q[:n] = W.make_multi_query(w, [1] * s.num_seqs, seed=700 + step).q[seqs]
    slots = np.full(S, -1, np.int64)
    slots[:n] = w.slot_mapping[seqs] + step  # stays in the fresh blocks
    nk = np.zeros((S, s.num_kv_heads, s.head_dim), np.uint16)
    nv = np.zeros_like(nk)
    nk[:n] = np.roll(w.new_k, step, axis=0)[seqs]
    nv[:n] = np.roll(w.new_v, -step, axis=0)[seqs]
    return ctx, tables, q, slots, nk, nv


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_graphs_at_several_buckets(lib, kv):
    """One graph per bucketed batch size (16, 64, 128 sequences: the graph
    per bucket of nanoVLLM «大模型推理优化技术：从nano-vLLM到连续批处理» §5.2),
    each capturing the write + decode step with the library's own plan for
    that size. Batches of 10, 100, 50, 128, 3 and 64 sequences are padded to
    the next bucket and replayed in that order; every replay is compared bit
    for bit with the same step run eagerly on a second copy of the caches,
    and one replay per bucket with the oracle."""
    rng = np.random.default_rng(44)
    n_pool = 128
    w = W.make_workload("mixed_batch", num_seqs=n_pool, context=("list", list(rng.integers(1, 1400, n_pool))))
    s = w.spec
    dev = torch.device("cuda")
    ks = vs = 1.0
    kc0, vc0 = w.k_cache, w.v_cache
    if kv == "fp8":
        ks, vs = w.fp8_scales
        kc0, vc0 = oracle.quantize_pool(kc0, ks), oracle.quantize_pool(vc0, vs)

    def dev_cache(a):
        return torch.from_numpy(a).cuda() if kv == "fp8" else dev_bf16(a)

    kc_g, vc_g = dev_cache(kc0), dev_cache(vc0)
    kc_e, vc_e = kc_g.clone(), vc_g.clone()
    MB = w.max_blocks_per_seq
    graphs = {}
    for B in BUCKETS:
        st = dict(q=torch.zeros((B, s.num_q_heads, s.head_dim), dtype=torch.bfloat16, device=dev),
                  ctx=torch.zeros(B, dtype=torch.int32, device=dev),
                  tab=torch.zeros((B, MB), dtype=torch.int32, device=dev),
                  slots=torch.full((B,), -1, dtype=torch.int64, device=dev),
                  nk=torch.zeros((B, s.num_kv_heads, s.head_dim), dtype=torch.bfloat16, device=dev))
        st["nv"] = torch.zeros_like(st["nk"])
        st["out"] = torch.zeros_like(st["q"])
        need = pa.pa_decode_workspace_size(st["q"], kc_g, st["tab"])
        st["ws"] = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        st["plan"] = pa.pa_decode_get_plan(st["q"], kc_g, st["tab"])

        def step_on(kc, vc, out, st=st):
            pa.pa_cache_write(st["nk"], st["nv"], st["slots"], kc, vc, ks, vs)
            pa.pa_decode(st["q"], kc, vc, st["tab"], st["ctx"], w.scale, out, workspace=st["ws"], k_scale=ks,
                         v_scale=vs)

        # warm up on a side stream (as torch asks before capture), on scratch caches
        kc_w, vc_w = kc_g.clone(), vc_g.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_on(kc_w, vc_w, torch.empty_like(st["out"]))
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        del kc_w, vc_w
        note(f"graph capture bucket {B} {kv} plan={st['plan']}")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step_on(kc_g, vc_g, st["out"])
        torch.cuda.synchronize()
        graphs[B] = (g, st, step_on)

    checked = set()
    for step, n in enumerate([10, 100, 50, 128, 3, 64]):
        B = min(b for b in BUCKETS if b >= n)
        g, st, step_on = graphs[B]
        seqs = np.sort(rng.choice(n_pool, n, replace=False))
        ctx, tables, q, slots, nk, nv = _padded_inputs(w, seqs, B, step)
        st["ctx"].copy_(torch.from_numpy(ctx))
        st["tab"].copy_(torch.from_numpy(tables))
        st["q"].copy_(dev_bf16(q))
        st["slots"].copy_(torch.from_numpy(slots))
        st["nk"].copy_(dev_bf16(nk))
        st["nv"].copy_(dev_bf16(nv))
        note(f"replay bucket {B} with {n} sequences, step {step}")
        g.replay()
        torch.cuda.synchronize()
        got = host_bits(st["out"])
        out_e = torch.empty_like(st["out"])
        step_on(kc_e, vc_e, out_e)
        torch.cuda.synchronize()
        assert np.array_equal(got, host_bits(out_e)), f"bucket {B}, step {step}"
        assert torch.equal(kc_g.view(torch.int16) if kv == "bf16" else kc_g, kc_e.view(torch.int16) if kv == "bf16" else kc_e)
        assert torch.equal(vc_g.view(torch.int16) if kv == "bf16" else vc_g, vc_e.view(torch.int16) if kv == "bf16" else vc_e)
        assert np.all(got[n:] == 0)  # padding sequences
        if B not in checked:
            checked.add(B)
            kh = kc_g.cpu().numpy() if kv == "fp8" else host_bits(kc_g)
            vh = vc_g.cpu().numpy() if kv == "fp8" else host_bits(vc_g)
            kvd = oracle.KV_FP8_E4M3FN if kv == "fp8" else oracle.KV_BF16
            ref = oracle.decode(q, kh, vh, tables, ctx, w.scale, kv_dtype=kvd, k_scale=ks, v_scale=vs)
            compare(got, ref, *((5e-2, 5e-3) if kv == "fp8" else (1e-2, 1e-3)))
    assert checked == set(BUCKETS)
