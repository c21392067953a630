"""The stream argument of the C ABI: every launch of a call (the cache write;
the work-list builder, the decode kernel and the merge of a split decode)
goes to the stream the caller names, not to the current or default stream.

A graph capture is begun on a side stream, the current stream is set back to
the default one, and the calls are made naming the side stream. Work on the
named stream is captured, not run: after the capture the output must still
hold the sentinel it was filled with (a launch on any other stream would
have run at once, or failed while the side stream captures). Replaying the
graph must then give the oracle's result.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_mapping_amd as pa
from paged_kv_decode_mapping_amd import workloads as W

from _gpu_util import DeviceWorkload, compare, host_bits, note

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1  # a bf16 NaN pattern that a decode never stores


@pytest.fixture(scope="module")
def lib(gpu):
    return pa.load_library()


@pytest.mark.parametrize("partition", [-1, 48])
def test_launches_follow_the_given_stream(lib, partition):
    ctx = [16, 100, 511, 512, 513, 900, 3000, 40, 8192, 77]
    w = W.make_workload("mixed_batch", num_seqs=len(ctx), context=("list", ctx))
    s = w.spec
    d = DeviceWorkload(w)
    kc_h, vc_h = w.k_cache.copy(), w.v_cache.copy()
    oracle.cache_write(w.new_k, w.new_v, w.slot_mapping, kc_h, vc_h)
    ref = oracle.decode(w.q, kc_h, vc_h, w.block_tables, w.context_lens, w.scale)

    need = pa.pa_decode_workspace_size(d.q, d.k_cache, d.block_tables, partition_tokens=partition)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty(tuple(d.q.shape), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()

    def calls():
        pa.pa_cache_write(d.new_k, d.new_v, d.slot_mapping, d.k_cache, d.v_cache, stream=side)
        pa.pa_decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, w.scale, out, workspace=ws,
                     partition_tokens=partition, stream=side)

    # warm-up on the side stream (the new tokens go to free slots, so
    # writing them twice changes nothing the decode reads)
    side.wait_stream(torch.cuda.current_stream())
    calls()
    side.synchronize()

    out.view(torch.int16).fill_(SENTINEL)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    note(f"stream argument: calls naming a capturing side stream, partition={partition}")
    with torch.cuda.stream(side):
        graph.capture_begin()
    assert torch.cuda.current_stream() != side
    calls()  # the current stream is not the side stream here
    with torch.cuda.stream(side):
        graph.capture_end()
    torch.cuda.synchronize()
    assert np.all(host_bits(out) == SENTINEL), "a launch did not go to the stream it was given"

    graph.replay()
    torch.cuda.synchronize()
    compare(host_bits(out), ref, 1e-2, 1e-3)
    rows = d.k_cache.view(-1, s.num_kv_heads, s.head_dim)[d.slot_mapping].cpu().view(torch.int16).numpy()
    assert np.array_equal(rows.view(np.uint16), kc_h.reshape(-1, s.num_kv_heads, s.head_dim)[w.slot_mapping])


def test_binding_allocations_follow_the_named_stream(lib):
    """With stream= and neither workspace nor out given, the binding
    allocates both on that stream. Right after the call, the current stream
    allocates blocks of the same sizes and overwrites them: had the
    workspace or out come from the current stream's pool and been released
    on return, those blocks could be handed out again and overwritten while
    the side stream's work list, partials and merge still use them."""
    w = W.make_workload("long_splitk", num_seqs=2, context=("list", [32768, 20000]))
    d = DeviceWorkload(w)
    ref = oracle.decode_workload(w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    need = pa.pa_decode_workspace_size(d.q, d.k_cache, d.block_tables, partition_tokens=512)
    assert need > 0
    note("binding allocations on the named stream")
    for _ in range(3):
        out = pa.pa_decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, w.scale,
                           partition_tokens=512, stream=side)
        junk_ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
        junk_out = torch.full(tuple(out.shape), float("nan"), dtype=torch.bfloat16, device="cuda")
        side.synchronize()
        torch.cuda.synchronize()
        compare(host_bits(out), ref, 1e-2, 1e-3)
        del junk_ws, junk_out
