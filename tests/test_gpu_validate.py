"""GPU tests of the opt-in precondition checks (pa_check_cache_write_inputs,
pa_check_decode_inputs, and the PA_DEBUG_VALIDATE switch of the hot-path
calls). The inputs that break a precondition are index arrays only; nothing
here launches a kernel on them: a check that fails returns before launching.
"""
import os

import numpy as np
import pytest
import torch

import paged_kv_decode_mapping_amd as pa
from paged_kv_decode_mapping_amd import workloads as W

from _gpu_util import DeviceWorkload, host_bits, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib(gpu):
    return pa.load_library()


@pytest.fixture
def debug_validate():
    old = os.environ.get("PA_DEBUG_VALIDATE")
    os.environ["PA_DEBUG_VALIDATE"] = "1"
    yield
    if old is None:
        del os.environ["PA_DEBUG_VALIDATE"]
    else:
        os.environ["PA_DEBUG_VALIDATE"] = old


def _pool(N, bs, Hkv=2, D=64):
    """The shape of a pool (the checks read its block count and block size)."""
    return pa.TensorSpec((N, bs, Hkv, D), pa.PA_DTYPE_BF16)


SMALL = {
    "tiny": dict(),
    "mixed_batch": dict(num_seqs=10, context=("list", [16, 100, 511, 512, 513, 900, 3000, 40, 8192, 77])),
    "long_splitk": dict(num_seqs=2, context=("list", [5000, 2049])),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_generated_workloads_pass(lib, name):
    w = W.make_workload(name, **SMALL[name])
    d = DeviceWorkload(w)
    note(f"checks accept {name}")
    bs = w.spec.block_size
    assert pa.pa_check_cache_write_inputs(d.slot_mapping, d.k_cache) == pa.PA_OK
    assert pa.pa_check_decode_inputs(d.block_tables, d.context_lens, d.k_cache) == pa.PA_OK


def test_bad_slots_are_reported(lib):
    N, bs = 32, 16
    cases = {
        "duplicate": [3, 17, 3, -1],
        "past the pool": [0, 1, N * bs, 5],
    }
    for what, slots in cases.items():
        note(f"slot check: {what}")
        t = torch.tensor(slots, dtype=torch.int64, device="cuda")
        assert pa.pa_check_cache_write_inputs(t, _pool(N, bs)) == pa.PA_ERR_PRECONDITION, what
    ok = torch.tensor([-1, -7, 0, N * bs - 1, 200], dtype=torch.int64, device="cuda")
    assert pa.pa_check_cache_write_inputs(ok, _pool(N, bs)) == pa.PA_OK


def test_bad_tables_and_lengths_are_reported(lib):
    N, bs = 32, 16
    good = np.array([[0, 1, 2, 3], [4, 5, -1, 99], [6, 7, 8, 9]], dtype=np.int32)
    ctx = np.array([64, 32, 1], dtype=np.int32)  # row 1 never reads its bad tail entries
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    note("decode check: valid tables")
    assert pa.pa_check_decode_inputs(t(good), t(ctx), _pool(N, bs)) == pa.PA_OK
    # a table that is a view with a row stride wider than its width
    wide = np.full((3, 9), -5, np.int32)
    wide[:, :4] = good
    assert pa.pa_check_decode_inputs(t(wide)[:, :4], t(ctx), _pool(N, bs)) == pa.PA_OK
    bad_tables = good.copy()
    bad_tables[1, 1] = N  # covers tokens 16..31 of a 32-token context
    neg_tables = good.copy()
    neg_tables[0, 3] = -2
    for what, tab, c in [("entry past the pool", bad_tables, ctx), ("negative entry", neg_tables, ctx),
                         ("context past the row", good, np.array([65, 32, 1], np.int32)),
                         ("negative context", good, np.array([64, -1, 1], np.int32))]:
        note(f"decode check: {what}")
        assert pa.pa_check_decode_inputs(t(tab), t(c), _pool(N, bs)) == pa.PA_ERR_PRECONDITION, what


def test_bad_query_counts_are_reported(lib):
    """pa_check_multi_inputs: a sequence's query tokens are among its cached
    ones, no more than max_query_len of them, and query_start rises from 0."""
    N, bs = 32, 16
    tab = np.arange(12, dtype=np.int32).reshape(3, 4)
    ctx = np.array([64, 3, 20], dtype=np.int32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).cuda()
    note("multi check: valid query counts")
    assert pa.pa_check_multi_inputs(t(tab), t(ctx), t([0, 4, 7, 8]), 4, _pool(N, bs)) == pa.PA_OK
    for what, qs, maxq in [("more queries than context", [0, 1, 5, 6], 4),
                           ("more than max_query_len", [0, 5, 6, 7], 4),
                           ("falling offsets", [0, 4, 3, 5], 4),
                           ("not starting at 0", [1, 2, 3, 4], 4)]:
        note(f"multi check: {what}")
        assert pa.pa_check_multi_inputs(t(tab), t(ctx), t(qs), maxq, _pool(N, bs)) == pa.PA_ERR_PRECONDITION, what


def test_debug_switch_stops_hot_path_calls(lib, debug_validate):
    w = W.make_workload("tiny")
    d = DeviceWorkload(w)
    note("PA_DEBUG_VALIDATE: valid inputs still run")
    out = d.decode()
    torch.cuda.synchronize()
    ref_bits = host_bits(out)
    # a table entry outside the pool: the call must refuse before launching
    bad = w.block_tables.copy()
    bad[0, 0] = w.num_blocks + 5
    d.block_tables = torch.from_numpy(bad).cuda()
    sentinel = torch.full_like(out, 7.0)
    note("PA_DEBUG_VALIDATE: bad table refused")
    with pytest.raises(pa.PAError) as e:
        d.decode(out=sentinel)
    assert e.value.status == pa.PA_ERR_PRECONDITION
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0)  # nothing was launched
    # a duplicated slot in the cache write
    slots = w.slot_mapping.copy()
    slots[1] = slots[0]
    kc = d.k_cache.clone()
    note("PA_DEBUG_VALIDATE: duplicate slot refused")
    with pytest.raises(pa.PAError) as e:
        pa.pa_cache_write(d.new_k, d.new_v, torch.from_numpy(slots).cuda(), d.k_cache, d.v_cache)
    assert e.value.status == pa.PA_ERR_PRECONDITION
    torch.cuda.synchronize()
    assert torch.equal(kc.view(torch.int16), d.k_cache.view(torch.int16))
    assert ref_bits.shape == (w.spec.num_seqs, w.spec.num_q_heads, w.spec.head_dim)


def test_stream_probe_reads_without_writing(lib):
    """The streaming-read reference kernel runs over a buffer with a ragged
    tail and leaves its sink untouched (its data never matches the magic)."""
    x = torch.zeros((1 << 20) + 48, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    note("stream probe")
    for nt in (False, True):
        pa.pa_probe_stream_read(x, sink, nt)
    torch.cuda.synchronize()
    assert torch.all(sink == 0)
