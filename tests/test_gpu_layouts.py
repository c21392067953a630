"""GPU parity on other memory layouts, through the C ABI's strides: a
head-major pool ([N, Hkv, bs, D] in memory, passed as the logical
[N, bs, Hkv, D] with its strides), query and output rows with padded
strides, new K/V rows as views, and block tables that are row slices of a
wider table. The results must equal the oracle's on the same logical
values (the layout changes where bytes live, not what is computed), and
bytes outside a written view must stay as they were.

Tolerances as elsewhere: max |err| 1e-2 / mean 1e-3 against the float64
oracle for bf16 caches, 5e-2 / 5e-3 for fp8 (same codes); writes bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_mapping_amd as pa
from paged_kv_decode_mapping_amd import workloads as W

from _gpu_util import REDUCED, DeviceWorkload, cache_bits, compare, dev_bf16, head_major, host_bits, note

pytestmark = pytest.mark.gpu

BF16_TOL = (1e-2, 1e-3)
FP8_TOL = (5e-2, 5e-3)
SENTINEL = 0x7FC1  # a quiet NaN no kernel writes


@pytest.fixture(scope="module")
def lib(gpu):
    return pa.load_library()


def _fp8(w):
    ks, vs = w.fp8_scales
    return oracle.quantize_pool(w.k_cache, ks), oracle.quantize_pool(w.v_cache, vs), ks, vs


@pytest.mark.parametrize("name", list(REDUCED))
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("variant", ["auto", "valu", "mfma"])
def test_head_major_decode_matches_oracle(lib, name, kv, variant):
    w = W.make_workload(name, **REDUCED[name])
    if variant == "valu" and w.spec.group > 4:
        pytest.skip("the VALU kernel takes groups of at most 4")
    kc, vc, ks, vs = (w.k_cache, w.v_cache, 1.0, 1.0) if kv == "bf16" else _fp8(w)
    kvd, tol = (oracle.KV_BF16, BF16_TOL) if kv == "bf16" else (oracle.KV_FP8_E4M3FN, FP8_TOL)
    d = DeviceWorkload(w, kc, vc, layout="head_major")
    plan = pa.pa_decode_get_plan(d.q, d.k_cache, d.block_tables, variant=variant)
    assert plan["heads_per_tile"] == 1
    note(f"head-major decode {name} {kv} {variant} plan={plan}")
    out = d.decode(variant=variant, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    ref = oracle.decode_workload(w, kv_dtype=kvd, k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs)
    compare(host_bits(out), ref, *tol)


@pytest.mark.parametrize("name", ["long_splitk", "mixed_batch"])
@pytest.mark.parametrize("partition,waves", [(16, 1), (48, 2), (512, 4), (512, 8)])
@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_head_major_split_plans(lib, name, partition, waves, variant):
    w = W.make_workload(name, **REDUCED[name])
    d = DeviceWorkload(w, layout="head_major")
    note(f"head-major split {name} P={partition} W={waves} {variant}")
    out = d.decode(partition_tokens=partition, waves=waves, variant=variant)
    torch.cuda.synchronize()
    compare(host_bits(out), oracle.decode_workload(w), *BF16_TOL)


@pytest.mark.parametrize("name", ["tiny", "mixed_batch", "long_splitk"])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_head_major_cache_write_bit_exact(lib, name, kv):
    """The whole pool after the write equals the oracle's scatter into the
    logical pool, untouched rows included."""
    w = W.make_workload(name, **REDUCED[name])
    kc, vc, ks, vs = (w.k_cache, w.v_cache, 1.0, 1.0) if kv == "bf16" else _fp8(w)
    kvd = oracle.KV_BF16 if kv == "bf16" else oracle.KV_FP8_E4M3FN
    d = DeviceWorkload(w, kc, vc, layout="head_major")
    note(f"head-major cache write {name} {kv}")
    pa.pa_cache_write(d.new_k, d.new_v, d.slot_mapping, d.k_cache, d.v_cache, ks, vs)
    torch.cuda.synchronize()
    kh, vh = kc.copy(), vc.copy()
    oracle.cache_write(w.new_k, w.new_v, w.slot_mapping, kh, vh, kv_dtype=kvd, k_scale=ks, v_scale=vs)
    assert np.array_equal(cache_bits(d.k_cache), kh)
    assert np.array_equal(cache_bits(d.v_cache), vh)


def test_strided_rows_and_tables(lib):
    """q and out as views with padded head and sequence strides, new K/V
    rows as views of wider buffers, a block table sliced out of a wider one;
    every byte outside the output view keeps its value."""
    w = W.make_workload("mixed_batch", **REDUCED["mixed_batch"])
    s = w.spec
    S, Hq, Hkv, D = s.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim
    d = DeviceWorkload(w)
    q_big = torch.zeros((S, Hq, D + 24), dtype=torch.bfloat16, device="cuda")
    q_big[:, :, 8:8 + D] = d.q
    q_view = q_big[:, :, 8:8 + D]  # head stride D + 24, base 16 bytes in
    out_big = torch.empty((S + 1, 2 * Hq, D), dtype=torch.bfloat16, device="cuda")
    out_big.view(torch.int16).fill_(SENTINEL)
    out_view = out_big[1:, ::2]  # every other head row, one sequence row in
    MB = w.max_blocks_per_seq
    tab_big = torch.full((S, MB + 5), -7, dtype=torch.int32, device="cuda")
    tab_big[:, 2:2 + MB] = d.block_tables
    tab_view = tab_big[:, 2:2 + MB]
    k_big = torch.zeros((len(w.slot_mapping), Hkv, 2 * D), dtype=torch.bfloat16, device="cuda")
    v_big = torch.zeros_like(k_big)
    k_big[:, :, D:] = d.new_k
    v_big[:, :, :D] = d.new_v
    note("strided views: cache write + decode")
    pa.pa_cache_write(k_big[:, :, D:], v_big[:, :, :D], d.slot_mapping, d.k_cache, d.v_cache)
    got = pa.pa_decode(q_view, d.k_cache, d.v_cache, tab_view, d.context_lens, w.scale, out_view,
                       partition_tokens=48)
    torch.cuda.synchronize()
    assert got.data_ptr() == out_view.data_ptr()
    kh, vh = w.k_cache.copy(), w.v_cache.copy()
    oracle.cache_write(w.new_k, w.new_v, w.slot_mapping, kh, vh)
    assert np.array_equal(cache_bits(d.k_cache), kh)
    assert np.array_equal(cache_bits(d.v_cache), vh)
    compare(host_bits(out_view.contiguous()), oracle.decode(w.q, kh, vh, w.block_tables, w.context_lens, w.scale),
            *BF16_TOL)
    untouched = host_bits(out_big).copy()
    untouched[1:, ::2] = SENTINEL
    assert np.all(untouched == SENTINEL), "a write landed outside the output view"


def test_head_major_multi_and_cascade(lib):
    """pa_decode_multi and pa_decode_cascade read a head-major pool too."""
    w = W.make_workload("mixed_batch", num_seqs=6, context=("list", [40, 700, 1030, 16, 2100, 333]))
    d = DeviceWorkload(w, layout="head_major")
    qlens = np.array([3, 5, 1, 2, 4, 4], np.int32)
    mq = W.make_multi_query(w, qlens)
    qm = dev_bf16(mq.q)
    qs = torch.from_numpy(mq.query_start).cuda()
    note("head-major multi")
    out = pa.pa_decode_multi(qm, d.k_cache, d.v_cache, d.block_tables, d.context_lens, qs, w.scale,
                             int(qlens.max()), partition_tokens=256)
    torch.cuda.synchronize()
    ref = oracle.multi_decode(mq.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, mq.query_start, w.scale)
    compare(host_bits(out), ref, *BF16_TOL)

    b = W.make_prefix_groups(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                             groups=[(64, [80, 200, 64]), (32, [40, 33])], lead=[100], seed=21)
    kc, vc = head_major(dev_bf16(b.k_cache)), head_major(dev_bf16(b.v_cache))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    note("head-major cascade")
    out = pa.pa_decode_cascade(dev_bf16(b.q), kc, vc, t(b.block_tables), t(b.context_lens), t(b.prefix_tables),
                               t(b.prefix_lens), t(b.group_start), b.scale, max_group_size=b.max_group_size)
    torch.cuda.synchronize()
    ref = oracle.cascade_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.prefix_tables,
                                b.prefix_lens, b.group_start, b.scale, max_group_size=b.max_group_size)
    compare(host_bits(out), ref, *BF16_TOL)


def test_head_major_copy_blocks(lib):
    w = W.make_workload("tiny")
    d = DeviceWorkload(w, layout="head_major")
    N = w.num_blocks
    pairs = np.array([[0, N - 1], [3, 7], [5, 2]], np.int64)
    note("head-major copy_blocks")
    pa.pa_copy_blocks(d.k_cache, d.v_cache, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    kh, vh = w.k_cache.copy(), w.v_cache.copy()
    oracle.copy_blocks(kh, vh, pairs)
    assert np.array_equal(cache_bits(d.k_cache), kh)
    assert np.array_equal(cache_bits(d.v_cache), vh)
