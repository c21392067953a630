"""pa_decode_no_alloc through the C ABI: the decode with the library's static
scratch in place of a caller workspace must give exactly pa_decode's output
(same plan, same kernels) and match the float64 oracle, on consecutive
calls that reuse the scratch -- a split plan, then a smaller batch, then
one that needs no workspace, and the MQA route (the multi-row kernel) --
and must refuse a plan whose workspace exceeds the scratch before touching
any tensor."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_mapping_amd as pa
from paged_kv_decode_mapping_amd import workloads as W

from _gpu_util import DeviceWorkload, compare, host_bits, note

pytestmark = pytest.mark.gpu

SCRATCH = pa.PA_NO_ALLOC_SCRATCH
PA_ERR_SCRATCH = pa.PA_ERR_SCRATCH


@pytest.fixture(scope="module")
def lib(gpu):
    return pa.load_library()


def _no_alloc(lib, tensors, scale, out, ks=1.0, vs=1.0, **opts):
    o = pa._opts(**opts)
    descs = [pa.desc(t) for t in tensors]
    return lib.pa_decode_no_alloc(*map(pa._ref, descs), scale, pa._ref(pa.desc(out)), ks, vs, ctypes.byref(o),
                                  int(torch.cuda.current_stream().cuda_stream))


CASES = [
    ("long_splitk", dict(num_seqs=2, context=("list", [20000, 9000])), dict(partition_tokens=512), "bf16"),
    ("mixed_batch", dict(num_seqs=5, context=("list", [16, 700, 3000, 40, 1500])), dict(partition_tokens=256), "fp8"),
    ("tiny", dict(), dict(partition_tokens=-1), "bf16"),
]


def test_no_alloc_matches_pa_decode_on_consecutive_calls(lib):
    sizes = []
    for name, shape, opts, kv in CASES:
        w = W.make_workload(name, **shape)
        kc, vc, ks, vs, kvd, tol = w.k_cache, w.v_cache, 1.0, 1.0, oracle.KV_BF16, (1e-2, 1e-3)
        if kv == "fp8":
            ks, vs = w.fp8_scales
            kc, vc = oracle.quantize_pool(kc, ks), oracle.quantize_pool(vc, vs)
            kvd, tol = oracle.KV_FP8_E4M3FN, (5e-2, 5e-3)
        d = DeviceWorkload(w, kc, vc)
        tensors = (d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens)
        need = pa.pa_decode_workspace_size(d.q, d.k_cache, d.block_tables, **opts)
        sizes.append(need)
        assert need <= SCRATCH
        note(f"no-alloc {name} {kv} opts={opts} workspace={need}")
        ref_out = pa.pa_decode(*tensors, w.scale, k_scale=ks, v_scale=vs, **opts)
        out = torch.full_like(d.q, float("nan"))
        assert _no_alloc(lib, tensors, w.scale, out, ks, vs, **opts) == pa.PA_OK
        torch.cuda.synchronize()
        got = host_bits(out)
        assert np.array_equal(got, host_bits(ref_out)), f"{name}: differs from pa_decode"
        compare(got, oracle.decode_workload(w, kv_dtype=kvd, k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs), *tol)
    assert sizes[0] > sizes[1] > sizes[2] == 0  # each call smaller than the one before


def test_no_alloc_refuses_plans_beyond_the_scratch(lib):
    """A plan needing more than the scratch is refused before any tensor is
    read (the descriptors here carry no data at all)."""
    q, kc, bt = pa.decode_specs(256, 32, 8, 128, 16, 4096, num_blocks=1 << 16)
    opts = dict(partition_tokens=64)
    assert pa.pa_decode_workspace_size(q, kc, bt, **opts) > SCRATCH
    cl = pa.TensorSpec((256,), pa.PA_DTYPE_I32)
    note("no-alloc: oversized plan refused")
    assert _no_alloc(lib, (q, kc, kc, bt, cl), 0.1, q, **opts) == PA_ERR_SCRATCH


def test_no_alloc_mqa_route(lib):
    """More than 16 query heads per KV head (MQA: 64 on one) go to the
    multi-row kernel; split, its partial states and merge use the scratch
    as well. Same bits as pa_decode, and the oracle's values."""
    w = W.make_workload("mixed_batch", num_seqs=6, context=("list", [1, 17, 300, 1000, 2100, 64]), num_q_heads=64,
                        num_kv_heads=1)
    d = DeviceWorkload(w)
    tensors = (d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens)
    opts = dict(partition_tokens=256)
    plan = pa.pa_decode_get_plan(d.q, d.k_cache, d.block_tables, **opts)
    assert plan["num_partitions"] > 1 and 0 < plan["workspace_bytes"] <= SCRATCH
    note(f"no-alloc MQA opts={opts} plan={plan}")
    ref_out = pa.pa_decode(*tensors, w.scale, **opts)
    out = torch.full_like(d.q, float("nan"))
    assert _no_alloc(lib, tensors, w.scale, out, **opts) == pa.PA_OK
    torch.cuda.synchronize()
    got = host_bits(out)
    assert np.array_equal(got, host_bits(ref_out)), "differs from pa_decode"
    compare(got, oracle.decode_workload(w), 1e-2, 1e-3)
