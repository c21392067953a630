"""What an fp8 KV cache costs in accuracy: reported, not gated.

The fp8 parity tests compare the fp8-KV kernel with the oracle reading the
same e4m3fn codes, which isolates the kernel. Here the same kernel output is
also compared with the float64 oracle on the values before quantisation
(the bf16 caches): quantisation error plus kernel error, the error a user of
an fp8 cache sees. The error metrics are those of Tutorial
«大模型推理优化与加速完全教程» §3.1 "量化基础" (the difference between the
dequantised and the original computation), taken as max and mean absolute
error over every output element. Each case prints one line

    FP8-ACCURACY {"workload": ..., "vs_bf16_values": {"max": .., "mean": ..},
                  "vs_fp8_codes": {"max": .., "mean": ..}}

and the test only requires finite outputs; the figures are recorded with
the design notes.
"""
import json

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_mapping_amd as pa
from paged_kv_decode_mapping_amd import workloads as W

from _gpu_util import REDUCED, DeviceWorkload, bf16_to_f64, host_bits, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib(gpu):
    return pa.load_library()


def _err(got, ref):
    e = np.abs(got - ref)
    return {"max": float(e.max()), "mean": float(e.mean())}


@pytest.mark.parametrize("name", [n for n in REDUCED if n != "tiny"] + ["tiny"])
def test_fp8_error_against_the_bf16_oracle(lib, name):
    w = W.make_workload(name, **REDUCED[name])
    ks, vs = w.fp8_scales
    kq, vq = oracle.quantize_pool(w.k_cache, ks), oracle.quantize_pool(w.v_cache, vs)
    d = DeviceWorkload(w, kq, vq)
    note(f"fp8 accuracy {name}")
    got = bf16_to_f64(host_bits(d.decode(k_scale=ks, v_scale=vs)))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(got))
    ref_values = oracle.decode_workload(w)  # the bf16 caches the codes were made from
    ref_codes = oracle.decode_workload(w, kv_dtype=oracle.KV_FP8_E4M3FN, k_cache=kq, v_cache=vq, k_scale=ks,
                                       v_scale=vs)
    rec = {"workload": name, "contexts": [int(c) for c in w.context_lens], "k_scale": ks, "v_scale": vs,
           "vs_bf16_values": _err(got, ref_values), "vs_fp8_codes": _err(got, ref_codes)}
    print("FP8-ACCURACY " + json.dumps(rec), flush=True)
