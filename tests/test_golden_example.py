"""Pins against the worked example of Tutorial «大模型推理优化与加速完全教程»
§4.2 (the PagedKVCache usage example: 5 sequences of 100 tokens in a pool of
500 blocks of 16 tokens), stored in tests/golden/ with its citation.

The fixture holds what the example's allocator leaves behind, derived by
hand: the block tables and the memory_usage figures. These tests check the
fixture against the page's formulas, then run the example's flow through the
oracle: each token is written to row j % block_size of block
table[j // block_size] (append_token's index and offset), and the decode over
those tables equals attention over the dense tokens (torch SDPA, float64).
"""
import json
import math
import os

import numpy as np
import torch

import oracle
from paged_kv_decode_mapping_amd import workloads as W

FX = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tutorial_4_2_paged_cache_example.json")))


def example_slots(fx):
    """Slot of every appended token, sequence after sequence: physical block
    table[j // bs] (the block the example's append_token picks), row j % bs."""
    bs = fx["block_size"]
    return np.array([fx["block_tables"][i][j // bs] * bs + j % bs
                     for i, L in enumerate(fx["seq_lengths"]) for j in range(L)], dtype=np.int64)


def test_fixture_obeys_the_memory_usage_formulas():
    m = FX["memory_usage"]
    bs, N, Hkv, D, layers = FX["block_size"], FX["num_blocks"], FX["num_kv_heads"], FX["head_dim"], FX["num_layers"]
    tables = FX["block_tables"]
    used = sorted(b for row in tables for b in row)
    assert len(used) == len(set(used)) == m["used_blocks"]
    assert m["used_blocks"] == sum(math.ceil(L / bs) for L in FX["seq_lengths"])
    assert m["free_blocks"] == N - m["used_blocks"] and m["total_blocks"] == N
    assert m["block_bytes"] == bs * Hkv * D * 2 * 2
    assert math.isclose(m["utilization"], m["used_blocks"] / N * 100, rel_tol=1e-12)
    assert math.isclose(m["total_memory_gb"], N * m["block_bytes"] * layers / 1e9, rel_tol=1e-12)
    assert math.isclose(m["used_memory_gb"], m["used_blocks"] * m["block_bytes"] * layers / 1e9, rel_tol=1e-12)


def test_example_flow_through_the_oracle():
    """One layer of the example: 500 tokens written through the fixture's
    slots, then a decode of each sequence over its 100 tokens (32 query heads
    on the example's 32 KV heads) against SDPA on the dense tokens."""
    bs, N, Hkv, D = FX["block_size"], FX["num_blocks"], FX["num_kv_heads"], FX["head_dim"]
    lens = FX["seq_lengths"]
    S, T = len(lens), sum(lens)
    rng = np.random.default_rng(42)
    bits = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    k = bits(rng.standard_normal((T, Hkv, D)))
    v = bits(rng.standard_normal((T, Hkv, D)))
    q = bits(rng.standard_normal((S, Hkv, D)))
    kc = np.zeros((N, bs, Hkv, D), np.uint16)
    vc = np.zeros_like(kc)
    assert oracle.cache_write(k, v, example_slots(FX), kc, vc) == T
    assert not kc[35:].any() and not vc[35:].any()  # blocks the example never hands out stay untouched
    tables = np.array(FX["block_tables"], np.int32)
    ctx = np.array(lens, np.int32)
    scale = 1.0 / math.sqrt(D)
    got = oracle.decode(q, kc, vc, tables, ctx, scale)
    f64 = lambda b: torch.from_numpy(W.bf16_bits_to_f32(b).astype(np.float64))
    start = 0
    for i, L in enumerate(lens):
        kt = f64(k[start:start + L]).permute(1, 0, 2)[None]
        vt = f64(v[start:start + L]).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(f64(q[i])[None, :, None, :], kt, vt, scale=scale)
        np.testing.assert_allclose(got[i], ref[0, :, 0, :].numpy(), rtol=0, atol=1e-12)
        start += L
