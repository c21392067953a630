"""Structure of the seeded synthetic workloads (host logic, no GPU)."""
import numpy as np
import pytest

from paged_kv_decode_mapping_amd import workloads as W


def _referenced_rows(w):
    bs = w.spec.block_size
    used = np.zeros((w.num_blocks, bs), bool)
    for i, c in enumerate(w.context_lens):
        for b in range((int(c) + bs - 1) // bs):
            n = min(bs, int(c) - b * bs)
            used[w.block_tables[i, b], :n] = True
    return used


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("llama7b_mha", dict(num_seqs=3, context=("list", [512, 700, 2048]))),
    ("llama70b_gqa", dict(num_seqs=2, context=("list", [4096, 4096]))),
    ("long_splitk", dict(num_seqs=2, context=("list", [1000, 2100]))),
    ("mixed_batch", dict(num_seqs=12, context=("list", [16, 100, 511, 512, 513, 900, 1000, 40, 2000, 77, 3000, 520]))),
])
def test_pool_and_tables_are_consistent(name, kw):
    w = W.make_workload(name, **kw)
    s = w.spec
    assert w.q.shape == (s.num_seqs, s.num_q_heads, s.head_dim)
    assert w.k_cache.shape == (w.num_blocks, s.block_size, s.num_kv_heads, s.head_dim)
    nblk = (w.context_lens + s.block_size - 1) // s.block_size
    assert w.block_tables.shape == (s.num_seqs, nblk.max())
    for i in range(s.num_seqs):
        assert np.all(w.block_tables[i, nblk[i]:] == w.poison_block)
        assert np.all((w.block_tables[i, :nblk[i]] >= 0) & (w.block_tables[i, :nblk[i]] < w.num_blocks))
        assert w.poison_block not in w.block_tables[i, :nblk[i]]
    used = _referenced_rows(w)
    kf = W.bf16_bits_to_f32(w.k_cache)
    # every referenced row is finite; every row nobody references is NaN
    assert np.all(np.isfinite(kf[used]))
    if s.shared_prefix_tokens == 0:
        assert np.all(np.isnan(kf[~used]))
    assert np.all(np.isnan(kf[w.poison_block]))
    # new tokens go to distinct rows of blocks no table refers to
    bs = s.block_size
    blocks = w.slot_mapping // bs
    assert len(set(w.slot_mapping.tolist())) == len(w.slot_mapping)
    referenced = set(w.block_tables[w.block_tables != w.poison_block].tolist())
    assert not (set(blocks.tolist()) & referenced)
    assert w.poison_block not in set(blocks.tolist())
    assert len(w.slot_mapping) == s.num_seqs


def test_tiny_matches_the_stated_recipe():
    w = W.make_workload("tiny")
    assert w.context_lens.tolist() == [1, 17, 64, 100]
    assert w.num_blocks == 32 and w.unique_blocks == 14
    assert w.spec.group == 4 and w.scale == 1 / 8
    # distinct physical blocks across sequences (no sharing here)
    ids = w.block_tables[w.block_tables != w.poison_block]
    assert len(set(ids.tolist())) == 14


def test_generation_is_seeded():
    a = W.make_workload("tiny")
    b = W.make_workload("tiny")
    c = W.make_workload("tiny", seed=99)
    assert np.array_equal(a.k_cache, b.k_cache) and np.array_equal(a.block_tables, b.block_tables)
    assert not np.array_equal(a.k_cache, c.k_cache)


def test_shared_prefix_blocks():
    ctx = [16, 100, 511, 512, 513, 900, 1000, 40, 2000, 77, 3000, 520]
    w = W.make_workload("mixed_batch", num_seqs=12, context=("list", ctx))
    sh = w.shared_seqs
    assert len(sh) == 6
    pb = 512 // 16
    full = [i for i in sh if ctx[i] >= 512]
    ref = w.block_tables[full[0], :pb]
    for i in sh:
        n = min(pb, -(-ctx[i] // 16))
        assert np.array_equal(w.block_tables[i, :n], ref[:n])
    others = [i for i in range(12) if i not in set(sh.tolist())]
    for i in others:
        assert not (set(w.block_tables[i, :-(-ctx[i] // 16)].tolist()) & set(ref.tolist()))


def test_pool_size_rule():
    w = W.make_workload("llama7b_mha", num_seqs=5, context=("list", [512, 600, 700, 800, 2048]))
    unique = sum(-(-c // 16) for c in [512, 600, 700, 800, 2048])
    assert w.unique_blocks == unique
    assert w.num_blocks == int(np.ceil(1.25 * unique))


def test_lognormal_context_recipe():
    rng = np.random.default_rng(1004)
    x = W._context_lens(W.SPECS["mixed_batch"], rng, 20000)
    assert x.min() >= 16 and x.max() <= 8192
    assert abs(np.median(x) - 1000) < 40


def test_fp8_scales_are_amax_over_448():
    w = W.make_workload("tiny")
    ks, vs = w.fp8_scales
    assert ks == float(np.float32(w.k_amax) / np.float32(448))
    used = _referenced_rows(w)
    kf = W.bf16_bits_to_f32(w.k_cache)
    amax = max(np.abs(kf[used]).max(), np.abs(W.bf16_bits_to_f32(w.new_k)).max())
    assert w.k_amax == amax
