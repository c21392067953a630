"""GPU parity: the HIP path (through the C ABI) against the float64 oracle,
element by element, on seeded workloads of every named shape at sizes the
oracle finishes in seconds (several tiles, ragged tails), plus edge cases.

Tolerances: decode outputs within max |err| 1e-2 and mean |err| 1e-3 of the
oracle for bf16 KV, 5e-2 / 5e-3 for fp8 KV (the fp8 oracle reads the same
cache codes); cache writes bit-exact over the whole cache, untouched bytes
included.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_mapping_amd as pa
from paged_kv_decode_mapping_amd import workloads as W

from _gpu_util import REDUCED, DeviceWorkload, compare, dev_bf16, dev_u8, host_bits, note

pytestmark = pytest.mark.gpu

BF16_TOL = (1e-2, 1e-3)
FP8_TOL = (5e-2, 5e-3)

@pytest.fixture(scope="module")
def lib(gpu):
    return pa.load_library()


def _oracle(w, **kw):
    return oracle.decode_workload(w, **kw)


@pytest.mark.parametrize("name", list(REDUCED))
@pytest.mark.parametrize("variant", ["auto", "valu", "mfma"])
def test_decode_matches_oracle(lib, name, variant):
    w = W.make_workload(name, **REDUCED[name])
    d = DeviceWorkload(w)
    if variant == "valu" and w.spec.group > 4:
        with pytest.raises(pa.PAError):
            d.decode(variant=variant)
        return
    ref = _oracle(w)
    note(f"decode {name} variant={variant} plan={pa.pa_decode_get_plan(d.q, d.k_cache, d.block_tables, variant=variant)}")
    out = d.decode(variant=variant)
    torch.cuda.synchronize()
    compare(host_bits(out), ref, *BF16_TOL)


@pytest.mark.parametrize("name", ["tiny", "long_splitk", "mixed_batch"])
@pytest.mark.parametrize("partition", [16, 48, 512, -1])
@pytest.mark.parametrize("waves", [1, 2, 4, 8])
@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_split_and_waves_agree_with_oracle(lib, name, partition, waves, variant):
    w = W.make_workload(name, **REDUCED[name])
    ref = _oracle(w)
    d = DeviceWorkload(w)
    prefetch = 1 + (waves + partition) % 3  # every ring depth, spread over the cases
    # device-built list, direct grid, or items found by each workgroup
    schedule = (1, -1, 2)[(waves + partition // 16) % 3]
    note(f"decode {name} partition={partition} waves={waves} variant={variant} prefetch={prefetch} "
         f"schedule={schedule}")
    out = d.decode(partition_tokens=partition, waves=waves, variant=variant, prefetch=prefetch,
                   schedule=schedule)
    torch.cuda.synchronize()
    compare(host_bits(out), ref, *BF16_TOL)


@pytest.mark.parametrize("name", ["tiny", "long_splitk", "mixed_batch"])
@pytest.mark.parametrize("partition", [16, 48, 512, 1024])
@pytest.mark.parametrize("wave_partitions", [1, -1])
@pytest.mark.parametrize("schedule", [1, -1, 2])
def test_wave_partitions_agree_with_oracle(lib, name, partition, wave_partitions, schedule):
    """Split contexts with one partition per wave (a workgroup covers W
    consecutive partitions, each wave storing its own state) and with the
    waves sharing one partition, on the device work list, with each
    workgroup finding its own item, and on the direct grid: ragged lengths, contexts shorter than one partition (whose single
    partition stores the output itself), a last group with waves past the
    context, and zero-length rows. bf16 and fp8 caches and both pool layouts
    alternate over the cases."""
    w = W.make_workload(name, **REDUCED[name])
    i = (partition // 16 + wave_partitions + schedule) % 4
    kv, layout = ("bf16", "fp8")[i % 2], ("page", "head_major")[i // 2]
    ks = vs = 1.0
    kc, vc, kvd, tol = w.k_cache, w.v_cache, oracle.KV_BF16, BF16_TOL
    if kv == "fp8":
        ks, vs = w.fp8_scales
        kc, vc = oracle.quantize_pool(kc, ks), oracle.quantize_pool(vc, vs)
        kvd, tol = oracle.KV_FP8_E4M3FN, FP8_TOL
    d = DeviceWorkload(w, kc, vc, layout=layout)
    opts = dict(partition_tokens=partition, wave_partitions=wave_partitions, schedule=schedule, variant="mfma")
    plan = pa.pa_decode_get_plan(d.q, d.k_cache, d.block_tables, **opts)
    assert plan["wave_partitions"] == (wave_partitions == 1 and plan["num_partitions"] > 1)
    note(f"wave partitions {name} {kv} {layout} {opts} plan={plan}")
    out = d.decode(k_scale=ks, v_scale=vs, **opts)
    torch.cuda.synchronize()
    ref = oracle.decode_workload(w, kv_dtype=kvd, k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs)
    compare(host_bits(out), ref, *tol)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("partitions", [2, 12, 24, 48, 100, 200])
def test_merge_of_many_partitions(lib, D, partitions):
    """The merge takes 1, 2, 4 or 8 waves per output row by the number of
    partition states (at 32-token partitions these counts reach each width
    for both head sizes, 200 takes several passes of the widest); rows
    ending inside a partition, and a short one that is not split."""
    P = 32
    w = W.make_workload("mixed_batch", num_seqs=3, head_dim=D,
                        context=("list", [partitions * P - 5, (partitions // 2) * P + 1, 7]))
    ref = _oracle(w)
    d = DeviceWorkload(w)
    note(f"merge D={D} partitions={partitions}")
    out = d.decode(partition_tokens=P, variant="mfma")
    torch.cuda.synchronize()
    compare(host_bits(out), ref, *BF16_TOL)


@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_decode_is_deterministic(lib, variant):
    """Repeat runs are bit-identical, and the device-built schedule (items in
    an order that depends on atomics) gives the same bits as the direct grid."""
    w = W.make_workload("mixed_batch", **REDUCED["mixed_batch"])
    d = DeviceWorkload(w)
    note(f"determinism mixed_batch {variant}")
    a = host_bits(d.decode(partition_tokens=512, variant=variant, schedule=1))
    b = host_bits(d.decode(partition_tokens=512, variant=variant, schedule=1))
    c = host_bits(d.decode(partition_tokens=512, variant=variant, schedule=-1))
    e = host_bits(d.decode(partition_tokens=512, variant=variant, schedule=2))
    assert np.array_equal(a, b)
    assert np.array_equal(a, c)
    assert np.array_equal(a, e)


@pytest.mark.parametrize("schedule", [1, -1, 2])
def test_full_size_mixed_batch_sampled(lib, schedule):
    """The mixed continuous batch at its full size (256 sequences, lognormal
    lengths, shared prefix), in the launch configuration the benchmark uses,
    checked on a sample of (sequence, KV head) units the oracle computes one
    by one."""
    w = W.make_workload("mixed_batch")
    d = DeviceWorkload(w)
    note(f"full-size mixed_batch schedule={schedule}")
    out = host_bits(d.decode(schedule=schedule))
    rng = np.random.default_rng(3)
    s = w.spec
    longest = int(np.argmax(w.context_lens))
    units = np.unique(np.concatenate([rng.choice(s.num_seqs * s.num_kv_heads, 24, replace=False),
                                      [longest * s.num_kv_heads, int(np.argmin(w.context_lens)) * s.num_kv_heads]]))
    ref = oracle.decode_workload(w, units=units)
    g = s.group
    got = np.stack([out[u // s.num_kv_heads, (u % s.num_kv_heads) * g:(u % s.num_kv_heads + 1) * g] for u in units])
    compare(got, ref, *BF16_TOL)


@pytest.mark.parametrize("name", ["llama7b_mha", "llama70b_gqa", "long_splitk", "mixed_batch"])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("layout", ["page", "head_major"])
def test_full_size_step_sampled(lib, name, kv, layout):
    """One step at the workload's full size, as the benchmark launches it:
    the cache write of the step's new tokens, then the decode with the
    library's own plan. The written rows must match the oracle's scatter
    bit for bit; the decode is checked on a sample of (sequence, KV head)
    units (the longest and the shortest context included) that the oracle
    computes one by one. fp8 caches are the oracle's quantisation of the
    whole pool (scales amax / 448). Both pool layouts: the page's
    [block, row, KV head, d] order and a head-major one."""
    w = W.make_workload(name)
    s = w.spec
    ks = vs = 1.0
    kc, vc, kvd, tol = w.k_cache, w.v_cache, oracle.KV_BF16, BF16_TOL
    if kv == "fp8":
        ks, vs = w.fp8_scales
        kc, vc = oracle.quantize_pool(kc, ks), oracle.quantize_pool(vc, vs)
        kvd, tol = oracle.KV_FP8_E4M3FN, FP8_TOL
    d = DeviceWorkload(w, kc, vc, layout=layout)
    note(f"full-size step {name} {kv} {layout} plan={pa.pa_decode_get_plan(d.q, d.k_cache, d.block_tables)}")
    pa.pa_cache_write(d.new_k, d.new_v, d.slot_mapping, d.k_cache, d.v_cache, ks, vs)
    out = host_bits(d.decode(k_scale=ks, v_scale=vs))
    torch.cuda.synchronize()

    # the host caches take the same write before the reference decode
    oracle.cache_write(w.new_k, w.new_v, w.slot_mapping, kc, vc, kv_dtype=kvd, k_scale=ks, v_scale=vs)
    slots = w.slot_mapping[w.slot_mapping >= 0]
    idx = torch.from_numpy(slots).cuda()
    for dev_cache, host_cache in ((d.k_cache, kc), (d.v_cache, vc)):
        bs = s.block_size
        rows = dev_cache[idx // bs, idx % bs].cpu()  # [T, Hkv, D] through either layout
        rows = rows.numpy() if kv == "fp8" else rows.view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(rows, host_cache.reshape(-1, s.num_kv_heads, s.head_dim)[slots])

    rng = np.random.default_rng(11)
    units = np.unique(np.concatenate([rng.choice(s.num_seqs * s.num_kv_heads, 24, replace=False),
                                      [int(np.argmax(w.context_lens)) * s.num_kv_heads + s.num_kv_heads - 1,
                                       int(np.argmin(w.context_lens)) * s.num_kv_heads]]))
    ref = oracle.decode_workload(w, units=units, kv_dtype=kvd, k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs)
    g = s.group
    got = np.stack([out[u // s.num_kv_heads, (u % s.num_kv_heads) * g:(u % s.num_kv_heads + 1) * g] for u in units])
    compare(got, ref, *tol)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("layout", ["page", "head_major"])
def test_full_size_long_contexts_at_512_token_partitions(lib, kv, layout):
    """The long-context batch as stated: 4 sequences of 32k-128k tokens split
    into flash-decoding partitions of 512 tokens (up to 256 per row) merged by
    log-sum-exp, after the step's cache write. Units are sampled over every
    sequence, each KV head of the 131,072-token one included."""
    w = W.make_workload("long_splitk")
    s = w.spec
    assert s.partition_tokens == 512
    ks = vs = 1.0
    kc, vc, kvd, tol = w.k_cache, w.v_cache, oracle.KV_BF16, BF16_TOL
    if kv == "fp8":
        ks, vs = w.fp8_scales
        kc, vc = oracle.quantize_pool(kc, ks), oracle.quantize_pool(vc, vs)
        kvd, tol = oracle.KV_FP8_E4M3FN, FP8_TOL
    d = DeviceWorkload(w, kc, vc, layout=layout)
    plan = pa.pa_decode_get_plan(d.q, d.k_cache, d.block_tables, partition_tokens=512)
    assert plan["partition_tokens"] == 512 and plan["num_partitions"] == 256
    note(f"full-size long_splitk P=512 {kv} {layout} plan={plan}")
    pa.pa_cache_write(d.new_k, d.new_v, d.slot_mapping, d.k_cache, d.v_cache, ks, vs)
    out = host_bits(d.decode(k_scale=ks, v_scale=vs, partition_tokens=512))
    torch.cuda.synchronize()
    oracle.cache_write(w.new_k, w.new_v, w.slot_mapping, kc, vc, kv_dtype=kvd, k_scale=ks, v_scale=vs)
    longest = int(np.argmax(w.context_lens))
    rng = np.random.default_rng(13)
    units = np.unique(np.concatenate([rng.choice(s.num_seqs * s.num_kv_heads, 12, replace=False),
                                      np.arange(s.num_seqs) * s.num_kv_heads + np.arange(s.num_seqs) % s.num_kv_heads,
                                      longest * s.num_kv_heads + np.arange(s.num_kv_heads)]))
    assert len(set(units // s.num_kv_heads)) == s.num_seqs
    ref = oracle.decode_workload(w, units=units, kv_dtype=kvd, k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs)
    g = s.group
    got = np.stack([out[u // s.num_kv_heads, (u % s.num_kv_heads) * g:(u % s.num_kv_heads + 1) * g] for u in units])
    compare(got, ref, *tol)


@pytest.mark.parametrize("bs", [32, 64, 256, 1024])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_other_block_sizes(lib, bs, kv):
    """Block sizes other than the workloads' 16 and 128 (any power of two from
    16 to 1024 is accepted): cache write bit-exact, decode on both kernels,
    unsplit and split, with contexts ending inside, at and just past a block."""
    ctx = [1, 17, bs - 1, bs, bs + 1, 2 * bs + 300, 40]
    w = W.make_workload("long_splitk", num_seqs=len(ctx), context=("list", ctx), block_size=bs)
    ks = vs = 1.0
    kc, vc, kvd, tol = w.k_cache, w.v_cache, oracle.KV_BF16, BF16_TOL
    if kv == "fp8":
        ks, vs = w.fp8_scales
        kc, vc = oracle.quantize_pool(kc, ks), oracle.quantize_pool(vc, vs)
        kvd, tol = oracle.KV_FP8_E4M3FN, FP8_TOL
    d = DeviceWorkload(w, kc, vc)
    note(f"block size {bs} {kv}: cache write")
    pa.pa_cache_write(d.new_k, d.new_v, d.slot_mapping, d.k_cache, d.v_cache, ks, vs)
    torch.cuda.synchronize()
    oracle.cache_write(w.new_k, w.new_v, w.slot_mapping, kc, vc, kv_dtype=kvd, k_scale=ks, v_scale=vs)
    for dev_cache, host_cache in ((d.k_cache, kc), (d.v_cache, vc)):
        got = dev_cache.cpu().numpy() if kv == "fp8" else host_bits(dev_cache)
        assert np.array_equal(got, host_cache)
    ref = _oracle(w, kv_dtype=kvd, k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs)
    for variant in ("valu", "mfma"):
        for part in (-1, 48, 512):
            note(f"block size {bs} {kv} {variant} partition={part}")
            got = host_bits(d.decode(k_scale=ks, v_scale=vs, variant=variant, partition_tokens=part))
            torch.cuda.synchronize()
            compare(got, ref, *tol)


@pytest.mark.parametrize("g", [2, 3, 5, 6, 7, 12, 16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_group_sizes(lib, g, D, kv):
    """GQA groups the named workloads do not have, powers of two or not: every
    kernel and packing that takes the shape (the VALU kernel up to 4 query
    heads per KV head, the matrix kernel up to 16, two KV heads per tile up
    to 8), unsplit and split."""
    Hkv = 4
    ctx = [1, 33, 200, 517, 1000]
    w = W.make_workload("tiny", num_seqs=len(ctx), context=("list", ctx), num_q_heads=g * Hkv,
                        num_kv_heads=Hkv, head_dim=D)
    ks = vs = 1.0
    kc, vc, kvd, tol = w.k_cache, w.v_cache, oracle.KV_BF16, BF16_TOL
    if kv == "fp8":
        ks, vs = w.fp8_scales
        kc, vc = oracle.quantize_pool(kc, ks), oracle.quantize_pool(vc, vs)
        kvd, tol = oracle.KV_FP8_E4M3FN, FP8_TOL
    ref = _oracle(w, kv_dtype=kvd, k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs)
    d = DeviceWorkload(w, kc, vc)
    shapes = [dict(variant="auto")]
    if g <= 4:
        shapes.append(dict(variant="valu"))
    shapes.append(dict(variant="mfma", heads_per_tile=1))
    if g <= 8:
        shapes.append(dict(variant="mfma", heads_per_tile=2))
    for opts in shapes:
        for part in (-1, 48):
            note(f"group {g} D {D} {kv} {opts} partition={part}")
            got = host_bits(d.decode(k_scale=ks, v_scale=vs, partition_tokens=part, **opts))
            torch.cuda.synchronize()
            compare(got, ref, *tol)


@pytest.mark.parametrize("g", [1, 8])
@pytest.mark.parametrize("scale", [0.0, 1.0, 8.0, 64.0])
def test_extreme_logits_and_a_moving_max(lib, g, scale):
    """The online softmax under stress: scores up to a few thousand (a nearly
    one-hot softmax), scale 0 (the mean of V), and for the first query head
    of every group keys aligned with its query and growing with the position,
    so that its running maximum moves on every tile and every rescale path
    runs. Both kernels where they apply, unsplit and split."""
    Hkv, D = 4, 128
    ctx = [1, 16, 17, 300, 1000]
    w = W.make_workload("tiny", num_seqs=len(ctx), context=("list", ctx), num_q_heads=g * Hkv,
                        num_kv_heads=Hkv, head_dim=D)
    kc = w.k_cache.copy()
    q32 = W.bf16_bits_to_f32(w.q)
    bs = w.spec.block_size
    for i, L in enumerate(ctx):
        for j in range(L):
            b, o = w.block_tables[i, j // bs], j % bs
            for h in range(Hkv):
                kc[b, o, h] = W._to_bf16_bits(q32[i, h * g] * np.float32(0.5 * (j + 1) / L))
    ref = oracle.decode(w.q, kc, w.v_cache, w.block_tables, w.context_lens, scale)
    d = DeviceWorkload(w, kc, w.v_cache)
    for variant in (["valu", "mfma"] if g <= 4 else ["mfma"]):
        for part in (-1, 48):
            note(f"extreme logits g={g} scale={scale} {variant} partition={part}")
            got = host_bits(pa.pa_decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, scale,
                                         variant=variant, partition_tokens=part))
            torch.cuda.synchronize()
            compare(got, ref, *BF16_TOL)


@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_edge_contexts(lib, variant):
    """ctx 0 (zeros), 1 (V exactly), exact multiples of the tile and block,
    and a context filling its whole table row."""
    ctx = [0, 1, 15, 16, 17, 32, 255, 256, 257]
    w = W.make_workload("tiny", num_seqs=len(ctx), context=("list", ctx))
    ref = _oracle(w)
    d = DeviceWorkload(w)
    for part in (-1, 16, 64):
        note(f"edge contexts partition={part} variant={variant}")
        got = host_bits(d.decode(partition_tokens=part, variant=variant))
        torch.cuda.synchronize()
        compare(got, ref, *BF16_TOL)
        assert np.all(got[0] == 0)
        g = w.spec.group
        for h in range(w.spec.num_q_heads):
            b, o = w.block_tables[1, 0], 0
            assert np.array_equal(got[1, h], w.v_cache[b, o, h // g])


@pytest.mark.parametrize("variant,name", [("valu", "llama7b_mha"), ("valu", "tiny"), ("mfma", "tiny"),
                                          ("mfma", "llama70b_gqa")])
def test_context_one_returns_v_bits(lib, variant, name):
    """ctx = 1 for every sequence: out is V's bf16 bits exactly."""
    w = W.make_workload(name, num_seqs=4, context=("list", [1] * 4))
    d = DeviceWorkload(w)
    note(f"ctx=1 exact {variant}")
    got = host_bits(d.decode(variant=variant))
    g = w.spec.group
    for i in range(4):
        b = w.block_tables[i, 0]
        for h in range(w.spec.num_q_heads):
            assert np.array_equal(got[i, h], w.v_cache[b, 0, h // g])


@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_long_block_size_128_partial_tiles(lib, variant):
    w = W.make_workload("long_splitk", num_seqs=3, context=("list", [129, 1000, 300]))
    ref = _oracle(w)
    d = DeviceWorkload(w)
    for part in (-1, 512, 128, 16):
        for prefetch in (1, 2, 3):
            note(f"bs128 partition={part} variant={variant} prefetch={prefetch}")
            compare(host_bits(d.decode(partition_tokens=part, variant=variant, prefetch=prefetch)), ref, *BF16_TOL)


def test_write_then_decode_next_position(lib):
    """A real decode step: write token ctx_i of every sequence into its next
    slot (a new block when the last one is full), then attend ctx_i + 1 tokens."""
    w = W.make_workload("tiny", context=("list", [1, 17, 63, 96]))
    bs = 16
    d = DeviceWorkload(w)
    kc_h, vc_h = w.k_cache.copy(), w.v_cache.copy()
    tables = w.block_tables.copy()
    free = [b for b in range(w.num_blocks) if b not in set(tables.ravel().tolist()) and b != w.poison_block]
    new_tables = np.full((4, tables.shape[1] + 1), w.poison_block, np.int32)
    slots = []
    for i, c in enumerate(w.context_lens):
        nb = -(-int(c) // bs)
        new_tables[i, :nb] = tables[i, :nb]
        if c % bs == 0:
            new_tables[i, nb] = free.pop()
        slots.append(int(new_tables[i, c // bs]) * bs + int(c) % bs)
    slots = np.array(slots, np.int64)
    oracle.cache_write(w.new_k, w.new_v, slots, kc_h, vc_h)
    ctx1 = (w.context_lens + 1).astype(np.int32)
    ref = oracle.decode(w.q, kc_h, vc_h, new_tables, ctx1, w.scale)
    note("write then decode")
    pa.pa_cache_write(d.new_k, d.new_v, torch.from_numpy(slots).cuda(), d.k_cache, d.v_cache)
    out = pa.pa_decode(d.q, d.k_cache, d.v_cache, torch.from_numpy(new_tables).cuda(),
                       torch.from_numpy(ctx1).cuda(), w.scale)
    compare(host_bits(out), ref, *BF16_TOL)
    assert np.array_equal(host_bits(d.k_cache), kc_h)


# ---------------------------------------------------------------- cache write

@pytest.mark.parametrize("name", ["tiny", "mixed_batch", "long_splitk"])
def test_cache_write_bf16_bit_exact(lib, name):
    w = W.make_workload(name, **REDUCED[name])
    d = DeviceWorkload(w)
    slots = w.slot_mapping.copy()
    slots[0] = -1  # padding token: nothing written
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    oracle.cache_write(w.new_k, w.new_v, slots, kc, vc)
    note(f"cache write bf16 {name}")
    pa.pa_cache_write(d.new_k, d.new_v, torch.from_numpy(slots).cuda(), d.k_cache, d.v_cache)
    assert np.array_equal(host_bits(d.k_cache), kc)
    assert np.array_equal(host_bits(d.v_cache), vc)


@pytest.mark.parametrize("name", ["tiny", "mixed_batch"])
def test_cache_write_fp8_bit_exact(lib, name):
    w = W.make_workload(name, **REDUCED[name])
    ks, vs = w.fp8_scales
    kq = oracle.quantize_pool(w.k_cache, ks)
    vq = oracle.quantize_pool(w.v_cache, vs)
    d = DeviceWorkload(w, kq, vq)
    kc, vc = kq.copy(), vq.copy()
    oracle.cache_write(w.new_k, w.new_v, w.slot_mapping, kc, vc, kv_dtype=oracle.KV_FP8_E4M3FN,
                       k_scale=ks, v_scale=vs)
    note(f"cache write fp8 {name}")
    pa.pa_cache_write(d.new_k, d.new_v, d.slot_mapping, d.k_cache, d.v_cache, ks, vs)
    assert np.array_equal(d.k_cache.cpu().numpy(), kc)
    assert np.array_equal(d.v_cache.cpu().numpy(), vc)


@pytest.mark.parametrize("scale", [1.0, 4.7 / 448, 0.0123, 17.0])
def test_cache_write_fp8_every_bf16_input(lib, scale):
    """Exhaustive device check of the quantiser: all 65536 bf16 patterns."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(512, 1, 128)
    slots = np.arange(512, dtype=np.int64)
    kc = np.zeros((32, 16, 1, 128), np.uint8)
    vc = np.zeros_like(kc)
    oracle.cache_write(bits, bits, slots, kc, vc, kv_dtype=oracle.KV_FP8_E4M3FN, k_scale=scale, v_scale=scale)
    dk, dv = dev_u8(np.zeros_like(kc)), dev_u8(np.zeros_like(vc))
    note(f"fp8 exhaustive scale={scale}")
    pa.pa_cache_write(dev_bf16(bits), dev_bf16(bits), torch.from_numpy(slots).cuda(), dk, dv, scale, scale)
    assert np.array_equal(dk.cpu().numpy(), kc)


# ---------------------------------------------------------------- fp8 decode

@pytest.mark.parametrize("name", ["tiny", "mixed_batch", "llama70b_gqa", "llama7b_mha"])
@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_decode_fp8_matches_oracle(lib, name, variant):
    w = W.make_workload(name, **REDUCED[name])
    if variant == "valu" and w.spec.group > 4:
        pytest.skip("the VALU kernel takes groups of at most 4 query heads")
    ks, vs = w.fp8_scales
    kq = oracle.quantize_pool(w.k_cache, ks)
    vq = oracle.quantize_pool(w.v_cache, vs)
    ref = _oracle(w, kv_dtype=oracle.KV_FP8_E4M3FN, k_cache=kq, v_cache=vq, k_scale=ks, v_scale=vs)
    d = DeviceWorkload(w, kq, vq)
    note(f"decode fp8 {name} {variant}")
    out = d.decode(k_scale=ks, v_scale=vs, variant=variant)
    compare(host_bits(out), ref, *FP8_TOL)
    # reported, and expected to hold: the kernel error alone is bf16-small
    compare(host_bits(out), ref, *BF16_TOL)


@pytest.mark.parametrize("name,hp", [("tiny", 1), ("tiny", 2), ("mixed_batch", 1), ("mixed_batch", 2),
                                     ("mixed_batch", 4), ("long_splitk", 4), ("llama70b_gqa", 1),
                                     ("llama70b_gqa", 2)])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_heads_per_tile_agree_with_oracle(lib, name, hp, kv):
    """The MFMA kernel packs HP adjacent KV heads into one 16-row tile (16 / HP
    tokens of each): every packing, unsplit and split, against the oracle."""
    w = W.make_workload(name, **REDUCED[name])
    ks = vs = 1.0
    kc, vc, kvd, tol = w.k_cache, w.v_cache, oracle.KV_BF16, BF16_TOL
    if kv == "fp8":
        ks, vs = w.fp8_scales
        kc, vc = oracle.quantize_pool(kc, ks), oracle.quantize_pool(vc, vs)
        kvd, tol = oracle.KV_FP8_E4M3FN, FP8_TOL
    ref = _oracle(w, kv_dtype=kvd, k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs)
    d = DeviceWorkload(w, kc, vc)
    for part in (-1, 48):
        note(f"heads_per_tile={hp} {name} {kv} partition={part}")
        got = host_bits(d.decode(k_scale=ks, v_scale=vs, variant="mfma", heads_per_tile=hp, partition_tokens=part))
        torch.cuda.synchronize()
        compare(got, ref, *tol)


@pytest.mark.parametrize("prefetch", [1, 2])
def test_fp8_decode_edge_contexts_and_pairs(lib, prefetch):
    """The fp8 MFMA kernel consumes a wave's tiles in pairs: contexts that
    leave a wave an odd number of tiles (the pair's second tile empty),
    partial tiles, one-tile partitions and empty contexts."""
    ctx = [0, 1, 15, 16, 17, 32, 48, 63, 64, 65, 200, 257]
    w = W.make_workload("tiny", num_seqs=len(ctx), context=("list", ctx))
    ks, vs = 0.02, 0.03
    kq = oracle.quantize_pool(w.k_cache, ks)
    vq = oracle.quantize_pool(w.v_cache, vs)
    ref = _oracle(w, kv_dtype=oracle.KV_FP8_E4M3FN, k_cache=kq, v_cache=vq, k_scale=ks, v_scale=vs)
    d = DeviceWorkload(w, kq, vq)
    for part in (-1, 16, 48):
        for waves in (1, 4):
            note(f"fp8 edges prefetch={prefetch} partition={part} waves={waves}")
            got = host_bits(d.decode(k_scale=ks, v_scale=vs, variant="mfma", prefetch=prefetch,
                                     partition_tokens=part, waves=waves))
            torch.cuda.synchronize()
            compare(got, ref, *FP8_TOL)
            compare(got, ref, *BF16_TOL)
            assert np.all(got[0] == 0)


@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_fp8_decode_reads_every_code_exactly(lib, variant):
    """ctx = 1 with V rows holding all 256 codes: out = code * v_scale exactly
    (NaN codes give NaN), so the device's e4m3fn decoding is the format's."""
    w = W.make_workload("tiny", num_seqs=2, context=("list", [1, 1]))
    kq = np.zeros(w.k_cache.shape, np.uint8)
    vq = np.zeros(w.v_cache.shape, np.uint8)
    codes = np.arange(256, dtype=np.uint8).reshape(2, 2, 64)  # [seq, kv head, D]
    for i in range(2):
        vq[w.block_tables[i, 0], 0] = codes[i]
    d = DeviceWorkload(w, kq, vq)
    note(f"fp8 all codes {variant}")
    got = host_bits(d.decode(k_scale=1.0, v_scale=1.0, variant=variant))
    want = oracle.e4m3fn_to_f64(codes)
    g = w.spec.group
    for i in range(2):
        for h in range(w.spec.num_q_heads):
            v = (got[i, h].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            ref = want[i, h // g]
            nan = np.isnan(ref)
            assert np.array_equal(np.isnan(v), nan)
            assert np.array_equal(v[~nan], ref[~nan])


@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_many_short_items_per_workgroup(lib, variant):
    """Hundreds of short and empty contexts: every persistent workgroup runs
    many items back to back (item lookahead, queue tickets, LDS reuse), and
    the schedule must still give the direct grid's bits."""
    rng = np.random.default_rng(21)
    ctx = rng.integers(0, 48, size=600).tolist()
    name = "llama7b_mha" if variant == "valu" else "mixed_batch"
    w = W.make_workload(name, num_seqs=len(ctx), context=("list", ctx), shared_prefix_tokens=0)
    ref = _oracle(w)
    d = DeviceWorkload(w)
    for part in (-1, 16):
        note(f"many short items {variant} partition={part}")
        a = host_bits(d.decode(variant=variant, partition_tokens=part, schedule=1))
        b = host_bits(d.decode(variant=variant, partition_tokens=part, schedule=-1))
        c = host_bits(d.decode(variant=variant, partition_tokens=part, schedule=2))
        compare(a, ref, *BF16_TOL)
        assert np.array_equal(a, b)
        assert np.array_equal(a, c)


@pytest.mark.parametrize("S,waves,partition,wpp", [(4096, 1, 16, -1), (4096, 4, 32, 1), (1, 8, 512, 1),
                                                    (37, 2, 48, -1), (256, 4, 16, -1), (64, 1, 512, -1),
                                                    (257, 8, 16, 1)])
def test_self_scheduled_items_cover_every_item(lib, S, waves, partition, wpp):
    """Each workgroup ranks its own block index among the items of
    context_lens (counts by length in LDS, then scans): by its first wave
    alone up to 256 sequences (4 a lane; 1, 37, 64 and 256 here), by the
    whole workgroup beyond (257, 4096), up to the largest batch it serves
    (4096 sequences with one wave: 64 sequences per thread). Zero,
    one-token, tile-edge, partition-edge and full-table contexts, spans of
    one partition and of a wave per partition: the oracle's output and the
    direct grid's bits."""
    rng = np.random.default_rng(S + waves)
    MB = 4
    cap = MB * 16
    edges = [0, 1, 15, 16, 17, partition - 1, partition, partition + 1, cap]
    ctx = [int(min(cap, rng.choice(edges) if rng.random() < 0.5 else rng.integers(0, cap + 1))) for _ in range(S)]
    w = W.make_workload("mixed_batch", num_seqs=S, num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                        context=("list", ctx), shared_prefix_tokens=0)
    ref = _oracle(w)
    d = DeviceWorkload(w)
    opts = dict(variant="mfma", waves=waves, partition_tokens=partition, wave_partitions=wpp)
    plan = pa.pa_decode_get_plan(d.q, d.k_cache, d.block_tables, schedule=2, **opts)
    assert plan["self_scheduled"]
    note(f"self-scheduled S={S} {opts} plan={plan}")
    a = host_bits(d.decode(schedule=2, **opts))
    b = host_bits(d.decode(schedule=-1, **opts))
    compare(a, ref, *BF16_TOL)
    assert np.array_equal(a, b)
    va = host_bits(d.decode(schedule=2, variant="valu", waves=waves, partition_tokens=partition))
    compare(va, ref, *BF16_TOL)


def _copy_case(rng, N, n, extra_bad=True):
    """n (src, dst) pairs: distinct destinations, no block both a source and a
    destination; plus padding and out-of-pool pairs that must be skipped."""
    ids = rng.permutation(N)
    pairs = [[int(ids[i]), int(ids[n + i])] for i in range(n)]
    if extra_bad:
        pairs += [[-1, int(ids[2 * n])], [int(ids[2 * n + 1]), -5], [N + 3, int(ids[2 * n + 2])],
                  [int(ids[2 * n + 3]), N]]
    return np.array(pairs, np.int64)


@pytest.mark.parametrize("name,kv", [("tiny", "bf16"), ("mixed_batch", "bf16"), ("mixed_batch", "fp8"),
                                     ("long_splitk", "bf16")])
def test_copy_blocks_bit_exact(lib, name, kv):
    """Every byte of both caches equals the oracle's copy (skipped pairs and
    untouched blocks included)."""
    rng = np.random.default_rng(21)
    w = W.make_workload(name, **REDUCED[name])
    kc, vc = w.k_cache, w.v_cache
    if kv == "fp8":
        kc = oracle.quantize_pool(kc, 0.05)
        vc = oracle.quantize_pool(vc, 0.07)
    N = w.num_blocks
    n = min(40, (N - 4) // 2)
    pairs = _copy_case(rng, N, n)
    ek, ev = kc.copy(), vc.copy()
    oracle.copy_blocks(ek, ev, pairs[(pairs >= 0).all(1) & (pairs < N).all(1)])
    d = DeviceWorkload(w, kc, vc)
    note(f"copy_blocks {name} {kv} pairs={len(pairs)}")
    pa.pa_copy_blocks(d.k_cache, d.v_cache, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    gk = d.k_cache.cpu().numpy() if d.fp8 else host_bits(d.k_cache)
    gv = d.v_cache.cpu().numpy() if d.fp8 else host_bits(d.v_cache)
    assert np.array_equal(gk, ek) and np.array_equal(gv, ev)


def test_copy_blocks_then_decode_through_copies(lib):
    """Copy-on-write round trip on the device: copy every block the batch
    uses to free blocks, repoint the tables, decode: the output bits equal
    the decode through the originals."""
    w = W.make_workload("mixed_batch", **REDUCED["mixed_batch"])
    d = DeviceWorkload(w)
    note("copy_blocks then decode")
    before = host_bits(d.decode())
    tb = w.block_tables.copy()
    nblk = [(int(c) + 15) // 16 for c in w.context_lens]
    every = {int(tb[i, j]) for i in range(len(nblk)) for j in range(nblk[i])}
    taken = every | {int(w.poison_block)} | set((w.slot_mapping // w.spec.block_size).tolist())
    free = [b for b in range(w.num_blocks) if b not in taken]
    # the sequences whose blocks fit in the free ones
    chosen, used = [], []
    for i in range(len(nblk)):
        new = [int(b) for b in dict.fromkeys(tb[i, :nblk[i]].tolist()) if int(b) not in used]
        if len(used) + len(new) <= len(free):
            chosen.append(i)
            used += new
    assert len(chosen) >= 3, chosen
    remap = dict(zip(used, free))
    pa.pa_copy_blocks(d.k_cache, d.v_cache, torch.tensor([[u, remap[u]] for u in used], dtype=torch.int64).cuda())
    for i in chosen:
        for j in range(nblk[i]):
            tb[i, j] = remap[int(tb[i, j])]
    d.block_tables = torch.from_numpy(tb).cuda()
    after = host_bits(d.decode())
    torch.cuda.synchronize()
    assert np.array_equal(before, after)


def test_tutorial_paged_cache_example(lib):
    """The worked example of Tutorial §4.2 (PagedKVCache usage: 5 sequences of
    100 tokens, 32 KV heads of 128, blocks of 16 in a pool of 500), one layer:
    pa_cache_write of all 500 tokens through the slots the example's block
    tables imply (tests/golden/), then pa_decode. The pool matches the
    oracle's cache write bit for bit and the output matches the oracle."""
    import json, math, os
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tutorial_4_2_paged_cache_example.json")))
    bs, N, Hkv, D = fx["block_size"], fx["num_blocks"], fx["num_kv_heads"], fx["head_dim"]
    lens = fx["seq_lengths"]
    S, T = len(lens), sum(lens)
    slots = np.array([fx["block_tables"][i][j // bs] * bs + j % bs for i, L in enumerate(lens) for j in range(L)],
                     np.int64)
    rng = np.random.default_rng(43)
    bits = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    k = bits(rng.standard_normal((T, Hkv, D)))
    v = bits(rng.standard_normal((T, Hkv, D)))
    q = bits(rng.standard_normal((S, Hkv, D)))
    kc = np.zeros((N, bs, Hkv, D), np.uint16)
    vc = np.zeros_like(kc)
    oracle.cache_write(k, v, slots, kc, vc)
    tables = np.array(fx["block_tables"], np.int32)
    ctx = np.array(lens, np.int32)
    ref = oracle.decode(q, kc, vc, tables, ctx, 1.0 / math.sqrt(D))
    dk = torch.zeros((N, bs, Hkv, D), dtype=torch.bfloat16, device="cuda")
    dv = torch.zeros_like(dk)
    note("tutorial paged cache example")
    pa.pa_cache_write(dev_bf16(k), dev_bf16(v), torch.from_numpy(slots).cuda(), dk, dv)
    out = pa.pa_decode(dev_bf16(q), dk, dv, torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda(),
                       1.0 / math.sqrt(D))
    assert np.array_equal(host_bits(dk), kc) and np.array_equal(host_bits(dv), vc)
    compare(host_bits(out), ref, *BF16_TOL)
