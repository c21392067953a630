"""Pins of the CPU oracle against things other than itself (no GPU).

Each test names what it pins the oracle to: a library routine (torch's
scaled_dot_product_attention in float64, torch's float8_e4m3fn conversion,
numpy's fancy-index assignment), a closed form, an invariant, or brute force.
Between them they catch the plausible mistakes: a wrong query-head -> KV-head
map, an off-by-one in the block-table walk, reading past the context, a
missing max subtraction, a wrong scale, a transposed operand, a wrong fp8
rounding or saturation rule.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_mapping_amd import workloads as W

bf16_f32 = W.bf16_bits_to_f32


def _bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _identity_paged(ctx, Hq, Hkv, D, bs, rng, k_mult=1.0, spare_blocks=2):
    """Contiguous per-sequence K/V (the non-paged KVCache form) stored in a pool
    whose block table is the identity: seq i owns consecutive blocks. The
    pool rows past each context and the spare blocks hold NaN."""
    S = len(ctx)
    nblk = [(c + bs - 1) // bs for c in ctx]
    N = sum(nblk) + spare_blocks
    MB = max(1, max(nblk))
    kpool = np.full((N * bs, Hkv, D), 0x7FC0, np.uint16)
    vpool = np.full((N * bs, Hkv, D), 0x7FC0, np.uint16)
    tables = np.full((S, MB), N - 1, np.int32)
    q = _bits(rng.standard_normal((S, Hq, D)))
    dense = []
    start = 0
    for i, c in enumerate(ctx):
        k = _bits(rng.standard_normal((c, Hkv, D)) * k_mult)
        v = _bits(rng.standard_normal((c, Hkv, D)))
        kpool[start * bs:start * bs + c] = k
        vpool[start * bs:start * bs + c] = v
        tables[i, :nblk[i]] = np.arange(start, start + nblk[i])
        dense.append((k, v))
        start += nblk[i]
    return (q, kpool.reshape(N, bs, Hkv, D), vpool.reshape(N, bs, Hkv, D), tables,
            np.asarray(ctx, np.int32), dense)


CASES = [  # (Hq, Hkv, D, bs, ctx)
    (8, 2, 64, 16, [1, 17, 64, 100]),
    (4, 4, 32, 4, [3, 8, 9, 30]),
    (8, 1, 16, 8, [5, 16, 33]),
    (6, 3, 8, 1, [1, 2, 7]),
    (16, 2, 128, 16, [40, 129]),
]


@pytest.mark.parametrize("Hq,Hkv,D,bs,ctx", CASES)
def test_decode_matches_torch_sdpa_f64(Hq, Hkv, D, bs, ctx):
    """Pin: torch.nn.functional.scaled_dot_product_attention (float64, enable_gqa)
    on the dense contiguous K/V equals the oracle on the identity-paged pool."""
    rng = np.random.default_rng(7)
    q, kc, vc, tables, ctxa, dense = _identity_paged(ctx, Hq, Hkv, D, bs, rng)
    scale = 1.0 / math.sqrt(D)
    got = oracle.decode(q, kc, vc, tables, ctxa, scale)
    for i, (k, v) in enumerate(dense):
        qt = torch.from_numpy(bf16_f32(q[i]).astype(np.float64))[None, :, None, :]
        kt = torch.from_numpy(bf16_f32(k).astype(np.float64)).permute(1, 0, 2)[None]
        vt = torch.from_numpy(bf16_f32(v).astype(np.float64)).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
        np.testing.assert_allclose(got[i], ref[0, :, 0, :].numpy(), rtol=0, atol=1e-12)


def test_decode_matches_sdpa_sharp_softmax():
    """Same library pin with K x 3 (the long-context recipe) and a larger scale."""
    rng = np.random.default_rng(11)
    q, kc, vc, tables, ctxa, dense = _identity_paged([300, 77], 8, 2, 64, 16, rng, k_mult=3.0)
    got = oracle.decode(q, kc, vc, tables, ctxa, 0.5)
    for i, (k, v) in enumerate(dense):
        qt = torch.from_numpy(bf16_f32(q[i]).astype(np.float64))[None, :, None, :]
        kt = torch.from_numpy(bf16_f32(k).astype(np.float64)).permute(1, 0, 2)[None]
        vt = torch.from_numpy(bf16_f32(v).astype(np.float64)).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.5, enable_gqa=True)
        np.testing.assert_allclose(got[i], ref[0, :, 0, :].numpy(), rtol=0, atol=1e-11)


def _permute_blocks(w_q, kc, vc, tables, rng):
    N = kc.shape[0]
    pi = rng.permutation(N)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    return kc2, vc2, pi[tables].astype(np.int32)


def test_block_permutation_invariance():
    """Pin (invariant): relabelling physical blocks, with the tables relabelled
    the same way, leaves the output bit-identical; so does changing what the
    unreferenced rows hold."""
    w = W.make_workload("tiny")
    base = oracle.decode_workload(w)
    rng = np.random.default_rng(3)
    for _ in range(3):
        kc, vc, tb = _permute_blocks(w.q, w.k_cache, w.v_cache, w.block_tables, rng)
        got = oracle.decode(w.q, kc, vc, tb, w.context_lens, w.scale)
        assert np.array_equal(got, base)
    # fill every unreferenced row with large finite values instead of NaN
    w2 = W.make_workload("tiny", poison=False)
    kc, vc = w2.k_cache.copy(), w2.v_cache.copy()
    used = np.zeros(kc.shape[:2], bool)
    for i, c in enumerate(w2.context_lens):
        for j in range(c):
            used[w2.block_tables[i, j // 16], j % 16] = True
    kc[~used] = _bits(np.full((1, 2, 64), 50.0))
    vc[~used] = _bits(np.full((1, 2, 64), -7.0))
    got = oracle.decode(w2.q, kc, vc, w2.block_tables, w2.context_lens, w2.scale)
    assert np.array_equal(got, base)
    assert np.all(np.isfinite(base))


def test_context_one_returns_v_exactly():
    """Closed form: with one cached token the softmax weight is exactly 1."""
    rng = np.random.default_rng(5)
    q, kc, vc, tables, ctxa, dense = _identity_paged([1, 1, 1], 8, 2, 64, 16, rng)
    got = oracle.decode(q, kc, vc, tables, ctxa, 0.125)
    for i, (k, v) in enumerate(dense):
        want = np.repeat(bf16_f32(v[0]).astype(np.float64), 4, axis=0)  # head h reads KV head h // 4
        assert np.array_equal(got[i], want)


def test_identical_keys_and_zero_scale_give_mean_v():
    """Closed forms: identical keys, or scale 0, give the plain mean of V."""
    rng = np.random.default_rng(9)
    q, kc, vc, tables, ctxa, dense = _identity_paged([37, 64], 4, 2, 32, 16, rng)
    for i, c in enumerate(ctxa):
        mean_v = bf16_f32(dense[i][1]).astype(np.float64).mean(axis=0)  # [Hkv, D]
        want = np.repeat(mean_v, 2, axis=0)
        got0 = oracle.decode(q, kc, vc, tables, ctxa, 0.0)[i]
        np.testing.assert_allclose(got0, want, rtol=1e-14, atol=1e-15)
    # identical keys: overwrite every context row's K with one row
    kc2 = kc.copy()
    one = _bits(rng.standard_normal((2, 32)))
    for i, c in enumerate(ctxa):
        for j in range(c):
            kc2[tables[i, j // 16], j % 16] = one
    got = oracle.decode(q, kc2, vc, tables, ctxa, 0.3)
    for i in range(2):
        mean_v = bf16_f32(dense[i][1]).astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(got[i], np.repeat(mean_v, 2, axis=0), rtol=1e-14, atol=1e-15)


def test_dominant_key_and_large_logits_are_stable():
    """Closed form: one key aligned with q at a huge logit takes all the weight;
    logits in the thousands must not overflow (max subtraction)."""
    rng = np.random.default_rng(13)
    q, kc, vc, tables, ctxa, dense = _identity_paged([50], 2, 1, 16, 16, rng)
    qf = bf16_f32(q[0, 0])
    star = 23
    kc2 = kc.copy()
    kc2[tables[0, star // 16], star % 16, 0] = _bits(qf * 100.0)
    got = oracle.decode(q, kc2, vc, tables, ctxa, 1.0)
    want = bf16_f32(dense[0][1][star, 0]).astype(np.float64)
    np.testing.assert_allclose(got[0, 0], want, rtol=0, atol=1e-12)
    assert np.all(np.isfinite(got))


def test_empty_context_gives_zero():
    rng = np.random.default_rng(1)
    q, kc, vc, tables, ctxa, _ = _identity_paged([5, 3], 4, 2, 16, 4, rng)
    ctxa = np.array([0, 3], np.int32)
    got = oracle.decode(q, kc, vc, tables, ctxa, 0.25)
    assert np.array_equal(got[0], np.zeros_like(got[0]))


def test_gqa_equals_mha_on_repeated_kv_heads():
    """Pin (special case): GQA with group g equals MHA on a cache whose KV heads
    are repeated g times in place (repeat_interleave along the head axis). A
    head map of h mod Hkv instead of h div g fails this."""
    w = W.make_workload("tiny")
    gqa = oracle.decode_workload(w)
    g = w.spec.group
    kc = np.repeat(w.k_cache, g, axis=2)
    vc = np.repeat(w.v_cache, g, axis=2)
    mha = oracle.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale)
    assert np.array_equal(gqa, mha)


def test_gqa_kv_head_permutation_permutes_outputs():
    """Invariant: permuting KV heads (and the matching query-head groups)
    permutes the outputs; equal queries inside a group give equal outputs."""
    rng = np.random.default_rng(17)
    q, kc, vc, tables, ctxa, _ = _identity_paged([20, 45], 12, 3, 32, 8, rng)
    base = oracle.decode(q, kc, vc, tables, ctxa, 0.2)
    sigma = np.array([2, 0, 1])
    g = 4
    qperm = q.reshape(2, 3, g, 32)[:, sigma].reshape(2, 12, 32)
    got = oracle.decode(qperm, kc[:, :, sigma], vc[:, :, sigma], tables, ctxa, 0.2)
    assert np.array_equal(got, base.reshape(2, 3, g, 32)[:, sigma].reshape(2, 12, 32))
    q2 = q.copy()
    q2[:, 4:8] = q2[:, 4:5]
    out2 = oracle.decode(q2, kc, vc, tables, ctxa, 0.2)
    for h in range(5, 8):
        assert np.array_equal(out2[:, h], out2[:, 4])


def test_decode_units_subset_matches_full():
    w = W.make_workload("tiny")
    full = oracle.decode_workload(w)
    units = [5, 0, 3]
    sub = oracle.decode_workload(w, units=units)
    g = w.spec.group
    for n, u in enumerate(units):
        s, k = divmod(u, w.spec.num_kv_heads)
        assert np.array_equal(sub[n], full[s, k * g:(k + 1) * g])


def test_split_merge_identity_f64():
    """Pins the split-K reading: partial softmax states over 512-, 48- and
    16-token partitions merged by log-sum-exp reproduce the oracle (an identity
    of exact arithmetic, checked to 1e-12)."""
    w = W.reduced("long_splitk", 2, [700, 1300], block_size=16)
    ref = oracle.decode_workload(w)
    S, Hq, D = w.q.shape
    Hkv = w.spec.num_kv_heads
    g = Hq // Hkv
    for P in (512, 48, 16):
        out = np.zeros_like(ref)
        for i in range(S):
            L = int(w.context_lens[i])
            rows = [(w.block_tables[i, j // 16], j % 16) for j in range(L)]
            K = bf16_f32(np.stack([w.k_cache[b, o] for b, o in rows])).astype(np.float64)
            V = bf16_f32(np.stack([w.v_cache[b, o] for b, o in rows])).astype(np.float64)
            for h in range(Hq):
                qh = bf16_f32(w.q[i, h]).astype(np.float64)
                ms, ls, os_ = [], [], []
                for p0 in range(0, L, P):
                    s = K[p0:p0 + P, h // g] @ qh * w.scale
                    m = s.max()
                    e = np.exp(s - m)
                    ms.append(m)
                    ls.append(e.sum())
                    os_.append(e @ V[p0:p0 + P, h // g])
                M = max(ms)
                Lsum = sum(l * math.exp(m - M) for m, l in zip(ms, ls))
                out[i, h] = sum(o * math.exp(m - M) for m, o in zip(ms, os_)) / Lsum
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- cache write

def test_cache_write_bf16_matches_numpy_scatter():
    """Pin: numpy fancy-index assignment into the flat [N*bs, Hkv, D] row view.
    Slot -1 writes nothing; every other byte is untouched."""
    w = W.make_workload("tiny")
    slots = w.slot_mapping.copy()
    slots[1] = -1
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    n = oracle.cache_write(w.new_k, w.new_v, slots, kc, vc)
    assert n == len(slots) - 1
    ek, ev = w.k_cache.copy(), w.v_cache.copy()
    keep = slots >= 0
    ek.reshape(-1, 2, 64)[slots[keep]] = w.new_k[keep]
    ev.reshape(-1, 2, 64)[slots[keep]] = w.new_v[keep]
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)


def test_cache_write_rejects_out_of_pool_slot():
    w = W.make_workload("tiny")
    slots = w.slot_mapping.copy()
    slots[0] = w.num_blocks * 16
    with pytest.raises(ValueError):
        oracle.cache_write(w.new_k, w.new_v, slots, w.k_cache.copy(), w.v_cache.copy())


# ---------------------------------------------------------------- multi-token

MULTI_CASES = [  # (Hq, Hkv, D, bs, ctx, q_lens)
    (8, 2, 64, 16, [1, 17, 64, 100], [1, 5, 16, 4]),
    (4, 4, 32, 4, [3, 8, 9, 30], [3, 2, 0, 7]),
    (8, 1, 16, 8, [5, 16, 33], [5, 1, 33]),
]


@pytest.mark.parametrize("Hq,Hkv,D,bs,ctx,qlens", MULTI_CASES)
def test_multi_matches_torch_sdpa_with_bottom_right_causal_mask(Hq, Hkv, D, bs, ctx, qlens):
    """Pin: torch scaled_dot_product_attention in float64 on the dense K/V of
    each sequence, with an explicit boolean mask that lets query r (position
    L - n + r) see positions 0..L - n + r."""
    rng = np.random.default_rng(41)
    _, kc, vc, tables, ctx_a, dense = _identity_paged(ctx, Hq, Hkv, D, bs, rng)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = _bits(rng.standard_normal((int(qs[-1]), Hq, D)))
    scale = 1.0 / math.sqrt(D)
    got = oracle.multi_decode(q, kc, vc, tables, ctx_a, qs, scale)
    g = Hq // Hkv
    for i, (k, v) in enumerate(dense):
        n, L = qlens[i], ctx[i]
        if n == 0:
            continue
        qt = torch.from_numpy(bf16_f32(q[qs[i]:qs[i + 1]]).astype(np.float64)).permute(1, 0, 2)  # [Hq, n, D]
        kt = torch.from_numpy(bf16_f32(k).astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)
        vt = torch.from_numpy(bf16_f32(v).astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)
        mask = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
        np.testing.assert_allclose(got[qs[i]:qs[i + 1]], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_multi_row_equals_decode_of_the_truncated_context():
    """Pin (invariant, against the decode oracle): query r of a sequence gives
    exactly the single-token decode of that query over the first L - n + r + 1
    tokens; with one query token per sequence the whole result is the decode."""
    w = W.make_workload("tiny", poison=True)
    qlens = [1, 9, 30, 17]
    mq = W.make_multi_query(w, qlens)
    got = oracle.multi_decode(mq.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, mq.query_start, w.scale)
    for i, n in enumerate(qlens):
        L = int(w.context_lens[i])
        for r in range(n):
            row = int(mq.query_start[i]) + r
            one_q = np.repeat(mq.q[row][None], w.spec.num_seqs, axis=0)
            trunc = w.context_lens.copy()
            trunc[:] = 0
            trunc[i] = L - n + r + 1
            ref = oracle.decode(one_q, w.k_cache, w.v_cache, w.block_tables, trunc, w.scale)
            assert np.array_equal(got[row], ref[i])
    mq1 = W.make_multi_query(w, [1] * w.spec.num_seqs)
    got1 = oracle.multi_decode(mq1.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, mq1.query_start,
                               w.scale)
    ref1 = oracle.decode(mq1.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale)
    assert np.array_equal(got1, ref1)


# ---------------------------------------------------------------- cascade (shared prefix)

def _dense_cascade(rng, Hq, Hkv, D, bs, groups, lead, tail, max_group_size):
    """Dense K/V of each group's prefix and each sequence's own tokens, stored
    in scattered pool blocks. Members' own rows name a NaN block wherever the
    prefix lies; a member past max_group_size holds its whole context in its
    own row. Returns the cascade arguments and, per sequence, the dense K/V
    it must attend to (prefix[:shared] followed by its own tokens)."""
    blocks = [np.full((bs, Hkv, D), 0x7FC0, np.uint16)]  # block 0: NaN
    kblk, vblk = [blocks[0]], [blocks[0].copy()]

    def store(k, v):
        ids = []
        for b0 in range(0, len(k), bs):
            kb = np.full((bs, Hkv, D), 0x7FC0, np.uint16)
            vb = kb.copy()
            kb[:len(k[b0:b0 + bs])] = k[b0:b0 + bs]
            vb[:len(v[b0:b0 + bs])] = v[b0:b0 + bs]
            kblk.append(kb)
            vblk.append(vb)
            ids.append(len(kblk) - 1)
        return ids

    ctx, grp = list(lead), [-1] * len(lead)
    starts = [len(lead)]
    prefixes, ptables = [], []
    for k, (ptok, members) in enumerate(groups):
        pk = _bits(rng.standard_normal((ptok, Hkv, D)))
        pv = _bits(rng.standard_normal((ptok, Hkv, D)))
        prefixes.append((pk, pv))
        ptables.append(store(pk, pv))
        ctx += members
        grp += [k if j < max_group_size else -1 for j in range(len(members))]
        starts.append(len(ctx))
    ctx += list(tail)
    grp += [-1] * len(tail)
    S = len(ctx)
    q = _bits(rng.standard_normal((S, Hq, D)))
    rows, dense = [], []
    for i in range(S):
        shared = min(ctx[i], groups[grp[i]][0]) if grp[i] >= 0 else 0
        own_k = _bits(rng.standard_normal((ctx[i] - shared, Hkv, D)))
        own_v = _bits(rng.standard_normal((ctx[i] - shared, Hkv, D)))
        row = [0] * ((shared + bs - 1) // bs) + store(own_k, own_v)
        rows.append(row)
        if grp[i] >= 0:
            pk, pv = prefixes[grp[i]]
            dense.append((np.concatenate([pk[:shared], own_k]), np.concatenate([pv[:shared], own_v])))
        else:
            dense.append((own_k, own_v))
    N = len(kblk)
    pi = np.concatenate([[0], 1 + rng.permutation(N - 1)])  # scatter every block but the NaN one
    kc = np.empty((N, bs, Hkv, D), np.uint16)
    vc = np.empty_like(kc)
    kc[pi] = np.stack(kblk)
    vc[pi] = np.stack(vblk)
    MB = max(1, max(len(r) for r in rows))
    tables = np.zeros((S, MB), np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = pi[r]
    PMB = max([1] + [len(t) for t in ptables])
    pt = np.zeros((len(groups), PMB), np.int32)
    for k, t in enumerate(ptables):
        pt[k, :len(t)] = pi[t]
    return (q, kc, vc, tables, np.asarray(ctx, np.int32), pt,
            np.array([g[0] for g in groups], np.int32), np.asarray(starts, np.int32), dense)


def test_cascade_matches_torch_sdpa_on_dense_prefix_and_suffix():
    """Pin: torch scaled_dot_product_attention (float64, enable_gqa) over
    prefix[:shared_i] followed by sequence i's own tokens, built as dense
    arrays. The members' own rows hold a NaN block where the prefix lies, so
    only a gather through the prefix table gives this. Covers a member
    shorter than its prefix, empty contexts, a zero-length prefix, an empty
    group, sequences in no group before and after the groups, and a member
    past max_group_size (it reads its whole context through its own row)."""
    rng = np.random.default_rng(97)
    Hq, Hkv, D, bs = 8, 2, 32, 8
    groups = [(24, [24, 40, 10, 30]), (0, [7]), (16, []), (40, [41, 80, 0])]
    q, kc, vc, tables, ctx, pt, pl, gs, dense = _dense_cascade(rng, Hq, Hkv, D, bs, groups, [9], [0, 33], 3)
    scale = 1.0 / math.sqrt(D)
    got = oracle.cascade_decode(q, kc, vc, tables, ctx, pt, pl, gs, scale, max_group_size=3)
    for i, (k, v) in enumerate(dense):
        if len(k) == 0:
            assert np.all(got[i] == 0.0)
            continue
        qt = torch.from_numpy(bf16_f32(q[i]).astype(np.float64))[None, :, None, :]
        kt = torch.from_numpy(bf16_f32(k).astype(np.float64)).permute(1, 0, 2)[None]
        vt = torch.from_numpy(bf16_f32(v).astype(np.float64)).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
        np.testing.assert_allclose(got[i], ref[0, :, 0, :].numpy(), rtol=0, atol=1e-12)
    # the members' own rows alone give NaN where they rely on the prefix
    plain = oracle.decode(q, kc, vc, tables, ctx, scale)
    assert np.isnan(plain[2]).all() and np.isfinite(got).all()


def test_cascade_equals_decode_when_members_name_the_prefix_blocks():
    """Pin (invariant, against the decode oracle): when every member's table
    names its group's prefix blocks, as a prefix cache hands them out, the
    cascade result is bit-identical to the decode of the same batch; with
    those entries of the members' rows replaced by a NaN block, the cascade
    result does not change while the plain decode turns NaN."""
    b = W.make_prefix_groups(num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                             groups=[(64, [64, 100, 30, 200]), (160, [500, 160, 1]), (32, []), (0, [50, 0])],
                             lead=[5], tail=[0, 17, 300], seed=5)
    args = (b.prefix_tables, b.prefix_lens, b.group_start, b.scale)
    ref = oracle.decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.scale)
    got = oracle.cascade_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, *args)
    assert np.array_equal(got, ref)
    poisoned = b.block_tables.copy()
    for k in range(b.num_groups):
        nb = int(b.prefix_lens[k]) // b.block_size
        poisoned[b.group_start[k]:b.group_start[k + 1], :nb] = b.poison_block
    got2 = oracle.cascade_decode(b.q, b.k_cache, b.v_cache, poisoned, b.context_lens, *args)
    assert np.array_equal(got2, ref)
    bad = oracle.decode(b.q, b.k_cache, b.v_cache, poisoned, b.context_lens, b.scale)
    assert np.isnan(bad[1:8]).any(axis=(1, 2)).all()  # members of groups 0 and 1


def test_cascade_tables_reject_malformed_groups():
    b = W.make_prefix_groups(num_q_heads=4, num_kv_heads=2, head_dim=16, block_size=16,
                             groups=[(32, [40, 50])], seed=1)
    base = (b.block_tables, b.context_lens)
    with pytest.raises(AssertionError):
        oracle.cascade_tables(*base, b.prefix_tables, np.array([20], np.int32), b.group_start, 16)
    with pytest.raises(AssertionError):
        oracle.cascade_tables(*base, b.prefix_tables, b.prefix_lens, np.array([2, 0], np.int32), 16)
    with pytest.raises(AssertionError):
        oracle.cascade_tables(*base, b.prefix_tables, np.array([48], np.int32), b.group_start, 16)


def test_multi_rejects_more_queries_than_context():
    w = W.make_workload("tiny")
    qs = np.array([0, 2, 2, 2, 2], np.int32)  # sequence 0 has one cached token
    q = np.zeros((2, 8, 64), np.uint16)
    with pytest.raises(ValueError):
        oracle.multi_decode(q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, qs, w.scale)


# ---------------------------------------------------------------- block copy

def _copy_pairs(rng, N, n):
    ids = rng.permutation(N)
    pairs = np.stack([ids[:n], ids[n:2 * n]], axis=1).astype(np.int64)
    return pairs


@pytest.mark.parametrize("dtype", [np.uint16, np.uint8])
def test_copy_blocks_matches_numpy_block_assignment(dtype):
    """Pin: numpy's block-level fancy-index assignment cache[dst] = cache[src]
    (the right side is gathered before the store, so it reads the pre-call
    state), including a chain where a destination is also a source and
    padding pairs; every other block is untouched."""
    rng = np.random.default_rng(11)
    N, bs, Hkv, D = 40, 16, 2, 64
    hi = 65535 if dtype == np.uint16 else 255
    kc = rng.integers(0, hi, (N, bs, Hkv, D), dtype=dtype)
    vc = rng.integers(0, hi, (N, bs, Hkv, D), dtype=dtype)
    pairs = np.concatenate([_copy_pairs(rng, N, 9), [[-1, 3], [4, -1], [7, 30], [30, 31]]]).astype(np.int64)
    pairs = pairs[np.unique(pairs[:, 1], return_index=True)[1]]  # distinct destinations
    ek, ev = kc.copy(), vc.copy()
    keep = (pairs >= 0).all(axis=1)
    ek[pairs[keep, 1]] = kc[pairs[keep, 0]]
    ev[pairs[keep, 1]] = vc[pairs[keep, 0]]
    n = oracle.copy_blocks(kc, vc, pairs)
    assert n == int(keep.sum())
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)


def test_copy_blocks_then_repointed_table_decodes_the_same():
    """Pin (invariant): after copying every block a sequence uses to fresh
    blocks and repointing its table there, the decode is bit-identical."""
    w = W.make_workload("tiny", poison=False)
    base = oracle.decode_workload(w)
    kc, vc, tb = w.k_cache.copy(), w.v_cache.copy(), w.block_tables.copy()
    used = sorted({int(tb[i, j]) for i, c in enumerate(w.context_lens) for j in range((c + 15) // 16)})
    free = [b for b in range(w.num_blocks) if b not in used][:len(used)]
    assert len(free) == len(used)
    oracle.copy_blocks(kc, vc, np.array(list(zip(used, free)), np.int64))
    remap = dict(zip(used, free))
    for i, c in enumerate(w.context_lens):
        for j in range((c + 15) // 16):
            tb[i, j] = remap[int(tb[i, j])]
    got = oracle.decode(w.q, kc, vc, tb, w.context_lens, w.scale)
    assert np.array_equal(got, base)


def test_copy_blocks_rejects_bad_pairs():
    kc = np.zeros((4, 2, 1, 8), np.uint16)
    vc = np.zeros_like(kc)
    with pytest.raises(ValueError):
        oracle.copy_blocks(kc, vc, [[0, 4]])
    with pytest.raises(ValueError):
        oracle.copy_blocks(kc, vc, [[0, 2], [1, 2]])


# ---------------------------------------------------------------- bf16 codec

def test_bf16_decode_all_patterns_match_torch():
    """Pin: torch's bfloat16 -> float64 over all 65,536 bit patterns (NaN
    payloads aside: every NaN pattern decodes to a NaN)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert nan.sum() == 2 * 127 and got[0x3F80] == 1.0 and got[0x0001] == 2.0 ** -133
    assert np.isinf(got[0x7F80]) and got[0xFF80] == -np.inf and math.copysign(1.0, got[0x8000]) == -1.0


# ---------------------------------------------------------------- fp8 codec

def test_e4m3fn_decode_all_codes_match_torch():
    """Pin: torch's float8_e4m3fn -> float64 over all 256 codes."""
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert nan.sum() == 2 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e4m3fn_encode_all_bf16_inputs():
    """Pin: every bf16 bit pattern (as float32) encodes as torch does where
    torch's rule is defined the same way (|x| <= 464, its tie point with the
    next binade), saturates to +-448 above, and NaN stays NaN."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16_f32(bits)
    got = oracle.f32_to_e4m3fn(x)
    ref = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    a = np.abs(x)
    inrange = a <= 464
    assert np.array_equal(got[inrange], ref[inrange])
    big = (a > 464) & np.isfinite(x)
    assert np.all((got[big] & 0x7F) == 0x7E)
    assert np.array_equal(got[big] >> 7, (x[big] < 0).astype(np.uint8))
    inf = np.isinf(x)
    assert np.all((got[inf] & 0x7F) == 0x7E)
    nan = np.isnan(x)
    assert np.all((got[nan] & 0x7F) == 0x7F)


def test_e4m3fn_encode_is_nearest_brute_force():
    """Brute force: the code is a nearest grid point; ties pick the even code."""
    rng = np.random.default_rng(23)
    x = np.concatenate([rng.standard_normal(3000) * 30, rng.standard_normal(1000) * 0.01]).astype(np.float32)
    grid = oracle.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    got = oracle.f32_to_e4m3fn(x)
    val = oracle.e4m3fn_to_f64(got)
    err = np.abs(val - x.astype(np.float64))
    best = np.min(np.abs(grid[None, :] - np.abs(x.astype(np.float64))[:, None]), axis=1)
    assert np.array_equal(err, best)
    # exact midpoints between neighbouring codes go to the even code
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    c = oracle.f32_to_e4m3fn(mids)
    assert np.all(c % 2 == 0)


@pytest.mark.parametrize("scale", [1.0, 4.7 / 448, 13.0 / 448, 0.0123])
def test_quantize_bf16_matches_torch_division_then_cast(scale):
    """Pin: torch float32 division then torch's e4m3fn cast, over all bf16 inputs."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.quantize_bf16(bits, scale)
    y = (torch.from_numpy(bf16_f32(bits).copy()) / torch.tensor(scale, dtype=torch.float32)).numpy()
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ok = np.abs(y) <= 464
    assert np.array_equal(got[ok], ref[ok])
    assert np.all((got[~ok & ~np.isnan(y)] & 0x7F) == 0x7E)


def test_cache_write_fp8_matches_numpy_scatter_of_torch_codes():
    w = W.make_workload("tiny")
    ks, vs = w.fp8_scales
    kc = np.zeros(w.k_cache.shape, np.uint8)
    vc = np.zeros(w.v_cache.shape, np.uint8)
    oracle.cache_write(w.new_k, w.new_v, w.slot_mapping, kc, vc, kv_dtype=oracle.KV_FP8_E4M3FN,
                       k_scale=ks, v_scale=vs)

    def codes(bits, s):
        y = torch.from_numpy(bf16_f32(bits).copy()) / torch.tensor(s, dtype=torch.float32)
        return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    ek = np.zeros_like(kc)
    ev = np.zeros_like(vc)
    ek.reshape(-1, 2, 64)[w.slot_mapping] = codes(w.new_k, ks)
    ev.reshape(-1, 2, 64)[w.slot_mapping] = codes(w.new_v, vs)
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)


def test_fp8_decode_equals_bf16_decode_on_dequantised_values():
    """Consistency pin: decoding fp8 codes with scales equals decoding a bf16
    cache holding code*scale when that product is exact in bf16 (scale 1, 2^-3)."""
    w = W.make_workload("tiny")
    for s in (1.0, 0.125):
        kq = oracle.quantize_pool(w.k_cache, s)
        vq = oracle.quantize_pool(w.v_cache, s)
        fp8 = oracle.decode_workload(w, kv_dtype=oracle.KV_FP8_E4M3FN, k_cache=kq, v_cache=vq,
                                     k_scale=s, v_scale=s)
        kb = _bits(oracle.e4m3fn_to_f64(kq) * s)
        vb = _bits(oracle.e4m3fn_to_f64(vq) * s)
        assert np.array_equal(bf16_f32(kb)[np.isfinite(bf16_f32(kb))],
                              (oracle.e4m3fn_to_f64(kq) * s)[np.isfinite(bf16_f32(kb))].astype(np.float32))
        ref = oracle.decode_workload(w, k_cache=kb, v_cache=vb)
        np.testing.assert_allclose(fp8, ref, rtol=0, atol=1e-13)
