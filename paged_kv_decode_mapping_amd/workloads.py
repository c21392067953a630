"""Seeded synthetic workloads for paged decode attention.

This module builds inputs only. It holds none of the attention, softmax,
quantisation or cache-write arithmetic: it draws values, lays out a physical
block pool and hands out block tables and slot ids, the state a serving
engine would hold when a decode step starts.

Pages cited (titles as printed at the top of each page):
  Tutorial = «大模型推理优化与加速完全教程» (LLM inference optimisation tutorial)
  TGI      = «TGI技术解析：大规模语言模型高效推理实践»

What the layout follows:
  * Physical pool per layer and per K/V: [num_blocks, block_size, num_kv_heads,
    head_dim], i.e. Tutorial §4.2 "PagedAttention", PagedKVCache.__init__
    block_pool with the layer and K/V axes dropped (one call per layer).
  * A sequence's logical block b lives in physical block block_tables[i][b];
    token j of the sequence is row j mod block_size of logical block
    j div block_size (Tutorial §4.2, append_token / get_kv).
  * A slot id is physical_block * block_size + row: the flat row index in
    the pool that append_token writes.
  * Model shapes: Tutorial §4.1 "KV Cache基础", analyze_kv_cache_memory
    (7B: 32 heads, head_dim 128, 32 KV heads; 70B: 64 heads, head_dim 128,
    8 KV heads).
  * Shared prefix blocks: Tutorial §4.3 "Prefix Caching" (requests sharing
    a system prompt point their tables at the same physical blocks).

Recipe (one numpy PCG64 stream per workload, draws in a fixed order):
  context lengths -> block permutation -> choice of prefix-sharing
  sequences -> q -> K/V of the shared prefix -> K/V of each sequence's own
  blocks -> new tokens' K/V -> slot ids of the new tokens.
Values are float32 N(0,1) rounded to bfloat16 (round to nearest even, by
torch on the CPU). Every row of the pool that no context token refers to is
filled with a quiet NaN, as is one dedicated "poison" block that pads every
block-table row past the sequence's last block, so any read past a context
shows up in the output.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    """Shape and recipe of one synthetic decode step."""

    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    # ("list", [ctx...]) | ("uniform", lo, hi) | ("const", n)
    # | ("lognormal", median, sigma, lo, hi)
    context: tuple
    # ("fixed", num_blocks) | ("factor", f): pool = ceil(f * blocks in use)
    pool: tuple = ("factor", 1.25)
    k_mult: float = 1.0
    shared_prefix_tokens: int = 0  # shared by shared_fraction of the sequences
    shared_fraction: float = 0.5
    seed: int = 1000
    partition_tokens: int = 0  # split-K partition the workload names (0 = none)
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# The five workloads, in order: tiny parity case, LLaMA-7B-shaped MHA layer,
# 70B-shaped GQA layer, long-context split-K batch, mixed continuous batch.
SPECS: Dict[str, WorkloadSpec] = {
    "tiny": WorkloadSpec(
        name="tiny", num_seqs=4, num_q_heads=8, num_kv_heads=2, head_dim=64,
        block_size=16, context=("list", [1, 17, 64, 100]), pool=("fixed", 32),
        seed=1000,
        description="4 seqs, ctx {1,17,64,100}, 8/2 heads, D 64, bs 16, pool 32 blocks"),
    "llama7b_mha": WorkloadSpec(
        name="llama7b_mha", num_seqs=64, num_q_heads=32, num_kv_heads=32,
        head_dim=128, block_size=16, context=("uniform", 512, 2048), seed=1001,
        description="batch 64, 32/32 heads, D 128, bs 16, ctx U[512,2048]"),
    "llama70b_gqa": WorkloadSpec(
        name="llama70b_gqa", num_seqs=128, num_q_heads=64, num_kv_heads=8,
        head_dim=128, block_size=16, context=("const", 4096), seed=1002,
        description="batch 128, 64/8 heads, D 128, bs 16, ctx 4096"),
    "long_splitk": WorkloadSpec(
        name="long_splitk", num_seqs=4, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block_size=128,
        context=("list", [32768, 65536, 98304, 131072]), k_mult=3.0, seed=1003,
        partition_tokens=512,
        description="4 seqs, ctx 32k..128k, 32/8 heads, D 128, bs 128, K x3, "
                    "512-token partitions"),
    "mixed_batch": WorkloadSpec(
        name="mixed_batch", num_seqs=256, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block_size=16, context=("lognormal", 1000.0, 1.0, 16, 8192),
        shared_prefix_tokens=512, seed=1004,
        description="256 seqs, ctx lognormal(median 1000, sigma 1) in [16,8192], "
                    "32/8 heads, D 128, bs 16, half share a 512-token prefix"),
}
ORDER: List[str] = ["tiny", "llama7b_mha", "llama70b_gqa", "long_splitk", "mixed_batch"]

# The MQA extreme of the 70B layer (Tutorial §4.4: one KV head for all query
# heads), for the wide-group route of pa_decode (g = 64).
SPECS["mqa_70b"] = WorkloadSpec(
    name="mqa_70b", num_seqs=128, num_q_heads=64, num_kv_heads=1, head_dim=128, block_size=16,
    context=("const", 4096), seed=1006,
    description="batch 128, 64/1 heads (MQA), D 128, bs 16, ctx 4096")

# A batch for the shared-prefix (cascade) decode beyond the five above: every
# request starts with the same long system prompt (Tutorial §4.3 names the
# shared system prompt as prefix caching's case), on the 70B layer shape.
SPECS["system_prompt"] = WorkloadSpec(
    name="system_prompt", num_seqs=128, num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
    context=("uniform", 4096 + 16, 4096 + 512), shared_prefix_tokens=4096, shared_fraction=1.0, seed=1005,
    description="128 seqs, 64/8 heads, D 128, bs 16, all share a 4096-token system prompt, "
                "own tokens U[16,512] after it")


@dataclasses.dataclass
class Workload:
    """One generated decode step. Arrays are host numpy; bf16 is stored as uint16 bits."""

    spec: WorkloadSpec
    context_lens: np.ndarray      # int32 [S]
    block_tables: np.ndarray      # int32 [S, max_blocks_per_seq]
    num_blocks: int               # N, physical blocks in the pool
    poison_block: int             # pool block full of NaN, pads every table row
    q: np.ndarray                 # uint16 [S, Hq, D]
    k_cache: np.ndarray           # uint16 [N, bs, Hkv, D]
    v_cache: np.ndarray           # uint16 [N, bs, Hkv, D]
    new_k: np.ndarray             # uint16 [T, Hkv, D]
    new_v: np.ndarray             # uint16 [T, Hkv, D]
    slot_mapping: np.ndarray      # int64 [T]
    k_amax: float                 # max |K| over context and new tokens
    v_amax: float
    shared_seqs: np.ndarray       # int64 indices of prefix-sharing sequences
    unique_blocks: int            # physical blocks holding context data
    prefix_ids: np.ndarray = dataclasses.field(  # int64 physical blocks of the shared prefix
        default_factory=lambda: np.zeros(0, np.int64))

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def scale(self) -> float:
        return self.spec.scale

    @property
    def fp8_scales(self):
        """Per-tensor fp8 scales, amax/448 computed in float32 (448 = largest e4m3fn value)."""
        k = np.float32(self.k_amax) / np.float32(448.0)
        v = np.float32(self.v_amax) / np.float32(448.0)
        return float(k), float(v)


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (the 16 bits become the high half)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _context_lens(spec: WorkloadSpec, rng: np.random.Generator, num_seqs: int) -> np.ndarray:
    kind = spec.context[0]
    if kind == "list":
        vals = list(spec.context[1])
        if len(vals) != num_seqs:
            raise ValueError(f"{spec.name}: {len(vals)} context lengths for {num_seqs} seqs")
        return np.asarray(vals, dtype=np.int64)
    if kind == "const":
        return np.full(num_seqs, int(spec.context[1]), dtype=np.int64)
    if kind == "uniform":
        lo, hi = spec.context[1], spec.context[2]
        return rng.integers(lo, hi + 1, size=num_seqs, dtype=np.int64)
    if kind == "lognormal":
        median, sigma, lo, hi = spec.context[1:]
        x = np.exp(rng.normal(math.log(median), sigma, size=num_seqs))
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    raise ValueError(kind)


def make_workload(name_or_spec, *, seed: Optional[int] = None, num_seqs: Optional[int] = None,
                  context: Optional[tuple] = None, num_new_tokens: Optional[int] = None,
                  poison: bool = True, **spec_overrides) -> Workload:
    """Generate one workload.

    `num_seqs`, `context` and other spec fields may be overridden to get
    smaller cases with the same structure (head counts, block size, value
    distribution, sharing and pool rules). The number of new tokens written
    by the step defaults to one per sequence.
    """
    spec = SPECS[name_or_spec] if isinstance(name_or_spec, str) else name_or_spec
    upd = dict(spec_overrides)
    if context is not None:
        upd["context"] = context
    if num_seqs is not None:
        upd["num_seqs"] = num_seqs
    if seed is not None:
        upd["seed"] = seed
    if upd:
        spec = dataclasses.replace(spec, **upd)
    S, Hq, Hkv, D, bs = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.block_size
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    rng = np.random.default_rng(spec.seed)

    ctx = _context_lens(spec, rng, S)
    nblk = (ctx + bs - 1) // bs

    # Which sequences share the prefix (drawn even when unused keeps the stream fixed).
    prefix_blocks = spec.shared_prefix_tokens // bs
    if spec.shared_prefix_tokens % bs:
        raise ValueError("shared prefix must be a whole number of blocks")
    n_shared = int(S * spec.shared_fraction)
    shared = np.sort(rng.choice(S, n_shared, replace=False)) if prefix_blocks else np.zeros(0, np.int64)
    is_shared = np.zeros(S, dtype=bool)
    is_shared[shared] = True
    own = np.where(is_shared, np.maximum(nblk - prefix_blocks, 0), nblk)
    unique = int(own.sum()) + (prefix_blocks if len(shared) else 0)

    T = S if num_new_tokens is None else int(num_new_tokens)
    if spec.pool[0] == "fixed":
        N = int(spec.pool[1])
    else:
        N = int(math.ceil(spec.pool[1] * unique))
    # room for the poison block and for the new tokens in fully free blocks
    need = unique + 1 + (T + bs - 1) // bs
    if N < need:
        N = need
    perm = rng.permutation(N).astype(np.int64)
    cursor = 0
    prefix_ids = perm[cursor:cursor + (prefix_blocks if len(shared) else 0)]
    cursor += len(prefix_ids)
    own_ids: List[np.ndarray] = []
    for i in range(S):
        own_ids.append(perm[cursor:cursor + own[i]])
        cursor += int(own[i])
    poison_block = int(perm[cursor])
    cursor += 1
    free_ids = perm[cursor:]

    MB = max(1, int(nblk.max()) if S else 1)
    tables = np.full((S, MB), poison_block, dtype=np.int64)
    for i in range(S):
        if is_shared[i]:
            np_ = min(int(nblk[i]), prefix_blocks)
            tables[i, :np_] = prefix_ids[:np_]
            tables[i, np_:nblk[i]] = own_ids[i]
        else:
            tables[i, :nblk[i]] = own_ids[i]

    fill = BF16_QNAN if poison else np.uint16(0)
    k_cache = np.full((N, bs, Hkv, D), fill, dtype=np.uint16)
    v_cache = np.full((N, bs, Hkv, D), fill, dtype=np.uint16)

    q = _to_bf16_bits(rng.standard_normal((S, Hq, D), dtype=np.float32))
    kmax = 0.0
    vmax = 0.0

    def draw(n_blocks: int, mult: float):
        x = rng.standard_normal((n_blocks, bs, Hkv, D), dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        return _to_bf16_bits(x)

    def amax_rows(bits: np.ndarray, rows: int) -> float:
        flat = bits.reshape(-1, Hkv, D)[:rows]
        if flat.size == 0:
            return 0.0
        return float(np.abs(bf16_bits_to_f32(flat)).max())

    if len(prefix_ids):
        kb = draw(len(prefix_ids), spec.k_mult)
        vb = draw(len(prefix_ids), 1.0)
        k_cache[prefix_ids] = kb
        v_cache[prefix_ids] = vb
        # amax covers the prefix rows some sequence actually uses
        used = int(min(spec.shared_prefix_tokens, ctx[is_shared].max()))
        kmax = max(kmax, amax_rows(kb, used))
        vmax = max(vmax, amax_rows(vb, used))
    for i in range(S):
        ids = own_ids[i]
        if len(ids) == 0:
            continue
        start_tok = prefix_blocks * bs if is_shared[i] else 0
        valid = int(ctx[i]) - start_tok  # rows of this sequence's own blocks holding context
        kb = draw(len(ids), spec.k_mult)
        vb = draw(len(ids), 1.0)
        kflat = kb.reshape(-1, Hkv, D)
        vflat = vb.reshape(-1, Hkv, D)
        kflat[valid:] = fill
        vflat[valid:] = fill
        kmax = max(kmax, amax_rows(kb, valid))
        vmax = max(vmax, amax_rows(vb, valid))
        k_cache[ids] = kb
        v_cache[ids] = vb

    new_k = _to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32) * np.float32(spec.k_mult))
    new_v = _to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32))
    if T:
        kmax = max(kmax, float(np.abs(bf16_bits_to_f32(new_k)).max()))
        vmax = max(vmax, float(np.abs(bf16_bits_to_f32(new_v)).max()))
    free_slots = (free_ids[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)
    if T > len(free_slots):
        raise ValueError("pool too small for the new tokens")
    slot_mapping = np.sort(rng.choice(free_slots, T, replace=False)) if T else np.zeros(0, np.int64)
    # a serving engine hands slots in token order, not sorted; shuffle with the same stream
    if T:
        slot_mapping = slot_mapping[rng.permutation(T)]

    return Workload(
        spec=spec, context_lens=ctx.astype(np.int32), block_tables=tables.astype(np.int32),
        num_blocks=N, poison_block=poison_block, q=q, k_cache=k_cache, v_cache=v_cache,
        new_k=new_k, new_v=new_v, slot_mapping=slot_mapping.astype(np.int64),
        k_amax=kmax, v_amax=vmax, shared_seqs=shared.astype(np.int64), unique_blocks=unique,
        prefix_ids=prefix_ids.astype(np.int64))


def reduced(name: str, num_seqs: int, context: Sequence[int], **kw) -> Workload:
    """Same structure as a named workload at a size the oracle finishes in seconds."""
    return make_workload(name, num_seqs=num_seqs, context=("list", list(context)), **kw)


@dataclasses.dataclass
class MultiQuery:
    """Query tokens for multi-token paged attention over a generated workload:
    sequence i's last q_lens[i] cached tokens are its queries (draft tokens
    being verified, or a prefill chunk whose K/V are already written)."""

    q: np.ndarray             # uint16 [T_q, Hq, D] bf16 bits, sequence-major
    query_start: np.ndarray   # int32 [S + 1], query_start[i+1] - query_start[i] = q_lens[i]
    q_lens: np.ndarray        # int32 [S]

    @property
    def num_tokens(self) -> int:
        return int(self.query_start[-1])


def make_multi_query(w: Workload, q_lens, *, seed: Optional[int] = None) -> MultiQuery:
    """Draw N(0,1) bf16 query rows for q_lens[i] query tokens of each sequence of
    `w` (each at most that sequence's context length). Seeded, one stream."""
    q_lens = np.asarray(q_lens, dtype=np.int64)
    s = w.spec
    if q_lens.shape != (s.num_seqs,):
        raise ValueError("one query length per sequence")
    if np.any(q_lens < 0) or np.any(q_lens > w.context_lens):
        raise ValueError("query lengths must lie in [0, context length]")
    rng = np.random.default_rng(s.seed + 7919 if seed is None else seed)
    T = int(q_lens.sum())
    q = _to_bf16_bits(rng.standard_normal((T, s.num_q_heads, s.head_dim), dtype=np.float32))
    qs = np.zeros(s.num_seqs + 1, dtype=np.int64)
    qs[1:] = np.cumsum(q_lens)
    return MultiQuery(q=q, query_start=qs.astype(np.int32), q_lens=q_lens.astype(np.int32))


@dataclasses.dataclass
class CascadeBatch:
    """A decode batch laid out for a cascade call: prefix group k is the run
    of sequences group_start[k] .. group_start[k+1] - 1, whose first
    prefix_lens[k] tokens are the cached prefix held in the blocks of
    prefix_tables[k] (Tutorial §4.3, prefix caching: the cache keeps each
    prefix's block list and length). Members' own table rows name the same
    blocks for those tokens, as a prefix cache hands them out."""

    q: np.ndarray                 # uint16 [S, Hq, D]
    k_cache: np.ndarray           # uint16 [N, bs, Hkv, D]
    v_cache: np.ndarray
    block_tables: np.ndarray      # int32 [S, MB]
    context_lens: np.ndarray      # int32 [S]
    prefix_tables: np.ndarray     # int32 [G, PMB]
    prefix_lens: np.ndarray       # int32 [G]
    group_start: np.ndarray       # int32 [G + 1]
    max_group_size: int
    num_blocks: int
    poison_block: int
    block_size: int
    scale: float
    order: Optional[np.ndarray] = None  # batch position -> sequence of the source workload

    @property
    def num_groups(self) -> int:
        return int(self.prefix_lens.shape[0])


def cascade_batch(w: Workload) -> CascadeBatch:
    """The workload's batch reordered for a cascade call: the sequences that
    share its prefix first, as one group, then the others in their order.
    Arrays are permuted copies; `order` maps batch positions back."""
    s = w.spec
    shared = np.asarray(w.shared_seqs, dtype=np.int64)
    rest = np.setdiff1d(np.arange(s.num_seqs), shared)
    order = np.concatenate([shared, rest])
    n = len(shared)
    pb = len(w.prefix_ids)
    return CascadeBatch(
        q=np.ascontiguousarray(w.q[order]), k_cache=w.k_cache, v_cache=w.v_cache,
        block_tables=np.ascontiguousarray(w.block_tables[order]),
        context_lens=np.ascontiguousarray(w.context_lens[order]),
        prefix_tables=np.asarray(w.prefix_ids, dtype=np.int32).reshape(1 if n else 0, pb if n else 1)
        if n else np.zeros((0, 1), np.int32),
        prefix_lens=np.array([s.shared_prefix_tokens] if n else [], dtype=np.int32),
        group_start=np.array([0, n] if n else [0], dtype=np.int32),
        max_group_size=max(n, 1), num_blocks=w.num_blocks, poison_block=w.poison_block,
        block_size=s.block_size, scale=s.scale, order=order)


def make_prefix_groups(*, num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                       groups: Sequence[tuple], lead: Sequence[int] = (), tail: Sequence[int] = (),
                       seed: int = 2024, pool_factor: float = 1.25) -> CascadeBatch:
    """A batch of `lead` ungrouped sequences, then one run per entry
    (prefix_tokens, [member context lengths]) of `groups`, then `tail`
    ungrouped sequences (each list gives context lengths). prefix_tokens is
    a whole number of blocks; a member may be shorter than its prefix.
    Every member's table names its group's prefix blocks for the prefix
    tokens it holds and its own blocks after them. Values are N(0,1) bf16;
    free rows and the poison block padding every table row hold NaN."""
    bs = block_size
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    rng = np.random.default_rng(seed)
    ctx = [int(c) for c in lead]
    member_group: List[int] = [-1] * len(lead)
    starts = [len(lead)]
    for k, (ptok, members) in enumerate(groups):
        if ptok % bs:
            raise ValueError("prefix lengths are whole blocks")
        ctx += [int(c) for c in members]
        member_group += [k] * len(members)
        starts.append(len(ctx))
    ctx += [int(c) for c in tail]
    member_group += [-1] * len(tail)
    S = len(ctx)
    ctx_a = np.asarray(ctx, dtype=np.int64)
    nblk = (ctx_a + bs - 1) // bs
    pblocks = [ptok // bs for ptok, _ in groups]
    shared_blk = np.array([min(int(nblk[i]), pblocks[member_group[i]]) if member_group[i] >= 0 else 0
                           for i in range(S)], dtype=np.int64)
    own = nblk - shared_blk
    used = int(own.sum()) + sum(pblocks)
    N = max(int(math.ceil(pool_factor * used)), used + 1)
    perm = rng.permutation(N).astype(np.int64)
    cur = 0
    prefix_ids = []
    for pbk in pblocks:
        prefix_ids.append(perm[cur:cur + pbk])
        cur += pbk
    own_ids = []
    for i in range(S):
        own_ids.append(perm[cur:cur + own[i]])
        cur += int(own[i])
    poison = int(perm[cur])
    MB = max(1, int(nblk.max()) if S else 1)
    PMB = max([1] + pblocks)
    tables = np.full((S, MB), poison, dtype=np.int64)
    for i in range(S):
        sb = int(shared_blk[i])
        if sb:
            tables[i, :sb] = prefix_ids[member_group[i]][:sb]
        tables[i, sb:nblk[i]] = own_ids[i]
    ptables = np.full((len(groups), PMB), poison, dtype=np.int64)
    for k, ids in enumerate(prefix_ids):
        ptables[k, :len(ids)] = ids
    k_cache = np.full((N, bs, Hkv, D), BF16_QNAN, dtype=np.uint16)
    v_cache = np.full((N, bs, Hkv, D), BF16_QNAN, dtype=np.uint16)
    q = _to_bf16_bits(rng.standard_normal((S, Hq, D), dtype=np.float32))
    for ids in prefix_ids:
        if len(ids):
            k_cache[ids] = _to_bf16_bits(rng.standard_normal((len(ids), bs, Hkv, D), dtype=np.float32))
            v_cache[ids] = _to_bf16_bits(rng.standard_normal((len(ids), bs, Hkv, D), dtype=np.float32))
    for i in range(S):
        ids = own_ids[i]
        if len(ids) == 0:
            continue
        valid = int(ctx_a[i]) - int(shared_blk[i]) * bs
        kb = _to_bf16_bits(rng.standard_normal((len(ids), bs, Hkv, D), dtype=np.float32))
        vb = _to_bf16_bits(rng.standard_normal((len(ids), bs, Hkv, D), dtype=np.float32))
        kb.reshape(-1, Hkv, D)[valid:] = BF16_QNAN
        vb.reshape(-1, Hkv, D)[valid:] = BF16_QNAN
        k_cache[ids] = kb
        v_cache[ids] = vb
    sizes = np.diff(np.asarray(starts))
    return CascadeBatch(
        q=q, k_cache=k_cache, v_cache=v_cache, block_tables=tables.astype(np.int32),
        context_lens=ctx_a.astype(np.int32), prefix_tables=ptables.astype(np.int32).reshape(len(groups), PMB),
        prefix_lens=np.array([ptok for ptok, _ in groups], dtype=np.int32),
        group_start=np.asarray(starts, dtype=np.int32), max_group_size=int(max([1] + list(sizes))),
        num_blocks=N, poison_block=poison, block_size=bs, scale=1.0 / math.sqrt(D))
