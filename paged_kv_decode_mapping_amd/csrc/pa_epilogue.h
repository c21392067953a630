// pa_epilogue.h -- the part of a decode workgroup after its tile loop:
// combine the per-wave online-softmax states and store either the final
// bf16 output or a split-K partial.
//
// A state over a token subset T is (m, l, o) with m = max_{j in T} x_j (x =
// score in log2 units), l = sum 2^(x_j - m), o = sum 2^(x_j - m) V_j. Two
// states combine exactly: M = max(m1, m2), l = l1 2^(m1-M) + l2 2^(m2-M),
// o = o1 2^(m1-M) + o2 2^(m2-M); the output is o / l. This is the
// softmax of Tutorial «大模型推理优化与加速完全教程» §4.4 evaluated in pieces
// (the tiling idea TGI «TGI技术解析» §5.2 credits to Flash Attention).
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Scale factor 2^(m_w - M) of a state with max m_w inside a combination with
// max M; an empty state (m_w = -inf) contributes nothing.
__device__ __forceinline__ float state_weight(float m_w, float M) {
    return (m_w == -INFINITY) ? 0.0f : fast_exp2(m_w - M);
}

// A workgroup's unit covers G consecutive query heads: unit * G .. unit * G
// + G - 1 (G = g with one KV head per unit, HP * g with HP of them).
// sm_ml: [W][G][2] (m, l); sm_o: [W][G][D]. Called by all threads of the
// workgroup after a barrier that follows the writes into LDS.
template <int D>
__device__ __forceinline__ void combine_and_store(const DecodeArgs& a, const float* sm_ml,
                                                  const float* sm_o, int W, int G, int seq, int unit,
                                                  int part, bool final_out) {
    const int g = G;
    const int kvh = unit;
    for (int idx = (int)threadIdx.x; idx < g * D; idx += (int)blockDim.x) {
        const int h = idx / D;
        const int d = idx - h * D;
        float M = -INFINITY;
        for (int w = 0; w < W; ++w) M = fmaxf(M, sm_ml[(w * g + h) * 2]);
        float L = 0.0f, O = 0.0f;
        if (M != -INFINITY) {
            for (int w = 0; w < W; ++w) {
                const float f = state_weight(sm_ml[(w * g + h) * 2], M);
                L += sm_ml[(w * g + h) * 2 + 1] * f;
                O += sm_o[(w * g + h) * D + d] * f;
            }
        }
        const int hq = kvh * g + h;
        const int64_t row = (int64_t)seq * a.num_q_heads + hq;
        if (final_out) {
            const float y = (L > 0.0f) ? (O * a.v_scale) / L : 0.0f;
            a.out[(int64_t)seq * a.out_seq + (int64_t)hq * a.out_head + d] = f32_to_bf16_rne(y);
        } else {
            const int64_t prow = row * a.num_partitions + part;
            a.part_o[prow * D + d] = O * a.v_scale;
            if (d == 0) {
                a.part_ml[prow * 2] = M;
                a.part_ml[prow * 2 + 1] = L;
            }
        }
    }
}

// Which tokens a decode workgroup owns and what it must store.
struct WorkItem {
    int seq, kvh, part;
    int t_begin, t_end;   // token range [t_begin, t_end) of the sequence
    bool final_out;       // store the bf16 output (else a partial)
    bool active;          // false: nothing to do (empty partition)
};

// Item `item` of (seq, unit): partitions item * wave_partitions onward,
// tokens [item * span, (item + 1) * span) clipped to the context, span =
// wave_partitions * partition_tokens.
__device__ __forceinline__ WorkItem make_work_item(const DecodeArgs& a, int seq, int kvh, int item) {
    WorkItem w;
    w.seq = seq;
    w.kvh = kvh;
    w.part = item;
    int ctx = a.context_lens[seq];
    const int cap = a.max_blocks_per_seq << a.block_size_log2;
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int span = a.partition_tokens * a.wave_partitions;
    const int items_used = (ctx + span - 1) / span;
    const int parts_used = (ctx + a.partition_tokens - 1) / a.partition_tokens;
    w.t_begin = item * span;
    w.t_end = min(w.t_begin + span, ctx);
    // Item 0 always runs, so that a zero-length context still gets its
    // (all-zero) output row.
    w.active = (item < items_used) || (item == 0);
    w.final_out = (a.num_partitions == 1) || (parts_used <= 1);
    return w;
}

// Direct grid: workgroup b takes item b % num_items of unit b / num_items
// (a sequence has units_per_seq units: its KV heads, or groups of them).
// Consecutive workgroups are dispatched round robin over the XCDs, so the
// items of one unit spread over all of them. (Item-major order, later items
// first, was measured slower: with few sequences the early items then all
// belong to the longest one, whose units map to the same few XCDs.)
__device__ __forceinline__ WorkItem decode_work_item(const DecodeArgs& a) {
    const int bid = (int)blockIdx.x;
    const int unit = bid / a.num_items;
    return make_work_item(a, unit / a.units_per_seq, unit % a.units_per_seq, bid % a.num_items);
}

__device__ __forceinline__ WorkItem scheduled_item(const int4& r) {
    WorkItem w;
    w.seq = r.x;
    w.kvh = r.y & 0xffff;
    w.part = r.y >> 16;
    w.t_begin = r.z;
    w.t_end = r.w & ~kItemFinal;
    w.final_out = (r.w & kItemFinal) != 0;
    w.active = true;
    return w;
}

// Exclusive prefix sum over the workgroup of one value per thread (in
// thread order); *total gets the sum. wsum: LDS scratch of >= 16 ints.
// Contains barriers: every thread of the workgroup must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
    const int t = (int)threadIdx.x, lane = t & 63, wave = t >> 6, nw = (int)(blockDim.x >> 6);
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < nw; ++w) {
        const int s = wsum[w];
        base += w < wave ? s : 0;
        tot += s;
    }
    __syncthreads();  // wsum is free again
    *total = tot;
    return base + x - v;
}

// Exclusive prefix sum over one wave (lane order); *total gets the sum.
__device__ __forceinline__ int wave_exclusive_scan(int v, int* total) {
    const int lane = (int)(threadIdx.x & 63);
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    *total = __builtin_amdgcn_readlane(x, 63);
    return x - v;
}

// Rank `b` among the items of a batch of at most kSelfWaveSeqs sequences,
// expanded over `units` units each, in longest-first order: the first wave
// alone does it (lane l holds sequences kSelfSeqsPerLane * l onward in
// registers, so context_lens is read once and the scans are wave-wide
// shuffles), and one barrier hands the result to the other waves. Items
// are `span` tokens of a sequence (a multiple of the tile), the last one
// shorter, a zero-length context one empty item; lengths are clamped to
// [0, cap]. The grid is sized for the most items there can be, so most
// workgroups of a ragged or short batch have none: those learn it from the
// item total alone, one wave-wide sum after the read, and exit before any
// of the ranking. Same order and result as the workgroup-wide search
// below. Returns false (uniformly) past the last item, else the item's
// sequence, its index within the sequence and the unit. lds: kSelfLdsInts
// ints of scratch, reusable by the caller once this returns. Contains
// barriers: every thread of the workgroup must call it.
__device__ __forceinline__ bool rank_item_wave(const int32_t* context_lens, int S, int span, int cap, int units,
                                               int b, int* lds, int* seq_out, int* part_out, int* unit_out) {
    const int t = (int)threadIdx.x, lane = t & 63;
    const int KT = span / kTile;  // tiles of a full item
    const int NB = KT + 1;        // buckets: k = KT - tiles, k = 0 holds full items
    int* hist = lds;  // [NB <= kSelfBuckets]
    int* res = lds + kSelfRes;
    const int pb = b / units, unit = b - pb * units;
    if (t < 64) {
        int full[kSelfSeqsPerLane], last[kSelfSeqsPerLane];  // full items; bucket of the last (-1: none)
        int fsum = 0, items = 0;
#pragma unroll
        for (int k = 0; k < kSelfSeqsPerLane; ++k) {
            const int i = kSelfSeqsPerLane * lane + k;
            full[k] = 0;
            last[k] = -1;
            if (i < S) {
                int ctx = context_lens[i];
                ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
                const int f = ctx / span, rem = ctx - f * span;
                full[k] = f;
                if (rem > 0 || ctx == 0) last[k] = KT - (rem + kTile - 1) / kTile;
            }
            fsum += full[k];
            items += full[k] + (last[k] >= 0 ? 1 : 0);
        }
        int total;
        (void)wave_exclusive_scan(items, &total);
        int seq = -1, part = 0;
        if (pb < total) {
            for (int k = lane; k < NB; k += 64) hist[k] = 0;
            int ftot;
            (void)wave_exclusive_scan(fsum, &ftot);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            if (lane == 0) atomicAdd(&hist[0], ftot);
#pragma unroll
            for (int k = 0; k < kSelfSeqsPerLane; ++k)
                if (last[k] >= 0) atomicAdd(&hist[last[k]], 1);
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            __builtin_amdgcn_wave_barrier();
            // buckets [k0, k1) of this lane, then their scan
            const int CB = (NB + 63) / 64;
            const int k0 = min(lane * CB, NB), k1 = min(k0 + CB, NB);
            int local = 0;
            for (int k = k0; k < k1; ++k) local += hist[k];
            int total_b;
            const int run = wave_exclusive_scan(local, &total_b);
            const bool mine = pb >= run && pb < run + local;
            const uint64_t hold = __builtin_amdgcn_ballot_w64(mine);
            // exactly one lane holds item pb's bucket (none only if the counts were inconsistent)
            const int src = hold != 0 ? (int)__builtin_ctzll(hold) : 0;
            int kb_l = -1, r_l = 0;
            if (mine) {
                int acc = run;
                for (int k = k0; k < k1; ++k) {
                    const int h = hist[k];
                    if (kb_l < 0 && pb < acc + h) {
                        kb_l = k;
                        r_l = pb - acc;
                    }
                    acc += h;
                }
            }
            const int kb = __builtin_amdgcn_readlane(kb_l, src), r = __builtin_amdgcn_readlane(r_l, src);
            // the r-th item of bucket kb in sequence order
            int cnt = 0;
#pragma unroll
            for (int k = 0; k < kSelfSeqsPerLane; ++k) cnt += (kb == 0 ? full[k] : 0) + (last[k] == kb ? 1 : 0);
            int tot2;
            const int pre = wave_exclusive_scan(cnt, &tot2);
            const bool mine2 = kb >= 0 && r >= pre && r < pre + cnt;
            const uint64_t hold2 = __builtin_amdgcn_ballot_w64(mine2);
            if (hold2 != 0) {
                const int src2 = (int)__builtin_ctzll(hold2);
                int seq_l = -1, part_l = 0;
                if (mine2) {
                    int acc = pre;
#pragma unroll
                    for (int k = 0; k < kSelfSeqsPerLane; ++k) {
                        const int c = (kb == 0 ? full[k] : 0) + (last[k] == kb ? 1 : 0);
                        if (seq_l < 0 && r < acc + c) {
                            const int j = r - acc;
                            seq_l = kSelfSeqsPerLane * lane + k;
                            part_l = (kb == 0 && j < full[k]) ? j : full[k];
                        }
                        acc += c;
                    }
                }
                seq = __builtin_amdgcn_readlane(seq_l, src2);
                part = __builtin_amdgcn_readlane(part_l, src2);
            }
        }
        if (lane == 0) {
            res[0] = seq;
            res[1] = part;
        }
    }
    __syncthreads();
    const int seq = res[0], part = res[1];
    __syncthreads();  // every thread has read res before the caller may reuse the LDS
    if (seq < 0 || seq >= S) return false;
    *seq_out = seq;
    *part_out = part;
    *unit_out = unit;
    return true;
}

// The decode kernels' self-scheduled item for batches of at most
// kSelfWaveSeqs sequences (see rank_item_wave).
__device__ __forceinline__ bool self_scheduled_item_wave(const DecodeArgs& a, int* lds, WorkItem* out) {
    int seq, part, unit;
    if (!rank_item_wave(a.context_lens, a.num_seqs, a.partition_tokens * a.wave_partitions,
                        a.max_blocks_per_seq << a.block_size_log2, a.units_per_seq, (int)blockIdx.x, lds, &seq,
                        &part, &unit))
        return false;
    *out = make_work_item(a, seq, unit, part);
    return true;
}

// Self-scheduled item of this workgroup: the (blockIdx / U)-th item, in
// longest-first order, of all (sequence, partition) items expanded over the
// U units of a sequence -- the order the work-list builder writes, found by
// each workgroup from context_lens without a pre-pass. Items are of `span`
// tokens except each sequence's last (a zero-length context has one empty
// item). Longest first means: by tile count, longest bucket first, and
// within a bucket in (sequence, partition) order. All full items share the
// first bucket; each sequence adds at most one shorter item. Returns false
// (uniformly) when the block index is past the last item. lds: kSelfLdsInts
// ints of scratch; contains barriers: every thread must call it.
__device__ __forceinline__ bool self_scheduled_item(const DecodeArgs& a, int* lds, WorkItem* out) {
    const int T = (int)blockDim.x, t = (int)threadIdx.x;
    const int S = a.num_seqs;
    const int span = a.partition_tokens * a.wave_partitions;
    const int KT = span / kTile;  // tiles of a full item (span is a multiple of the tile)
    const int NB = KT + 1;        // buckets: k = KT - tiles, k = 0 holds full items
    const int cap = a.max_blocks_per_seq << a.block_size_log2;
    int* hist = lds;               // [NB <= kSelfBuckets]
    int* wsum = lds + kSelfBuckets;
    int* res = wsum + 16;          // [4]: bucket, rank in it, then sequence, item
    // thread t owns sequences [i0, i1) (contiguous, so prefix sums follow sequence order)
    const int C = (S + T - 1) / T;
    const int i0 = min(t * C, S), i1 = min(i0 + C, S);
    for (int k = t; k < NB; k += T) hist[k] = 0;
    if (t == 0) res[2] = -1;  // no sequence found: skip rather than read out of bounds
    __syncthreads();
    int full = 0;
    for (int i = i0; i < i1; ++i) {
        int ctx = a.context_lens[i];
        ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
        const int f = ctx / span, rem = ctx - f * span;
        full += f;
        if (rem > 0 || ctx == 0) atomicAdd(&hist[KT - (rem + kTile - 1) / kTile], 1);
    }
    if (full > 0) atomicAdd(&hist[0], full);
    __syncthreads();
    // prefix over the buckets: thread t owns buckets [k0, k1)
    const int CB = (NB + T - 1) / T;
    const int k0 = min(t * CB, NB), k1 = min(k0 + CB, NB);
    int local = 0;
    for (int k = k0; k < k1; ++k) local += hist[k];
    int total = 0;
    const int run = block_exclusive_scan(local, wsum, &total);
    const int b = (int)blockIdx.x;
    const int pb = b / a.units_per_seq, unit = b - pb * a.units_per_seq;
    if (pb >= total) return false;
    if (pb >= run && pb < run + local) {  // exactly one thread holds the bucket of item pb
        int acc = run;
        for (int k = k0; k < k1; ++k) {
            const int h = hist[k];
            if (pb < acc + h) {
                res[0] = k;
                res[1] = pb - acc;
                break;
            }
            acc += h;
        }
    }
    __syncthreads();
    const int kb = res[0], r = res[1];
    // the r-th item of bucket kb in sequence order
    auto count_in_bucket = [&](int ctx, int* part_of_last) -> int {
        const int f = ctx / span, rem = ctx - f * span;
        const bool partial = rem > 0 || ctx == 0;
        *part_of_last = f;
        return (kb == 0 ? f : 0) + ((partial && KT - (rem + kTile - 1) / kTile == kb) ? 1 : 0);
    };
    int cnt = 0;
    for (int i = i0; i < i1; ++i) {
        int ctx = a.context_lens[i];
        ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
        int pl;
        cnt += count_in_bucket(ctx, &pl);
    }
    int tot2 = 0;
    const int pre = block_exclusive_scan(cnt, wsum, &tot2);
    if (r >= pre && r < pre + cnt) {
        int acc = pre;
        for (int i = i0; i < i1; ++i) {
            int ctx = a.context_lens[i];
            ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
            int f;
            const int c = count_in_bucket(ctx, &f);
            if (r < acc + c) {
                const int j = r - acc;  // the j-th item of this sequence in bucket kb
                res[2] = i;
                res[3] = (kb == 0 && j < f) ? j : f;  // a full item, or the sequence's last one
                break;
            }
            acc += c;
        }
    }
    __syncthreads();
    const int seq = res[2], part = res[3];
    __syncthreads();  // every thread has read res before the body may reuse the LDS
    if (seq < 0 || seq >= S) return false;
    *out = make_work_item(a, seq, unit, part);
    return true;
}

// Runs `body(item)` for this workgroup's work item: with no schedule, the
// (sequence, KV head, partition) its block index names; self-scheduled, the
// item of the longest-first order it finds itself; with a schedule, the
// block index's entry of the device-built list. The list (and the
// self-scheduled order) is compact and longest first, so workgroups are
// dispatched in that order and those past its end (the grid is sized for
// the most items there can be) exit at once, after every real item has
// been dispatched. `body` must be called by the whole workgroup. lds: the
// kernel's LDS, kSelfLdsInts ints of which serve as scratch before `body`.
template <class Body>
__device__ __forceinline__ void for_each_item(const DecodeArgs& a, int* lds, Body&& body) {
    if (a.items == nullptr) {
        if (a.self_schedule) {
            WorkItem wi;
            const bool found = a.num_seqs <= kSelfWaveSeqs ? self_scheduled_item_wave(a, lds, &wi)
                                                            : self_scheduled_item(a, lds, &wi);
            if (found) body(wi);
            return;
        }
        const WorkItem wi = decode_work_item(a);
        if (wi.active) body(wi);
        return;
    }
    const int b = (int)blockIdx.x;
    const int count = *a.item_count;
    const int4 rec = a.items[b];  // in bounds: the list has room for the whole grid
    if (b >= count) return;
    body(scheduled_item(rec));
}

// Block-table reads for a wave's sequence of tiles, one tile ahead. The
// entry of the next tile a wave will issue is fetched with a vector (buffer)
// load while the current tile's loads go out. Vector loads complete in issue
// order, so when the entry is needed one step later the wait for it only
// covers loads issued before the tile in flight; a scalar load would share
// its counter with the LDS traffic of the tile being consumed, and since
// scalar loads may complete out of order the compiler has to wait for all of
// it before the next issue.
struct TableReader {
    __amdgpu_buffer_rsrc_t rsrc;  // this sequence's table row
    int t_begin;                  // first token of the item
    int last_tile;                // entries past the item's last tile read its entry
    int tile_tokens;              // tokens per tile (a divisor of the block size)
    int block_size_log2;
    int last_block;
};

__device__ __forceinline__ TableReader make_table_reader(const int32_t* block_tables, int64_t table_stride,
                                                         int max_blocks_per_seq, int block_size_log2, int last_block,
                                                         int seq, int t_begin, int last_tile, int tile_tokens = kTile) {
    TableReader r;
    r.rsrc = make_rsrc(block_tables + (int64_t)seq * table_stride, (uint32_t)max_blocks_per_seq * 4u);
    r.t_begin = t_begin;
    r.last_tile = last_tile;
    r.tile_tokens = tile_tokens;
    r.block_size_log2 = block_size_log2;
    r.last_block = last_block;
    return r;
}

__device__ __forceinline__ TableReader make_table_reader(const DecodeArgs& a, const WorkItem& wi, int last_tile,
                                                         int tile_tokens = kTile) {
    return make_table_reader(a.block_tables, a.table_stride, a.max_blocks_per_seq, a.block_size_log2, a.last_block,
                             wi.seq, wi.t_begin, last_tile, tile_tokens);
}

// Start fetching the table entry of tile t (an index within the item).
__device__ __forceinline__ uint32_t table_fetch(const TableReader& r, int t) {
    const int tok = r.t_begin + min(t, r.last_tile) * r.tile_tokens;
    return __builtin_amdgcn_raw_buffer_load_b32(r.rsrc, (uint32_t)(tok >> r.block_size_log2) << 2, 0, 0);
}

// The physical block of a fetched entry, clamped into the pool so that a bad
// table entry cannot address memory outside it. The clamp is 32-bit (table
// entries are int32) so it stays in scalar registers.
__device__ __forceinline__ int64_t table_block(const TableReader& r, uint32_t entry) {
    int b = __builtin_amdgcn_readfirstlane((int)entry);
    b = b < 0 ? 0 : b;
    b = b > r.last_block ? r.last_block : b;
    return (int64_t)b;
}

}  // namespace pa
