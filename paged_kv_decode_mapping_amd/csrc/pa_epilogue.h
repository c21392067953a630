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

__device__ __forceinline__ WorkItem make_work_item(const DecodeArgs& a, int seq, int kvh, int part) {
    WorkItem w;
    w.seq = seq;
    w.kvh = kvh;
    w.part = part;
    int ctx = a.context_lens[seq];
    const int cap = a.max_blocks_per_seq << a.block_size_log2;
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int parts_used = (ctx + a.partition_tokens - 1) / a.partition_tokens;
    w.t_begin = part * a.partition_tokens;
    w.t_end = min(w.t_begin + a.partition_tokens, ctx);
    // Partition 0 always runs, so that a zero-length context still gets its
    // (all-zero) output row.
    w.active = (part < parts_used) || (part == 0);
    w.final_out = (a.num_partitions == 1) || (parts_used <= 1);
    return w;
}

// Direct grid: workgroup b takes item (unit = b / P, part = b % P); a
// sequence has units_per_seq units (its KV heads, or groups of them).
__device__ __forceinline__ WorkItem decode_work_item(const DecodeArgs& a) {
    const int bid = (int)blockIdx.x;
    const int P = a.num_partitions;
    const int unit = bid / P;
    return make_work_item(a, unit / a.units_per_seq, unit % a.units_per_seq, bid % P);
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

// Runs `body(item)` for this workgroup's work item: with no schedule, the
// (sequence, KV head, partition) its block index names; with a schedule, the
// block index's entry of the device-built list. That list is compact and
// longest first, so workgroups are dispatched in that order and those past
// its end (the grid is sized for the most items there can be) exit at once,
// after every real item has been dispatched. `body` must be called by the
// whole workgroup.
template <class Body>
__device__ __forceinline__ void for_each_item(const DecodeArgs& a, Body&& body) {
    if (a.items == nullptr) {
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
