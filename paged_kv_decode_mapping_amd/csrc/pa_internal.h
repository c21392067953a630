// pa_internal.h -- kernel argument blocks and launcher declarations inside
// libpa (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kTile = 16;  // tokens per decode tile (one MFMA M/N extent)

// Shared-prefix groups of a cascade call. Group k is the run of sequences
// group_start[k] .. group_start[k+1] - 1 (at most max_group_size of them);
// its members' first prefix_lens[k] tokens (whole blocks, at most
// max_prefix_tokens) sit in the blocks of prefix table row k.
struct CascadeGroups {
    const int32_t* group_start;    // [num_groups + 1]; null = no groups
    const int32_t* prefix_lens;    // [num_groups] tokens
    int32_t num_groups, max_group_size, max_prefix_tokens;
    int32_t max_context;           // members' table rows: max_blocks_per_seq * block_size
};

// Where a paged cache's rows are: element (block b, row r, KV head h, d)
// sits at byte b * block + r * token + h * head + d * element size from the
// cache's base (Tutorial §4.2's pool order [N, bs, Hkv, D] has token =
// Hkv * D * e and head = D * e; a head-major pool has token = D * e, head =
// bs * D * e). K and V share it.
struct CacheLayout {
    int64_t block;                 // bytes between physical blocks
    uint32_t token;                // bytes between rows of a block (>= D * e)
    uint32_t head;                 // bytes between KV heads of a row
};

// Arguments of the decode kernels, passed by value.
struct DecodeArgs {
    const uint16_t* q;             // [S, Hq, D] bf16, element strides q_seq, q_head
    const uint8_t* k_cache;        // [N, bs, Hkv, D] bf16 or e4m3fn, at `cache`
    const uint8_t* v_cache;
    const int32_t* block_tables;   // [S, MB], row stride table_stride
    const int32_t* context_lens;   // [S]
    uint16_t* out;                 // [S, Hq, D] bf16, element strides out_seq, out_head
    float* part_ml;                // [S, Hq, P, 2] (max in log2 units, sum), split only
    float* part_o;                 // [S, Hq, P, D] unnormalised outputs, split only
    int64_t q_seq, q_head, out_seq, out_head, table_stride;
    int32_t num_seqs, num_q_heads, num_kv_heads, group;
    int32_t units_per_seq;         // work units per sequence: KV heads / heads per unit
    int32_t block_size_log2, max_blocks_per_seq;
    int32_t partition_tokens, num_partitions;
    // Partitions per work item: 1, or the workgroup's W waves, each of which
    // then takes one whole partition of the item (and stores its state);
    // items per (sequence, unit) = ceil(num_partitions / wave_partitions).
    int32_t wave_partitions, num_items;
    int32_t last_block;            // min(num_blocks, 2^31) - 1: the largest usable block id
    CacheLayout cache;
    float qk_scale_log2;           // scale * k_scale * log2(e)
    float v_scale;                 // 1 for bf16
    // Device schedule (null = direct grid, one workgroup per item):
    const int4* items;             // see ScheduleArgs, longest first
    const int* item_count;         // number of valid items
    // Self-scheduled (items null): workgroup b finds the b-th item of the
    // longest-first order itself from context_lens (see pa_epilogue.h).
    int32_t self_schedule;
};

// Self-scheduling: items (one per (sequence, unit) partition, or group of
// partitions) are counted in buckets by tile count; full items all fall in
// the first bucket, so a bucket per possible tile count of a sequence's last
// item suffices: span / 16 + 1 <= kSelfBuckets for spans up to 4096 tokens.
constexpr int kSelfBuckets = 264;
constexpr int kSelfMaxSeqs = 4096;              // larger batches use the work-list builder
// LDS scratch of the search (ints): bucket counts, then (workgroup-wide
// search) the scan's wave sums and the handed-over item.
constexpr int kSelfRes = kSelfBuckets + 16;
constexpr int kSelfLdsInts = kSelfRes + 4;
// Batches up to kSelfWaveSeqs sequences are ranked by one wave, with
// kSelfSeqsPerLane sequences a lane (the default); larger ones (up to
// kSelfMaxSeqs) by the whole workgroup.
constexpr int kSelfSeqsPerLane = 4;
constexpr int kSelfWaveSeqs = 64 * kSelfSeqsPerLane;

// A scheduled work item: (seq, part << 16 | kv head, t_begin, t_end | kItemFinal).
constexpr int kItemFinal = 1 << 30;  // the item stores the final output (no merge)

struct ScheduleArgs {
    const int32_t* context_lens;
    int4* items;
    int* item_count;
    // Items cover partition_tokens each (num_partitions of them per
    // sequence); an item stores the final output when its sequence's
    // context, counted in split_tokens-token partitions (split_count per
    // row), is a single partition. The two differ when an item spans
    // several partitions, one per wave.
    int32_t num_seqs, num_kv_heads, partition_tokens, num_partitions;
    int32_t split_tokens, split_count;
    int32_t max_context;           // max_blocks_per_seq * block_size
    // Cascade suffix pass: a sequence's items start after the tokens its
    // prefix group covers and, when it has any, none stores the final output.
    CascadeGroups cascade;
    int32_t block_size_log2;
};

struct MergeArgs {
    const int32_t* context_lens;
    const float* part_ml;
    const float* part_o;
    uint16_t* out;                 // [S, Hq, D], element strides out_seq, out_head
    int64_t out_seq, out_head;
    int32_t num_seqs, num_q_heads, head_dim, partition_tokens, num_partitions;
    int32_t max_context;           // max_blocks_per_seq * block_size
};

struct CacheWriteArgs {
    const uint16_t* k;             // [T, Hkv, D], element strides k_token, k_head
    const uint16_t* v;             // [T, Hkv, D], element strides v_token, v_head
    const int64_t* slot_mapping;   // [T]
    uint8_t* k_cache;              // [N, bs, Hkv, D] at `cache`
    uint8_t* v_cache;
    int64_t k_token, k_head, v_token, v_head;
    int64_t num_tokens;
    int64_t num_slots;             // N * bs
    int32_t num_kv_heads, head_dim, block_size_log2;
    CacheLayout cache;
    float k_scale, v_scale;        // fp8 only
};

// Arguments of the multi-row kernel (several query tokens per sequence,
// or more than 16 query heads per KV head), passed by value.
struct MultiArgs {
    const uint16_t* q;             // [num_query_rows, Hq, D] bf16, element strides q_row, q_head
    const uint8_t* k_cache;        // [N, bs, Hkv, D] bf16 or e4m3fn, at `cache`
    const uint8_t* v_cache;
    const int32_t* block_tables;   // [S, MB], row stride table_stride
    const int32_t* context_lens;   // [S]
    const int32_t* query_start;    // [S + 1]; null = one query token per sequence (row = seq)
    uint16_t* out;                 // [num_query_rows, Hq, D] bf16, element strides out_row, out_head
    float* part_ml;                // [num_query_rows, Hq, P, 2], split only
    float* part_o;                 // [num_query_rows, Hq, P, D], split only
    int64_t q_row, q_head, out_row, out_head, table_stride;
    int32_t num_seqs, num_query_rows, max_query_len;
    int32_t num_q_heads, num_kv_heads, group;
    int32_t block_size_log2, max_blocks_per_seq;
    int32_t partition_tokens, num_partitions;
    int32_t row_blocks;            // blocks of 16 * waves * row tiles rows per (sequence, KV head)
    int32_t last_block;
    CacheLayout cache;
    float qk_scale_log2, v_scale;
    // Device work list (null = direct grid): the decode work list of
    // (sequence, KV head, partition) items, longest first; workgroup b takes
    // item b / row_blocks, row block b % row_blocks.
    const int4* items;
    const int* item_count;
    // Self-scheduled (items null): workgroup b ranks itself in the same order
    // (batches of at most kSelfWaveSeqs sequences).
    int32_t self_schedule;
    // Cascade prefix pass (cascade.group_start non-null): the grid's
    // "sequence" k is prefix group k, block_tables holds the prefix tables,
    // the query rows are the members' (one token each, q row = sequence),
    // member i attends the first cascade_shared() tokens, and every state is
    // stored as a partial (stride num_partitions).
    CascadeGroups cascade;
};

// Arguments of the cascade merge: per (sequence, query head) the states of
// the prefix pass (prefix_partitions slots) and of the suffix pass
// (num_partitions slots), combined by log-sum-exp.
struct CascadeMergeArgs {
    const int32_t* context_lens;
    CascadeGroups cascade;
    const float* pre_ml;           // [S, Hq, prefix_partitions, 2]
    const float* pre_o;            // [S, Hq, prefix_partitions, D]
    const float* part_ml;          // [S, Hq, num_partitions, 2]
    const float* part_o;           // [S, Hq, num_partitions, D]
    uint16_t* out;                 // [S, Hq, D], element strides out_seq, out_head
    int64_t out_seq, out_head;
    int32_t num_seqs, num_q_heads, head_dim;
    int32_t prefix_partition_tokens, prefix_partitions;
    int32_t partition_tokens, num_partitions;
    int32_t max_context, block_size_log2;
};

struct CopyBlocksArgs {
    uint8_t* k_cache;              // [N, bs, Hkv, D]: block b is the byte range
    uint8_t* v_cache;              //   [b * block_stride, b * block_stride + block_bytes)
    const int64_t* pairs;          // [num_pairs][2] (src, dst)
    int64_t num_pairs;
    int64_t num_blocks;
    int64_t block_stride;          // bytes between blocks
    int64_t block_bytes;           // bs * Hkv * D * element size (a multiple of 16)
};

// How a decode kernel is launched.
struct LaunchShape {
    int waves;          // wavefronts per workgroup
    int depth;          // tiles a wave keeps in its register ring (2..4)
    int heads_per_unit; // MFMA kernel: adjacent KV heads sharing one 16-row tile (1, 2 or 4)
    bool wave_partitions; // MFMA kernel: each wave takes one whole partition of the item
};

// A dispatch counts its work-items in 32 bits: the plans refuse
// (PA_ERR_UNSUPPORTED, before any launch) a grid of 2^32 work-items or more
// rather than let it wrap.
inline bool grid_fits(int64_t blocks, int64_t threads_per_block) {
    return blocks >= 0 && blocks <= ((int64_t(1) << 32) - 1) / threads_per_block;
}

constexpr int kCopyThreads = 256;  // pa_copy_blocks: threads per block pair

// Launchers: return the hipError_t of the launch.
hipError_t launch_decode_valu(const DecodeArgs& a, int head_dim, bool fp8, const LaunchShape& ls, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs& a, int head_dim, bool fp8, const LaunchShape& ls, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_cascade_merge(const CascadeMergeArgs& a, hipStream_t s);
hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t s);
hipError_t launch_cache_write(const CacheWriteArgs& a, bool fp8, hipStream_t s);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s);
// streaming-read reference kernel (probe.hip)
hipError_t launch_probe_read(const void* buf, int64_t bytes, bool nontemporal, uint32_t* sink, int cus,
                             hipStream_t s);
// the multi-row kernel, then (split, not a cascade prefix pass) its merge
hipError_t launch_multi(const MultiArgs& a, int head_dim, bool fp8, int waves, int row_tiles, hipStream_t s);

// PA_DEBUG_VALIDATE set (and not "0"): the hot-path calls first run the
// precondition checks of validate.hip.
bool debug_validate_enabled();

}  // namespace pa
