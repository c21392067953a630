// pa_internal.h -- kernel argument blocks and launcher declarations inside
// libpa (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kTile = 16;  // tokens per decode tile (one MFMA M/N extent)

// Arguments of the decode kernels, passed by value.
struct DecodeArgs {
    const uint16_t* q;             // [S, Hq, D] bf16
    const uint8_t* k_cache;        // [N, bs, Hkv, D] bf16 or e4m3fn
    const uint8_t* v_cache;
    const int32_t* block_tables;   // [S, MB]
    const int32_t* context_lens;   // [S]
    uint16_t* out;                 // [S, Hq, D] bf16
    float* part_ml;                // [S, Hq, P, 2] (max in log2 units, sum), split only
    float* part_o;                 // [S, Hq, P, D] unnormalised outputs, split only
    int32_t num_seqs, num_q_heads, num_kv_heads, group;
    int32_t units_per_seq;         // work units per sequence: KV heads / heads per unit
    int32_t block_size_log2, max_blocks_per_seq;
    int32_t partition_tokens, num_partitions;
    int32_t last_block;            // min(num_blocks, 2^31) - 1: the largest usable block id
    uint32_t block_bytes;          // bytes of one physical block
    uint32_t slot_bytes;           // bytes of one token row (all KV heads)
    uint32_t head_bytes;           // bytes of one KV head's row
    float qk_scale_log2;           // scale * k_scale * log2(e)
    float v_scale;                 // 1 for bf16
    // Device schedule (null = direct grid, one workgroup per item):
    const int4* items;             // see ScheduleArgs, longest first
    const int* item_count;         // number of valid items
};

// A scheduled work item: (seq, part << 16 | kv head, t_begin, t_end | kItemFinal).
constexpr int kItemFinal = 1 << 30;  // the item stores the final output (no merge)

struct ScheduleArgs {
    const int32_t* context_lens;
    int4* items;
    int* item_count;
    int32_t num_seqs, num_kv_heads, partition_tokens, num_partitions;
    int32_t max_context;           // max_blocks_per_seq * block_size
};

struct MergeArgs {
    const int32_t* context_lens;
    const float* part_ml;
    const float* part_o;
    uint16_t* out;
    int32_t num_seqs, num_q_heads, head_dim, partition_tokens, num_partitions;
    int32_t max_context;           // max_blocks_per_seq * block_size
};

struct CacheWriteArgs {
    const uint16_t* k;             // [T, Hkv, D]
    const uint16_t* v;
    const int64_t* slot_mapping;   // [T]
    uint8_t* k_cache;              // [N, bs, Hkv, D]
    uint8_t* v_cache;
    int64_t num_tokens;
    int64_t num_slots;             // N * bs
    int32_t num_kv_heads, head_dim;
    float k_scale, v_scale;        // fp8 only
};

// Arguments of the multi-row kernel (several query tokens per sequence,
// or more than 16 query heads per KV head), passed by value.
struct MultiArgs {
    const uint16_t* q;             // [num_query_rows, Hq, D] bf16
    const uint8_t* k_cache;        // [N, bs, Hkv, D] bf16 or e4m3fn
    const uint8_t* v_cache;
    const int32_t* block_tables;   // [S, MB]
    const int32_t* context_lens;   // [S]
    const int32_t* query_start;    // [S + 1]; null = one query token per sequence (row = seq)
    uint16_t* out;                 // [num_query_rows, Hq, D] bf16
    float* part_ml;                // [num_query_rows, Hq, P, 2], split only
    float* part_o;                 // [num_query_rows, Hq, P, D], split only
    int32_t num_seqs, num_query_rows, max_query_len;
    int32_t num_q_heads, num_kv_heads, group;
    int32_t block_size_log2, max_blocks_per_seq;
    int32_t partition_tokens, num_partitions;
    int32_t row_blocks;            // blocks of 16 * waves rows per (sequence, KV head)
    int32_t last_block;
    uint32_t block_bytes, slot_bytes, head_bytes;
    float qk_scale_log2, v_scale;
    // Device work list (null = direct grid): the decode work list of
    // (sequence, KV head, partition) items, longest first; workgroup b takes
    // item b / row_blocks, row block b % row_blocks.
    const int4* items;
    const int* item_count;
};

struct CopyBlocksArgs {
    uint8_t* k_cache;              // [N, bs, Hkv, D]
    uint8_t* v_cache;
    const int64_t* pairs;          // [num_pairs][2] (src, dst)
    int64_t num_pairs;
    int64_t num_blocks;
    int64_t block_bytes;           // bs * Hkv * D * element size (a multiple of 16)
};

// How a decode kernel is launched.
struct LaunchShape {
    int waves;          // wavefronts per workgroup
    int depth;          // tiles a wave keeps in its register ring (2..4)
    int heads_per_unit; // MFMA kernel: adjacent KV heads sharing one 16-row tile (1, 2 or 4)
};

// Launchers: return the hipError_t of the launch.
hipError_t launch_decode_valu(const DecodeArgs& a, int head_dim, bool fp8, const LaunchShape& ls, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs& a, int head_dim, bool fp8, const LaunchShape& ls, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t s);
hipError_t launch_cache_write(const CacheWriteArgs& a, bool fp8, hipStream_t s);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s);
// streaming-read reference kernel (probe.hip)
hipError_t launch_probe_read(const void* buf, int64_t bytes, bool nontemporal, uint32_t* sink, int cus,
                             hipStream_t s);
// the multi-row kernel, then (split) its merge
hipError_t launch_multi(const MultiArgs& a, int head_dim, bool fp8, int waves, hipStream_t s);

// PA_DEBUG_VALIDATE set (and not "0"): the hot-path calls first run the
// precondition checks of validate.hip.
bool debug_validate_enabled();

}  // namespace pa
