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
    int32_t block_size_log2, max_blocks_per_seq;
    int32_t partition_tokens, num_partitions;
    int64_t num_blocks;
    uint32_t block_bytes;          // bytes of one physical block
    uint32_t slot_bytes;           // bytes of one token row (all KV heads)
    uint32_t head_bytes;           // bytes of one KV head's row
    float qk_scale_log2;           // scale * k_scale * log2(e)
    float v_scale;                 // 1 for bf16
    // Device schedule (null = direct grid, one workgroup per item):
    const int2* items;             // (seq, part << 16 | kv head), longest first
    const int* item_count;         // number of valid items
    int* queue;                    // next item to hand out (zeroed by the scheduler)
};

struct ScheduleArgs {
    const int32_t* context_lens;
    int2* items;
    int* item_count;
    int* queue;
    int32_t num_seqs, num_kv_heads, partition_tokens;
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

// How a decode kernel is launched.
struct LaunchShape {
    int waves;          // wavefronts per workgroup
    int depth;          // tiles a wave keeps in its register ring (2..4)
    int num_cus;        // compute units of the device
    int64_t max_items;  // persistent grid: upper bound on scheduled items (0 = direct grid)
};

// Workgroups to launch: one per (sequence, KV head, partition) for a direct
// grid; for a scheduled (persistent) grid, as many as can be resident at
// once (occupancy x compute units), but no more than there can be items.
inline int64_t grid_size(const void* kernel, const DecodeArgs& a, const LaunchShape& ls, size_t lds) {
    if (a.items == nullptr) return (int64_t)a.num_seqs * a.num_kv_heads * a.num_partitions;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * ls.waves, lds) != hipSuccess ||
        per_cu <= 0)
        per_cu = 1;
    const int64_t n = (int64_t)per_cu * ls.num_cus;
    return n < ls.max_items ? n : ls.max_items;
}

// Launchers: return the hipError_t of the launch.
hipError_t launch_decode_valu(const DecodeArgs& a, int head_dim, bool fp8, const LaunchShape& ls, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs& a, int head_dim, bool fp8, const LaunchShape& ls, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t s);
hipError_t launch_cache_write(const CacheWriteArgs& a, bool fp8, hipStream_t s);

}  // namespace pa
