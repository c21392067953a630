// pa_cascade.h -- prefix groups of a cascade (shared-prefix) decode, as
// the work-list builder, the prefix pass and the cascade merge see them.
//
// Tutorial «大模型推理优化与加速完全教程» §4.3 (Prefix Caching): requests
// that share a prompt prefix reuse the physical blocks cached for it; the
// prefix cache keeps each prefix's block list and length. A cascade call
// groups the sequences that share one: group k is a run of consecutive
// sequences whose first prefix_lens[k] tokens are read through prefix
// table row k (once for the whole group) and whose remaining tokens are
// read through their own rows.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Prefix group of sequence `seq` in a cascade call, or -1: the last k with
// group_start[k] <= seq, if seq is also below group_start[k + 1] and among
// the group's first max_group_size sequences. Every index read stays inside
// group_start[0 .. num_groups] whatever the array holds.
__device__ __forceinline__ int cascade_group(const CascadeGroups& c, int seq) {
    if (c.group_start == nullptr || c.num_groups <= 0 || c.group_start[0] > seq) return -1;
    int lo = 0, hi = c.num_groups - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (c.group_start[mid] <= seq) lo = mid;
        else hi = mid - 1;
    }
    const int first = c.group_start[lo];
    if (seq >= c.group_start[lo + 1] || seq - first >= c.max_group_size) return -1;
    return lo;
}

// Prefix length of group k: clamped to its table row, whole blocks.
__device__ __forceinline__ int cascade_prefix_tokens(const CascadeGroups& c, int k, int block_size_log2) {
    int pl = c.prefix_lens[k];
    pl = pl < 0 ? 0 : (pl > c.max_prefix_tokens ? c.max_prefix_tokens : pl);
    return (pl >> block_size_log2) << block_size_log2;
}

// Tokens of sequence `seq` (context ctx) read through its group's prefix
// table: min(ctx, prefix length), 0 outside every group. The rest, ctx -
// shared, are read through the sequence's own table row.
__device__ __forceinline__ int cascade_shared(const CascadeGroups& c, int seq, int ctx, int block_size_log2) {
    const int k = cascade_group(c, seq);
    if (k < 0) return 0;
    return min(ctx, cascade_prefix_tokens(c, k, block_size_log2));
}

}  // namespace pa
