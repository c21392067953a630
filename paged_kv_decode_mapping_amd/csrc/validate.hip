// validate.hip -- opt-in checks of the device-side preconditions that the
// hot-path calls leave unchecked (host code; synchronises the stream).
//
// pa_cache_write and pa_decode check their arguments on the host only and
// never read device memory before launching. What lives in device memory --
// slot ids, block-table entries, context lengths -- is a precondition there:
// the kernels stay inside the pool whatever those hold, but the results are
// unspecified when they are wrong. These entry points copy those index
// arrays to the host and check them. They are for debugging: each call
// synchronises `stream` and costs a device-to-host copy.
//
// What is checked (Tutorial «大模型推理优化与加速完全教程» §4.2,
// PagedKVCache: a token's K/V live in row `offset` of the physical block its
// table entry names; allocate/append hand out each slot once):
//   cache write: every slot is negative (padding) or inside the pool
//                [0, num_blocks * block_size), and no slot appears twice;
//   decode:      every context length is in [0, max_blocks_per_seq *
//                block_size], and the table entries that cover it (the first
//                ceil(ctx / block_size) of the row) name blocks inside the pool;
//   cascade:     the group offsets rise from >= 0 to <= num_seqs, no group
//                has more than max_group_size sequences, every prefix length
//                is a whole number of blocks within its table row, and the
//                entries that cover it name blocks inside the pool (Tutorial
//                §4.3: a cached prefix is shared as whole blocks).
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

template <class T>
int copy_to_host(std::vector<T>& dst, const T* src, int64_t n, hipStream_t s) {
    dst.resize((size_t)n);
    if (n == 0) return PA_OK;
    if (hipMemcpyAsync(dst.data(), src, (size_t)n * sizeof(T), hipMemcpyDeviceToHost, s) != hipSuccess)
        return PA_ERR_LAUNCH;
    if (hipStreamSynchronize(s) != hipSuccess) return PA_ERR_LAUNCH;
    return PA_OK;
}

}  // namespace

namespace pa {

bool debug_validate_enabled() {
    const char* e = std::getenv("PA_DEBUG_VALIDATE");
    return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
}

}  // namespace pa

extern "C" {

int pa_check_cache_write_inputs(const int64_t* slot_mapping, int64_t num_tokens, int32_t block_size,
                                int64_t num_blocks, void* stream) {
    if (num_tokens < 0 || block_size <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
    if (num_tokens == 0) return PA_OK;
    if (!slot_mapping) return PA_ERR_NULL;
    std::vector<int64_t> slots;
    const int st = copy_to_host(slots, slot_mapping, num_tokens, static_cast<hipStream_t>(stream));
    if (st != PA_OK) return st;
    const int64_t num_slots = num_blocks * block_size;
    std::vector<int64_t> used;
    used.reserve(slots.size());
    for (const int64_t s : slots) {
        if (s < 0) continue;
        if (s >= num_slots) return PA_ERR_PRECONDITION;
        used.push_back(s);
    }
    std::sort(used.begin(), used.end());
    if (std::adjacent_find(used.begin(), used.end()) != used.end()) return PA_ERR_PRECONDITION;
    return PA_OK;
}

int pa_check_decode_inputs(const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                           int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                           void* stream) {
    if (num_seqs < 0 || block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
    if (num_seqs == 0) return PA_OK;
    if (!block_tables || !context_lens) return PA_ERR_NULL;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<int32_t> ctx, table;
    int st = copy_to_host(ctx, context_lens, num_seqs, s);
    if (st != PA_OK) return st;
    st = copy_to_host(table, block_tables, (int64_t)num_seqs * max_blocks_per_seq, s);
    if (st != PA_OK) return st;
    const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
    for (int32_t i = 0; i < num_seqs; ++i) {
        const int64_t c = ctx[(size_t)i];
        if (c < 0 || c > cap) return PA_ERR_PRECONDITION;
        const int64_t nb = (c + block_size - 1) / block_size;
        const int32_t* row = table.data() + (size_t)i * max_blocks_per_seq;
        for (int64_t b = 0; b < nb; ++b)
            if (row[b] < 0 || row[b] >= num_blocks) return PA_ERR_PRECONDITION;
    }
    return PA_OK;
}

int pa_check_cascade_inputs(const int32_t* prefix_tables, const int32_t* prefix_lens, const int32_t* group_start,
                            int32_t num_groups, int32_t max_group_size, int32_t max_prefix_blocks, int32_t num_seqs,
                            int32_t block_size, int64_t num_blocks, void* stream) {
    if (num_groups < 0 || max_group_size < 0 || max_prefix_blocks < 0 || num_seqs < 0 || block_size <= 0 ||
        num_blocks <= 0)
        return PA_ERR_SHAPE;
    if (num_groups == 0) return PA_OK;
    if (!group_start || !prefix_lens || (max_prefix_blocks > 0 && !prefix_tables)) return PA_ERR_NULL;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<int32_t> starts, lens, table;
    int st = copy_to_host(starts, group_start, (int64_t)num_groups + 1, s);
    if (st != PA_OK) return st;
    st = copy_to_host(lens, prefix_lens, num_groups, s);
    if (st != PA_OK) return st;
    st = copy_to_host(table, prefix_tables, (int64_t)num_groups * max_prefix_blocks, s);
    if (st != PA_OK) return st;
    if (starts[0] < 0 || starts[(size_t)num_groups] > num_seqs) return PA_ERR_PRECONDITION;
    for (int32_t k = 0; k < num_groups; ++k) {
        const int64_t n = (int64_t)starts[(size_t)k + 1] - starts[(size_t)k];
        if (n < 0 || n > max_group_size) return PA_ERR_PRECONDITION;
        const int64_t pl = lens[(size_t)k];
        if (pl < 0 || pl % block_size != 0 || pl > (int64_t)max_prefix_blocks * block_size) return PA_ERR_PRECONDITION;
        const int32_t* row = table.data() + (size_t)k * max_prefix_blocks;
        for (int64_t b = 0; b < pl / block_size; ++b)
            if (row[b] < 0 || row[b] >= num_blocks) return PA_ERR_PRECONDITION;
    }
    return PA_OK;
}

}  // extern "C"
