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
//   multi-token: those of decode, and each sequence's query tokens are some
//                of its cached ones (query_start rises from 0 by n_i with
//                0 <= n_i <= min(max_query_len, context length)): Tutorial
//                §5.1 verifies drafts that were appended to the cache and
//                §6.2's chunks attend over what is already cached;
//   cascade:     the group offsets rise from >= 0 to <= num_seqs, no group
//                has more than max_group_size sequences, every prefix length
//                is a whole number of blocks within its table row, and the
//                entries that cover it name blocks inside the pool (Tutorial
//                §4.3: a cached prefix is shared as whole blocks).
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "pa_abi.h"

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

// A table [rows, cols] with row stride `stride` into a dense host copy.
int copy_table(std::vector<int32_t>& dst, const pa::abi::Table& t, hipStream_t s) {
    dst.resize((size_t)t.rows * t.cols);
    if (t.rows == 0 || t.cols == 0) return PA_OK;
    if (hipMemcpy2DAsync(dst.data(), (size_t)t.cols * 4, t.data, (size_t)t.stride * 4, (size_t)t.cols * 4,
                         (size_t)t.rows, hipMemcpyDeviceToHost, s) != hipSuccess)
        return PA_ERR_LAUNCH;
    if (hipStreamSynchronize(s) != hipSuccess) return PA_ERR_LAUNCH;
    return PA_OK;
}

// Context lengths within their table rows, covering entries inside the pool.
int check_tables(const std::vector<int32_t>& ctx, const std::vector<int32_t>& table, int64_t S, int32_t MB,
                 int32_t bs, int64_t N) {
    const int64_t cap = (int64_t)MB * bs;
    for (int64_t i = 0; i < S; ++i) {
        const int64_t c = ctx[(size_t)i];
        if (c < 0 || c > cap) return PA_ERR_PRECONDITION;
        const int64_t nb = (c + bs - 1) / bs;
        const int32_t* row = table.data() + (size_t)i * MB;
        for (int64_t b = 0; b < nb; ++b)
            if (row[b] < 0 || row[b] >= N) return PA_ERR_PRECONDITION;
    }
    return PA_OK;
}

// The tables and lengths of a decode-family call: their arguments checked
// (parse_decode_inputs, no device access), then read to the host.
int parse_decode_inputs(const pa_tensor* block_tables, const pa_tensor* context_lens, const pa_tensor* k_cache,
                        pa::abi::Table* t, pa::abi::Cache* c, const int32_t** cl) {
    int st = pa::abi::cache(k_cache, c, false);
    if (st != PA_OK) return st;
    st = pa::abi::table(block_tables, t);
    if (st != PA_OK) return st;
    int64_t n = 0;
    st = pa::abi::vec(context_lens, PA_DTYPE_I32, cl, &n);
    if (st != PA_OK) return st;
    if (n != t->rows) return PA_ERR_SHAPE;
    if (n > 0 && t->cols <= 0) return PA_ERR_SHAPE;
    return PA_OK;
}

int read_decode_inputs(const pa::abi::Table& t, const int32_t* cl, hipStream_t s, std::vector<int32_t>* ctx,
                       std::vector<int32_t>* table) {
    if (t.rows == 0) return PA_OK;
    int st = copy_to_host(*ctx, cl, t.rows, s);
    if (st != PA_OK) return st;
    return copy_table(*table, t, s);
}

}  // namespace

namespace pa {

bool debug_validate_enabled() {
    const char* e = std::getenv("PA_DEBUG_VALIDATE");
    return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
}

}  // namespace pa

extern "C" {

int pa_check_cache_write_inputs(const pa_tensor* slot_mapping, const pa_tensor* k_cache, void* stream) {
    pa::abi::Cache c;
    int st = pa::abi::cache(k_cache, &c, false);
    if (st != PA_OK) return st;
    const int64_t* sm = nullptr;
    int64_t n = 0;
    st = pa::abi::vec(slot_mapping, PA_DTYPE_I64, &sm, &n);
    if (st != PA_OK) return st;
    if (n == 0) return PA_OK;
    std::vector<int64_t> slots;
    st = copy_to_host(slots, sm, n, static_cast<hipStream_t>(stream));
    if (st != PA_OK) return st;
    const int64_t num_slots = c.N * c.bs;
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

int pa_check_decode_inputs(const pa_tensor* block_tables, const pa_tensor* context_lens, const pa_tensor* k_cache,
                           void* stream) {
    pa::abi::Table t;
    pa::abi::Cache c;
    const int32_t* cl = nullptr;
    int st = parse_decode_inputs(block_tables, context_lens, k_cache, &t, &c, &cl);
    if (st != PA_OK || t.rows == 0) return st;
    std::vector<int32_t> ctx, table;
    st = read_decode_inputs(t, cl, static_cast<hipStream_t>(stream), &ctx, &table);
    if (st != PA_OK) return st;
    return check_tables(ctx, table, t.rows, t.cols, c.bs, c.N);
}

int pa_check_multi_inputs(const pa_tensor* block_tables, const pa_tensor* context_lens, const pa_tensor* query_start,
                          int32_t max_query_len, const pa_tensor* k_cache, void* stream) {
    if (max_query_len < 0) return PA_ERR_SHAPE;
    pa::abi::Table t;
    pa::abi::Cache c;
    const int32_t* cl = nullptr;
    int st = parse_decode_inputs(block_tables, context_lens, k_cache, &t, &c, &cl);
    if (st != PA_OK) return st;
    const int32_t* qs = nullptr;
    int64_t n = 0;
    st = pa::abi::vec(query_start, PA_DTYPE_I32, &qs, &n);
    if (st != PA_OK) return st;
    if (n != t.rows + 1) return PA_ERR_SHAPE;
    if (t.rows == 0) return PA_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<int32_t> ctx, table, starts;
    st = read_decode_inputs(t, cl, s, &ctx, &table);
    if (st != PA_OK) return st;
    st = check_tables(ctx, table, t.rows, t.cols, c.bs, c.N);
    if (st != PA_OK) return st;
    st = copy_to_host(starts, qs, n, s);
    if (st != PA_OK) return st;
    if (starts[0] != 0) return PA_ERR_PRECONDITION;
    for (int64_t i = 0; i < t.rows; ++i) {
        const int64_t q = (int64_t)starts[(size_t)i + 1] - starts[(size_t)i];
        if (q < 0 || q > max_query_len || q > ctx[(size_t)i]) return PA_ERR_PRECONDITION;
    }
    return PA_OK;
}

int pa_check_cascade_inputs(const pa_tensor* prefix_tables, const pa_tensor* prefix_lens, const pa_tensor* group_start,
                            int32_t max_group_size, int32_t num_seqs, const pa_tensor* k_cache, void* stream) {
    if (max_group_size < 0 || num_seqs < 0) return PA_ERR_SHAPE;
    pa::abi::Cache c;
    int st = pa::abi::cache(k_cache, &c, false);
    if (st != PA_OK) return st;
    if (prefix_tables == nullptr) return PA_OK;  // no groups
    pa::abi::Table t;
    st = pa::abi::table(prefix_tables, &t);
    if (st != PA_OK) return st;
    const int64_t G = t.rows;
    if (G == 0) return PA_OK;
    const int32_t *pl = nullptr, *gs = nullptr;
    int64_t n = 0;
    st = pa::abi::vec(prefix_lens, PA_DTYPE_I32, &pl, &n);
    if (st != PA_OK) return st;
    if (n != G) return PA_ERR_SHAPE;
    st = pa::abi::vec(group_start, PA_DTYPE_I32, &gs, &n);
    if (st != PA_OK) return st;
    if (n != G + 1) return PA_ERR_SHAPE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<int32_t> starts, lens, table;
    st = copy_to_host(starts, gs, G + 1, s);
    if (st != PA_OK) return st;
    st = copy_to_host(lens, pl, G, s);
    if (st != PA_OK) return st;
    st = copy_table(table, t, s);
    if (st != PA_OK) return st;
    const int32_t bs = c.bs;
    if (starts[0] < 0 || starts[(size_t)G] > num_seqs) return PA_ERR_PRECONDITION;
    for (int64_t k = 0; k < G; ++k) {
        const int64_t m = (int64_t)starts[(size_t)k + 1] - starts[(size_t)k];
        if (m < 0 || m > max_group_size) return PA_ERR_PRECONDITION;
        const int64_t len = lens[(size_t)k];
        if (len < 0 || len % bs != 0 || len > (int64_t)t.cols * bs) return PA_ERR_PRECONDITION;
        const int32_t* row = table.data() + (size_t)k * t.cols;
        for (int64_t b = 0; b < len / bs; ++b)
            if (row[b] < 0 || row[b] >= c.N) return PA_ERR_PRECONDITION;
    }
    return PA_OK;
}

}  // extern "C"
