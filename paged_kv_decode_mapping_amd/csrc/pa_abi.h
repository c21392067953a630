// pa_abi.h -- host-side reading of the pa_tensor arguments of the C ABI:
// element type, shape and stride rules, and the geometry the kernels are
// launched with. Host code only (pa_api.hip and validate.hip).
#pragma once

#include <algorithm>
#include <cstdint>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace pa {
namespace abi {

inline bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
inline int log2i(int64_t x) {
    int r = 0;
    while ((int64_t(1) << r) < x) ++r;
    return r;
}
inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline int64_t numel(const pa_tensor& t) {
    int64_t n = 1;
    for (int i = 0; i < t.ndim; ++i) n *= t.shape[i];
    return n;
}

// Checks common to every tensor argument: a known rank, sizes >= 0,
// strides >= 0, the last dimension contiguous (size-1 dimensions excepted),
// and (need_data: a call that runs, not a plan) data unless it is empty.
inline int basic(const pa_tensor* t, int ndim, int dtype, bool need_data = true) {
    if (t == nullptr) return PA_ERR_NULL;
    if (t->ndim != ndim) return PA_ERR_SHAPE;
    if (t->dtype != dtype) return PA_ERR_DTYPE;
    for (int i = 0; i < ndim; ++i) {
        if (t->shape[i] < 0) return PA_ERR_SHAPE;
        if (t->stride[i] < 0) return PA_ERR_LAYOUT;
    }
    if (t->shape[ndim - 1] > 1 && t->stride[ndim - 1] != 1) return PA_ERR_LAYOUT;
    if (need_data && numel(*t) > 0 && t->data == nullptr) return PA_ERR_NULL;
    return PA_OK;
}

// No two index tuples of the tensor share an element: with the dimensions
// of size > 1 sorted by stride, each stride reaches past the previous
// dimension's whole extent.
inline bool no_self_overlap(const pa_tensor& t) {
    int64_t st[4], sz[4];
    int n = 0;
    for (int i = 0; i < t.ndim; ++i)
        if (t.shape[i] > 1) {
            if (t.stride[i] == 0) return false;  // every index of this dimension is the same element
            st[n] = t.stride[i];
            sz[n] = t.shape[i];
            ++n;
        }
    for (int i = 1; i < n; ++i)  // insertion sort by stride
        for (int j = i; j > 0 && st[j] < st[j - 1]; --j) {
            std::swap(st[j], st[j - 1]);
            std::swap(sz[j], sz[j - 1]);
        }
    for (int i = 1; i < n; ++i)
        if (st[i] < st[i - 1] * sz[i - 1]) return false;
    return true;
}

// [rows, heads, head_dim] bf16 rows (q, out, k, v): strides of 16-byte
// multiples, 16-byte aligned data.
struct Rows {
    void* data;
    int64_t rows;
    int32_t heads, dim;
    int64_t s_row, s_head;  // element strides
};

inline int rows(const pa_tensor* t, bool written, Rows* r, bool need_data = true) {
    int st = basic(t, 3, PA_DTYPE_BF16, need_data);
    if (st != PA_OK) return st;
    if (t->shape[1] > INT32_MAX || t->shape[2] > INT32_MAX || t->shape[0] > INT32_MAX) return PA_ERR_UNSUPPORTED;
    r->data = t->data;
    r->rows = t->shape[0];
    r->heads = (int32_t)t->shape[1];
    r->dim = (int32_t)t->shape[2];
    r->s_row = t->shape[0] > 1 ? t->stride[0] : 0;
    r->s_head = t->shape[1] > 1 ? t->stride[1] : 0;
    if (r->s_row % 8 != 0 || r->s_head % 8 != 0) return PA_ERR_LAYOUT;
    if (written && !no_self_overlap(*t)) return PA_ERR_LAYOUT;
    if (numel(*t) > 0 && !aligned(t->data, 16)) return PA_ERR_ALIGN;
    return PA_OK;
}

// A paged cache [num_blocks, block_size, num_kv_heads, head_dim].
struct Cache {
    uint8_t* data;
    int64_t N;
    int32_t bs, Hkv, D, dtype, esz;
    CacheLayout lay;        // byte strides
    bool heads_adjacent;    // head stride == head_dim: a row's KV heads are one contiguous run
    bool blocks_contiguous; // every block is one dense byte range (pa_copy_blocks)
    int64_t block_bytes;    // bs * Hkv * D * esz
};

inline int cache(const pa_tensor* t, Cache* c, bool need_data = true) {
    if (t == nullptr) return PA_ERR_NULL;
    if (t->dtype != PA_DTYPE_BF16 && t->dtype != PA_DTYPE_FP8_E4M3FN) return PA_ERR_DTYPE;
    int st = basic(t, 4, t->dtype, need_data);
    if (st != PA_OK) return st;
    const int64_t N = t->shape[0], bs = t->shape[1], Hkv = t->shape[2], D = t->shape[3];
    if (N <= 0 || bs <= 0 || Hkv <= 0 || D <= 0) return PA_ERR_SHAPE;
    if (D != 64 && D != 128) return PA_ERR_UNSUPPORTED;
    if (!is_pow2(bs) || bs < kTile || bs > 1024) return PA_ERR_UNSUPPORTED;
    if (Hkv > 65535) return PA_ERR_UNSUPPORTED;
    const int esz = t->dtype == PA_DTYPE_BF16 ? 2 : 1;
    const int64_t unit = 16 / esz;  // elements per 16 bytes
    const int64_t sN = t->stride[0], sT = t->stride[1], sH = Hkv > 1 ? t->stride[2] : D;
    if (sN % unit != 0 || sT % unit != 0 || sH % unit != 0) return PA_ERR_LAYOUT;
    if (!no_self_overlap(*t)) return PA_ERR_LAYOUT;
    // a block's rows must be addressable with 32-bit byte offsets
    const int64_t extent = ((bs - 1) * sT + (Hkv - 1) * sH + D) * esz;
    if (extent >= (int64_t(1) << 31)) return PA_ERR_LAYOUT;
    if (N > 1 && sN > (INT64_MAX / esz) / N) return PA_ERR_LAYOUT;
    if (!aligned(t->data, 16)) return PA_ERR_ALIGN;
    c->data = static_cast<uint8_t*>(t->data);
    c->N = N;
    c->bs = (int32_t)bs;
    c->Hkv = (int32_t)Hkv;
    c->D = (int32_t)D;
    c->dtype = t->dtype;
    c->esz = esz;
    c->lay.block = (N > 1 ? sN : extent / esz) * esz;
    c->lay.token = (uint32_t)(sT * esz);
    c->lay.head = (uint32_t)(sH * esz);
    c->heads_adjacent = sH == D;
    c->block_bytes = bs * Hkv * D * esz;
    // A block is one dense byte range when its elements (which do not
    // overlap) reach exactly as far as their count.
    c->blocks_contiguous = extent == c->block_bytes && (N == 1 || sN >= bs * Hkv * D);
    return PA_OK;
}

// K and V caches: one layout, one element type.
inline int caches(const pa_tensor* k, const pa_tensor* v, Cache* c) {
    int st = cache(k, c);
    if (st != PA_OK) return st;
    Cache cv;
    st = cache(v, &cv);
    if (st != PA_OK) return st;
    if (cv.dtype != c->dtype) return PA_ERR_DTYPE;
    if (cv.N != c->N || cv.bs != c->bs || cv.Hkv != c->Hkv || cv.D != c->D) return PA_ERR_SHAPE;
    if (cv.lay.block != c->lay.block || cv.lay.token != c->lay.token || cv.lay.head != c->lay.head)
        return PA_ERR_LAYOUT;
    return PA_OK;
}

// [rows, cols] int32 table (block tables, prefix tables): unit inner
// stride, any row stride >= cols.
struct Table {
    const int32_t* data;
    int64_t rows;
    int32_t cols;
    int64_t stride;
};

inline int table(const pa_tensor* t, Table* b, bool need_data = true) {
    int st = basic(t, 2, PA_DTYPE_I32, need_data);
    if (st != PA_OK) return st;
    if (t->shape[0] > INT32_MAX || t->shape[1] > INT32_MAX) return PA_ERR_UNSUPPORTED;
    b->data = static_cast<const int32_t*>(t->data);
    b->rows = t->shape[0];
    b->cols = (int32_t)t->shape[1];
    b->stride = t->shape[0] > 1 ? t->stride[0] : t->shape[1];
    if (t->shape[0] > 1 && b->stride < b->cols) return PA_ERR_LAYOUT;
    if (numel(*t) > 0 && !aligned(t->data, 4)) return PA_ERR_ALIGN;
    return PA_OK;
}

// A contiguous 1-D index array.
template <class T>
inline int vec(const pa_tensor* t, int dtype, const T** data, int64_t* n) {
    int st = basic(t, 1, dtype);
    if (st != PA_OK) return st;
    *data = static_cast<const T*>(t->data);
    *n = t->shape[0];
    if (*n > 0 && !aligned(t->data, sizeof(T))) return PA_ERR_ALIGN;
    return PA_OK;
}

}  // namespace abi
}  // namespace pa
