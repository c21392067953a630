// cache_write.hip -- store the new tokens' K/V rows into the paged caches.
//
// Tutorial «大模型推理优化与加速完全教程» §4.2 "PagedAttention"
// (PagedKVCache.append_token) writes the new token's K and V at row
// `offset` of physical block `block`; the slot id here is that row's flat
// index block * block_size + offset. For an fp8 cache every element becomes
// the e4m3fn code of x / scale (Tutorial §3.1 "量化基础", symmetric_quantize).
//
// One thread moves one 8-element chunk of one (token, KV head) row of K and
// the same chunk of V (16 bytes read; 16 bytes written for bf16, 8 for fp8);
// consecutive threads cover consecutive chunks of a row, so each source and
// destination row is read and written by D / 8 neighbouring threads. Source
// rows and cache rows are addressed through their strides (any layout of
// the pool: the page's [block, row, KV head, d] order or a head-major one).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

template <bool FP8>
__global__ __launch_bounds__(256) void pa_cache_write_kernel(CacheWriteArgs a) {
    constexpr int ESZ = FP8 ? 1 : 2;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int chunks_per_row = a.head_dim / 8;
    const int64_t per_token = (int64_t)a.num_kv_heads * chunks_per_row;
    if (gid >= a.num_tokens * per_token) return;
    const int64_t t = gid / per_token;
    const int h = (int)((gid - t * per_token) / chunks_per_row);
    const int ch = (int)(gid - t * per_token - (int64_t)h * chunks_per_row);
    const int64_t slot = a.slot_mapping[t];
    if (slot < 0 || slot >= a.num_slots) return;  // padding, or outside the pool
    const int64_t blk = slot >> a.block_size_log2;
    const uint32_t row = (uint32_t)(slot & ((1 << a.block_size_log2) - 1));
    // byte offset of this 8-element chunk in the caches
    const int64_t dst = blk * a.cache.block + (int64_t)row * a.cache.token + (int64_t)h * a.cache.head + ch * 8 * ESZ;
    const u32x4 kw = *reinterpret_cast<const u32x4*>(a.k + t * a.k_token + (int64_t)h * a.k_head + 8 * ch);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(a.v + t * a.v_token + (int64_t)h * a.v_head + 8 * ch);
    if constexpr (!FP8) {
        *reinterpret_cast<u32x4*>(a.k_cache + dst) = kw;
        *reinterpret_cast<u32x4*>(a.v_cache + dst) = vw;
    } else {
        u32x2 kc, vc;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint32_t kk = 0, vv = 0;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t kwj = kw[2 * i + j], vwj = vw[2 * i + j];
                const uint32_t k0 = fp8_e4m3fn_encode(bf16_lo(kwj) / a.k_scale);
                const uint32_t k1 = fp8_e4m3fn_encode(bf16_hi(kwj) / a.k_scale);
                const uint32_t v0 = fp8_e4m3fn_encode(bf16_lo(vwj) / a.v_scale);
                const uint32_t v1 = fp8_e4m3fn_encode(bf16_hi(vwj) / a.v_scale);
                kk |= (k0 | (k1 << 8)) << (16 * j);
                vv |= (v0 | (v1 << 8)) << (16 * j);
            }
            kc[i] = kk;
            vc[i] = vv;
        }
        *reinterpret_cast<u32x2*>(a.k_cache + dst) = kc;
        *reinterpret_cast<u32x2*>(a.v_cache + dst) = vc;
    }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, bool fp8, hipStream_t s) {
    const int64_t threads = a.num_tokens * a.num_kv_heads * (a.head_dim / 8);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (fp8) hipLaunchKernelGGL(pa_cache_write_kernel<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(pa_cache_write_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace pa
