// copy_blocks.hip -- duplicate physical blocks of the paged caches: the copy
// step of copy-on-write.
//
// Tutorial «大模型推理优化与加速完全教程» §4.2 lists copy-on-write among
// PagedKVCache's features (beam search forks share blocks), and §4.3
// "Prefix Caching" shares a prefix's blocks between sequences. Before one
// sharer may append into a shared block, the block is duplicated into a
// free one and that sharer's table entry is repointed. This kernel does the
// duplication: for each (src, dst) pair, block dst of K and of V becomes a
// byte-for-byte copy of block src (all rows, all KV heads).
//
// A block is one contiguous byte range (the block dimension outermost in
// memory, whatever the order of the other three). Workgroup p copies pair
// p's block in both caches: each thread moves
// 16-byte chunks t, t + 256, ..., issuing kUnroll loads of K and of V before
// their stores so that enough bytes are in flight. The data is read once and
// written once, so loads and stores are marked non-temporal. Pairs with a
// negative or out-of-pool id are skipped.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kUnroll = 8;

__global__ __launch_bounds__(kCopyThreads) void pa_copy_blocks_kernel(CopyBlocksArgs a) {
    const int64_t p = blockIdx.x;
    const int64_t src = a.pairs[2 * p];
    const int64_t dst = a.pairs[2 * p + 1];
    if (src < 0 || dst < 0 || src >= a.num_blocks || dst >= a.num_blocks) return;
    const int64_t chunks = a.block_bytes / 16;
    const u32x4* ks = reinterpret_cast<const u32x4*>(a.k_cache + src * a.block_stride);
    const u32x4* vs = reinterpret_cast<const u32x4*>(a.v_cache + src * a.block_stride);
    u32x4* kd = reinterpret_cast<u32x4*>(a.k_cache + dst * a.block_stride);
    u32x4* vd = reinterpret_cast<u32x4*>(a.v_cache + dst * a.block_stride);
    for (int64_t base = threadIdx.x; base < chunks; base += (int64_t)kUnroll * kCopyThreads) {
        u32x4 k[kUnroll], v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kCopyThreads;
            if (i < chunks) {
                k[u] = __builtin_nontemporal_load(ks + i);
                v[u] = __builtin_nontemporal_load(vs + i);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kCopyThreads;
            if (i < chunks) {
                __builtin_nontemporal_store(k[u], kd + i);
                __builtin_nontemporal_store(v[u], vd + i);
            }
        }
    }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(pa_copy_blocks_kernel, dim3((unsigned)a.num_pairs), dim3(kCopyThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace pa
