// schedule.hip -- build the decode work list on the device, longest first.
//
// A decode step's work is a set of items (sequence, KV head, partition),
// each the online softmax over one partition's tokens (the per-partition
// states are merged by log-sum-exp afterwards). Context lengths live on the
// device, so the host cannot size or order this set without a
// synchronisation. This kernel (one workgroup) does it in place:
//   1. count every (sequence, partition) pair into a bucket by its number of
//      16-token tiles, largest first (a sequence of length 0 still gets one
//      pair: its output row must be written, as zeros);
//   2. prefix-sum the buckets;
//   3. place each pair at its bucket's next slot and expand it over the KV
//      heads;
//   4. publish the item count and reset the queue counter the persistent
//      decode workgroups pull from.
// Handing out long items first keeps a long context from starting last and
// stretching the tail (longest-processing-time-first list scheduling). Items
// within a bucket land in an arbitrary order; the result does not depend on
// which workgroup computes an item, so the outputs are still deterministic.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kBuckets = 1024;
constexpr int kThreads = 1024;

__device__ __forceinline__ int pair_key(int len) {
    const int tiles = (len + kTile - 1) / kTile;
    return kBuckets - 1 - min(tiles, kBuckets - 1);  // longer -> smaller key -> earlier
}

__global__ __launch_bounds__(kThreads) void pa_schedule_kernel(ScheduleArgs a) {
    __shared__ int hist[kBuckets];
    __shared__ int wsum[kThreads / 64];
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwaves = kThreads / 64;
    const int P = a.partition_tokens;
    for (int b = tid; b < kBuckets; b += kThreads) hist[b] = 0;
    __syncthreads();

    // 1. histogram of (sequence, partition) pairs; one wave per sequence
    for (int i = wave; i < a.num_seqs; i += nwaves) {
        int ctx = a.context_lens[i];
        ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
        const int np = max((ctx + P - 1) / P, 1);
        for (int p = lane; p < np; p += 64) atomicAdd(&hist[pair_key(min(P, ctx - p * P))], 1);
    }
    __syncthreads();

    // 2. exclusive prefix sum over the buckets (one bucket per thread)
    const int mine = hist[tid];
    int x = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    __syncthreads();
    hist[tid] = base + x - mine;  // now: next free slot of the bucket
    if (tid == kThreads - 1) {
        *a.item_count = (base + x) * a.num_kv_heads;
        *a.queue = 0;
    }
    __syncthreads();

    // 3. scatter, expanded over KV heads
    for (int i = wave; i < a.num_seqs; i += nwaves) {
        int ctx = a.context_lens[i];
        ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
        const int np = max((ctx + P - 1) / P, 1);
        for (int p = lane; p < np; p += 64) {
            const int pos = atomicAdd(&hist[pair_key(min(P, ctx - p * P))], 1);
            for (int h = 0; h < a.num_kv_heads; ++h)
                a.items[(int64_t)pos * a.num_kv_heads + h] = make_int2(i, (p << 16) | h);
        }
    }
}

}  // namespace

hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(pa_schedule_kernel, dim3(1), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace pa
