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
//      heads; an item carries its token range and whether it stores the
//      final output, so the decode kernel needs no further lookup;
//   4. publish the item count.
// Handing out long items first keeps a long context from starting last and
// stretching the tail (longest-processing-time-first list scheduling). Items
// within a bucket land in an arbitrary order; the result does not depend on
// which workgroup computes an item, so the outputs are still deterministic.
//
// In a cascade call's suffix pass a sequence's pairs start after the tokens
// its prefix group covers (those are attended once for the whole group by
// the prefix pass); a sequence with such tokens gets no pair when nothing
// follows them, and its items never store the final output, which the
// cascade merge forms from both passes' states.
//
// Context lengths are staged through LDS in chunks, so the loops below hold
// no global loads: a load there would make every iteration wait for the
// previous iteration's item stores (both count in the same vmcnt counter).
#include "pa_cascade.h"

namespace pa {
namespace {

constexpr int kBuckets = 1024;
constexpr int kThreads = 1024;
constexpr int kChunk = 4096;  // sequences staged in LDS at a time

__device__ __forceinline__ int pair_key(int len) {
    const int tiles = (len + kTile - 1) / kTile;
    return kBuckets - 1 - min(tiles, kBuckets - 1);  // longer -> smaller key -> earlier
}

// Stage the clamped lengths of sequences [c0, c0 + n) into sctx and the
// token their pairs start at into sbeg (0 unless a cascade prefix covers it).
__device__ __forceinline__ void stage_lengths(const ScheduleArgs& a, int* sctx, int* sbeg, int c0, int n) {
    for (int i = (int)threadIdx.x; i < n; i += kThreads) {
        int ctx = a.context_lens[c0 + i];
        ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
        sctx[i] = ctx;
        sbeg[i] = cascade_shared(a.cascade, c0 + i, ctx, a.block_size_log2);
    }
}

// (sequence, partition) pairs of a sequence whose pairs cover [beg, ctx).
__device__ __forceinline__ int pair_count(int beg, int ctx, int P) {
    const int np = (ctx - beg + P - 1) / P;
    return beg > 0 ? np : max(np, 1);
}

__global__ __launch_bounds__(kThreads) void pa_schedule_kernel(ScheduleArgs a) {
    __shared__ int hist[kBuckets];
    __shared__ int wsum[kThreads / 64];
    __shared__ int sctx[kChunk];
    __shared__ int sbeg[kChunk];
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwaves = kThreads / 64;
    const int P = a.partition_tokens;
    for (int b = tid; b < kBuckets; b += kThreads) hist[b] = 0;

    // 1. histogram of (sequence, partition) pairs; one wave per sequence,
    //    lanes over its partitions
    for (int c0 = 0; c0 < a.num_seqs; c0 += kChunk) {
        const int n = min(kChunk, a.num_seqs - c0);
        stage_lengths(a, sctx, sbeg, c0, n);
        __syncthreads();
        for (int i = wave; i < n; i += nwaves) {
            const int ctx = sctx[i], beg = sbeg[i];
            const int np = pair_count(beg, ctx, P);
            for (int p = lane; p < np; p += 64) atomicAdd(&hist[pair_key(min(P, ctx - beg - p * P))], 1);
        }
        __syncthreads();
    }

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
    }

    // 3. scatter, expanded over KV heads
    for (int c0 = 0; c0 < a.num_seqs; c0 += kChunk) {
        const int n = min(kChunk, a.num_seqs - c0);
        __syncthreads();
        stage_lengths(a, sctx, sbeg, c0, n);
        __syncthreads();
        for (int i = wave; i < n; i += nwaves) {
            const int ctx = sctx[i], beg = sbeg[i];
            const int np = pair_count(beg, ctx, P);
            const int flags = (beg == 0 && (np <= 1 || a.num_partitions == 1)) ? kItemFinal : 0;
            const int Hkv = a.num_kv_heads;
            for (int p0 = 0; p0 < np; p0 += 64) {
                // one slot per pair (lane p0 + lane), then the pair's Hkv items
                // spread over the lanes so that each store instruction writes
                // consecutive items
                const int p = p0 + lane;
                const int len = p < np ? min(P, ctx - beg - p * P) : 0;
                const int pos = p < np ? atomicAdd(&hist[pair_key(len)], 1) : 0;
                const int nitems = min(64, np - p0) * Hkv;
                for (int f0 = 0; f0 < nitems; f0 += 64) {  // uniform trip count: the shuffle sees all lanes
                    const int f = f0 + lane;
                    const int pp = f / Hkv;  // pair within this group of 64
                    const int slot = __shfl(pos, pp < 64 ? pp : 0, 64);
                    if (f < nitems) {
                        const int h = f - pp * Hkv;
                        const int tb = beg + (p0 + pp) * P;
                        a.items[(int64_t)slot * Hkv + h] =
                            make_int4(c0 + i, ((p0 + pp) << 16) | h, tb, min(tb + P, ctx) | flags);
                    }
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(pa_schedule_kernel, dim3(1), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace pa
