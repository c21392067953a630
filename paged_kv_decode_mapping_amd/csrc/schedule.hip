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
// Parallel over (sequence, partition) pairs, not over sequences: the
// lengths of a chunk of sequences are staged in LDS with one thread per four
// sequences, a block-wide scan numbers their pairs, and then one thread per
// pair counts and places it (a binary search over the scanned offsets finds
// its sequence). A loop with one sequence per wave and iteration, the
// simpler form, cost about 1 µs per iteration on MI355X (19 µs for 256
// sequences); here a batch of up to 1024 pairs takes one pass.
#include "pa_cascade.h"

namespace pa {
namespace {

constexpr int kBuckets = 1024;
constexpr int kThreads = 1024;
constexpr int kPerThread = 4;
constexpr int kChunk = kThreads * kPerThread;  // sequences staged in LDS at a time

__device__ __forceinline__ int pair_key(int len) {
    const int tiles = (len + kTile - 1) / kTile;
    return kBuckets - 1 - min(tiles, kBuckets - 1);  // longer -> smaller key -> earlier
}

// (sequence, partition) pairs of a sequence whose pairs cover [beg, ctx).
__device__ __forceinline__ int pair_count(int beg, int ctx, int P) {
    const int np = (ctx - beg + P - 1) / P;
    return beg > 0 ? np : max(np, 1);
}

struct Chunk {
    int* ctx;   // [kChunk] clamped context lengths
    int* beg;   // [kChunk] first token of the sequence's pairs
    int* off;   // [kChunk] first pair of each sequence (exclusive scan of the pair counts)
    int* wsum;  // [kThreads / 64] scratch of the scan
    int* total; // pairs of the chunk
};

// Stage sequences [c0, c0 + n) (thread t: sequences 4t .. 4t + 3 of the
// chunk) and number their pairs. Ends with a barrier.
__device__ __forceinline__ void stage_chunk(const ScheduleArgs& a, const Chunk& ch, int c0, int n) {
    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int cnt[kPerThread];
    int local = 0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int j = tid * kPerThread + k;
        cnt[k] = 0;
        if (j < n) {
            int ctx = a.context_lens[c0 + j];
            ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
            const int beg = cascade_shared(a.cascade, c0 + j, ctx, a.block_size_log2);
            ch.ctx[j] = ctx;
            ch.beg[j] = beg;
            cnt[k] = pair_count(beg, ctx, a.partition_tokens);
        }
        local += cnt[k];
    }
    int x = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) ch.wsum[wave] = x;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += ch.wsum[w];
    int run = base + x - local;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int j = tid * kPerThread + k;
        if (j < n) ch.off[j] = run;
        run += cnt[k];
    }
    if (tid == kThreads - 1) *ch.total = base + x;
    __syncthreads();
}

// Sequence (within the chunk) of pair f: the last j with off[j] <= f.
__device__ __forceinline__ int pair_seq(const int* off, int n, int f) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= f) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(kThreads) void pa_schedule_kernel(ScheduleArgs a) {
    __shared__ int hist[kBuckets];
    __shared__ int wsum[kThreads / 64];
    __shared__ int sctx[kChunk], sbeg[kChunk], soff[kChunk];
    __shared__ int stotal;
    const Chunk ch{sctx, sbeg, soff, wsum, &stotal};
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int P = a.partition_tokens;
    const int Hkv = a.num_kv_heads;
    const int nchunks = (a.num_seqs + kChunk - 1) / kChunk;
    static_assert(kBuckets == kThreads, "one bucket per thread");
    hist[tid] = 0;

    // 1. histogram of (sequence, partition) pairs, one thread per pair
    for (int c = 0; c < nchunks; ++c) {
        const int c0 = c * kChunk, n = min(kChunk, a.num_seqs - c0);
        __syncthreads();  // the previous chunk's readers are done (and hist is zeroed)
        stage_chunk(a, ch, c0, n);
        const int pairs = stotal;
        for (int f = tid; f < pairs; f += kThreads) {
            const int j = pair_seq(soff, n, f);
            const int p = f - soff[j];
            atomicAdd(&hist[pair_key(min(P, sctx[j] - sbeg[j] - p * P))], 1);
        }
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
    if (tid == kThreads - 1) *a.item_count = (base + x) * Hkv;

    // 3. place each pair at its bucket's next slot, expanded over the KV heads
    for (int c = 0; c < nchunks; ++c) {
        const int c0 = c * kChunk, n = min(kChunk, a.num_seqs - c0);
        __syncthreads();  // bucket offsets published; the previous chunk's readers are done
        if (nchunks > 1) stage_chunk(a, ch, c0, n);  // a single chunk is still staged
        const int pairs = stotal;
        for (int f = tid; f < pairs; f += kThreads) {
            const int j = pair_seq(soff, n, f);
            const int p = f - soff[j];
            const int ctx = sctx[j], beg = sbeg[j];
            const int pos = atomicAdd(&hist[pair_key(min(P, ctx - beg - p * P))], 1);
            const int nsplit = (ctx - beg + a.split_tokens - 1) / a.split_tokens;
            const int flags = (beg == 0 && (nsplit <= 1 || a.split_count == 1)) ? kItemFinal : 0;
            const int tb = beg + p * P;
            const int4 rec = make_int4(c0 + j, p << 16, tb, min(tb + P, ctx) | flags);
            int4* dst = a.items + (int64_t)pos * Hkv;
            for (int h = 0; h < Hkv; ++h) dst[h] = make_int4(rec.x, rec.y | h, rec.z, rec.w);
        }
    }
}

}  // namespace

hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(pa_schedule_kernel, dim3(1), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace pa
