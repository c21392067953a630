// merge.hip -- log-sum-exp merge of split-K partitions.
//
// When a context is split into partitions, each (sequence, KV head,
// partition) workgroup leaves for every query head a state (m_p, l_p, o_p)
// over its tokens: m_p the largest score (log2 units), l_p = sum 2^(x - m_p),
// o_p = sum 2^(x - m_p) V. With M = max_p m_p the output is
//     sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,
// which is exactly the softmax-weighted sum of Tutorial
// «大模型推理优化与加速完全教程» §4.4 over the whole context. The pages do
// not describe the split; the partitioned evaluation is the flash-decoding
// form of the tiling TGI «TGI技术解析» §5.2 describes for Flash Attention.
#include "pa_cascade.h"
#include "pa_merge.h"

namespace pa {
namespace {

// One workgroup of 64 * W threads per (sequence, query head) row.
template <int D, int W>
__global__ __launch_bounds__(64 * W) void pa_merge_kernel(MergeArgs a) {
    __shared__ __align__(16) float red[merge_lds_floats<D, W>()];
    const int row = (int)blockIdx.x;  // seq * Hq + q head
    const int seq = row / a.num_q_heads;
    const int head = row - seq * a.num_q_heads;
    int ctx = a.context_lens[seq];
    ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
    const int np = (ctx + a.partition_tokens - 1) / a.partition_tokens;
    if (np <= 1) return;  // the decode kernel stored the output itself
    const float* ml = a.part_ml + (int64_t)row * a.num_partitions * 2;
    const float* po = a.part_o + (int64_t)row * a.num_partitions * D;
    merge_row<D, W>(ml, po, np, nullptr, nullptr, 0, a.out + (int64_t)seq * a.out_seq + (int64_t)head * a.out_head,
                    red);
}

// Few partitions (at most kFlatMergeMaxStates): one thread per (sequence,
// query head, float4 column), 256 threads a workgroup.
template <int D, int NP>
__global__ __launch_bounds__(256) void pa_merge_flat_kernel(MergeArgs a) {
    constexpr int C = D / 4;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / C;  // seq * Hq + q head
    const int c = (int)(gid - row * C);
    if (row >= (int64_t)a.num_seqs * a.num_q_heads) return;
    const int seq = (int)(row / a.num_q_heads);
    const int head = (int)(row - (int64_t)seq * a.num_q_heads);
    int ctx = a.context_lens[seq];
    ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
    const int np = (ctx + a.partition_tokens - 1) / a.partition_tokens;
    if (np <= 1) return;  // the decode kernel stored the output itself
    merge_column<D, NP>(a.part_ml + row * a.num_partitions * 2, a.part_o + row * a.num_partitions * D, np, c,
                        a.out + (int64_t)seq * a.out_seq + (int64_t)head * a.out_head);
}

// Cascade merge: one workgroup per (sequence, query head). A sequence with
// prefix tokens combines the prefix pass's states over them (partitions of
// prefix_partition_tokens) with the suffix pass's states over the rest; a
// sequence without them merges its suffix partitions as pa_merge_kernel
// does, and one with a single unshared partition was finished by the
// suffix pass.
template <int D, int W>
__global__ __launch_bounds__(64 * W) void pa_cascade_merge_kernel(CascadeMergeArgs a) {
    __shared__ __align__(16) float red[merge_lds_floats<D, W>()];
    const int row = (int)blockIdx.x;  // seq * Hq + q head
    const int seq = row / a.num_q_heads;
    const int head = row - seq * a.num_q_heads;
    int ctx = a.context_lens[seq];
    ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
    const int shared = cascade_shared(a.cascade, seq, ctx, a.block_size_log2);
    const int npp = (shared + a.prefix_partition_tokens - 1) / a.prefix_partition_tokens;
    const int nps = (ctx - shared + a.partition_tokens - 1) / a.partition_tokens;
    if (shared == 0 && nps <= 1) return;  // the suffix pass stored the output itself
    merge_row<D, W>(a.pre_ml + (int64_t)row * a.prefix_partitions * 2,
                    a.pre_o + (int64_t)row * a.prefix_partitions * D, npp,
                    a.part_ml + (int64_t)row * a.num_partitions * 2,
                    a.part_o + (int64_t)row * a.num_partitions * D, nps,
                    a.out + (int64_t)seq * a.out_seq + (int64_t)head * a.out_head, red);
}

template <int D, int W>
void launch_w(const MergeArgs& a, int64_t rows, hipStream_t s) {
    hipLaunchKernelGGL((pa_merge_kernel<D, W>), dim3((unsigned)rows), dim3(64 * W), 0, s, a);
}

template <int D, int W>
void launch_w(const CascadeMergeArgs& a, int64_t rows, hipStream_t s) {
    hipLaunchKernelGGL((pa_cascade_merge_kernel<D, W>), dim3((unsigned)rows), dim3(64 * W), 0, s, a);
}

template <int D, class Args>
void launch_rows(const Args& a, int64_t rows, int waves, hipStream_t s) {
    if (waves <= 1) launch_w<D, 1>(a, rows, s);
    else if (waves == 2) launch_w<D, 2>(a, rows, s);
    else if (waves == 4) launch_w<D, 4>(a, rows, s);
    else launch_w<D, 8>(a, rows, s);
}

}  // namespace

hipError_t launch_cascade_merge(const CascadeMergeArgs& a, hipStream_t s) {
    const int64_t rows = (int64_t)a.num_seqs * a.num_q_heads;
    const int w = merge_waves(a.head_dim, (int64_t)a.prefix_partitions + a.num_partitions, rows);
    if (a.head_dim == 64) launch_rows<64>(a, rows, w, s);
    else launch_rows<128>(a, rows, w, s);
    return hipGetLastError();
}

template <int D>
void launch_flat(const MergeArgs& a, int64_t rows, hipStream_t s) {
    const dim3 grid((unsigned)((rows * (D / 4) + 255) / 256));
    const int np = flat_merge_states(a.num_partitions);
    if (np == 2) hipLaunchKernelGGL((pa_merge_flat_kernel<D, 2>), grid, dim3(256), 0, s, a);
    else if (np == 4) hipLaunchKernelGGL((pa_merge_flat_kernel<D, 4>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((pa_merge_flat_kernel<D, 8>), grid, dim3(256), 0, s, a);
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
    const int64_t rows = (int64_t)a.num_seqs * a.num_q_heads;
    if (a.num_partitions <= kFlatMergeMaxStates) {
        if (a.head_dim == 64) launch_flat<64>(a, rows, s);
        else launch_flat<128>(a, rows, s);
        return hipGetLastError();
    }
    const int w = merge_waves(a.head_dim, a.num_partitions, rows);
    if (a.head_dim == 64) launch_rows<64>(a, rows, w, s);
    else launch_rows<128>(a, rows, w, s);
    return hipGetLastError();
}

}  // namespace pa
