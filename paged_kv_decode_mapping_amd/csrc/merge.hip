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
#include "pa_epilogue.h"

namespace pa {
namespace {

template <int D>
__global__ __launch_bounds__(64) void pa_merge_kernel(MergeArgs a) {
    constexpr int PER = D / 64;
    const int row = (int)blockIdx.x;  // seq * Hq + q head
    const int seq = row / a.num_q_heads;
    int ctx = a.context_lens[seq];
    ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
    const int np = (ctx + a.partition_tokens - 1) / a.partition_tokens;
    if (np <= 1) return;  // the decode kernel stored the output itself
    const int lane = (int)threadIdx.x;
    const float* ml = a.part_ml + (int64_t)row * a.num_partitions * 2;
    const float* po = a.part_o + (int64_t)row * a.num_partitions * D + lane * PER;
    float M = -INFINITY;
    for (int p = 0; p < np; ++p) M = fmaxf(M, ml[2 * p]);
    float L = 0.0f;
    float O[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) O[e] = 0.0f;
#pragma unroll 4
    for (int p = 0; p < np; ++p) {
        const float f = state_weight(ml[2 * p], M);
        L = fmaf(ml[2 * p + 1], f, L);
#pragma unroll
        for (int e = 0; e < PER; ++e) O[e] = fmaf(po[(int64_t)p * D + e], f, O[e]);
    }
    uint16_t* dst = a.out + (int64_t)row * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e] = f32_to_bf16_rne(L > 0.0f ? O[e] / L : 0.0f);
}

// Cascade merge: one workgroup per (sequence, query head). A sequence with
// prefix tokens combines the prefix pass's states over them (partitions of
// prefix_partition_tokens) with the suffix pass's states over the rest
// (partitions of partition_tokens; none when nothing follows the prefix).
// A sequence without any is an ordinary decode row: merged here only when
// its context was split, as in pa_merge_kernel.
template <int D>
__global__ __launch_bounds__(64) void pa_cascade_merge_kernel(CascadeMergeArgs a) {
    constexpr int PER = D / 64;
    const int row = (int)blockIdx.x;  // seq * Hq + q head
    const int seq = row / a.num_q_heads;
    int ctx = a.context_lens[seq];
    ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
    const int shared = cascade_shared(a.cascade, seq, ctx, a.block_size_log2);
    const int npp = (shared + a.prefix_partition_tokens - 1) / a.prefix_partition_tokens;
    const int nps = (ctx - shared + a.partition_tokens - 1) / a.partition_tokens;
    if (shared == 0 && nps <= 1) return;  // the suffix pass stored the output itself
    const int lane = (int)threadIdx.x;
    const float* pml = a.pre_ml + (int64_t)row * a.prefix_partitions * 2;
    const float* pmo = a.pre_o + (int64_t)row * a.prefix_partitions * D + lane * PER;
    const float* sml = a.part_ml + (int64_t)row * a.num_partitions * 2;
    const float* smo = a.part_o + (int64_t)row * a.num_partitions * D + lane * PER;
    float M = -INFINITY;
    for (int p = 0; p < npp; ++p) M = fmaxf(M, pml[2 * p]);
    for (int p = 0; p < nps; ++p) M = fmaxf(M, sml[2 * p]);
    float L = 0.0f;
    float O[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) O[e] = 0.0f;
    for (int p = 0; p < npp; ++p) {
        const float f = state_weight(pml[2 * p], M);
        L = fmaf(pml[2 * p + 1], f, L);
#pragma unroll
        for (int e = 0; e < PER; ++e) O[e] = fmaf(pmo[(int64_t)p * D + e], f, O[e]);
    }
    for (int p = 0; p < nps; ++p) {
        const float f = state_weight(sml[2 * p], M);
        L = fmaf(sml[2 * p + 1], f, L);
#pragma unroll
        for (int e = 0; e < PER; ++e) O[e] = fmaf(smo[(int64_t)p * D + e], f, O[e]);
    }
    uint16_t* dst = a.out + (int64_t)row * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e] = f32_to_bf16_rne(L > 0.0f ? O[e] / L : 0.0f);
}

}  // namespace

hipError_t launch_cascade_merge(const CascadeMergeArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)a.num_seqs * a.num_q_heads));
    if (a.head_dim == 64) hipLaunchKernelGGL(pa_cascade_merge_kernel<64>, grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL(pa_cascade_merge_kernel<128>, grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)a.num_seqs * a.num_q_heads));
    if (a.head_dim == 64) hipLaunchKernelGGL(pa_merge_kernel<64>, grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL(pa_merge_kernel<128>, grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace pa
