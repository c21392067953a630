// decode_valu.hip -- paged decode attention with the dot products on the
// vector ALUs; the kernel for small GQA groups (MHA and g = 2), where a
// 16-row matrix tile would be mostly padding.
//
// Pages cited (titles as printed at the top of each page):
//   Tutorial = «大模型推理优化与加速完全教程» (LLM inference optimisation tutorial)
//   nanoVLLM = «大模型推理优化技术：从nano-vLLM到连续批处理»
//
// What it computes: for every (sequence, KV head, partition) workgroup, the
// softmax(q.K^T * scale).V of Tutorial §4.4 (GroupedQueryAttention.forward)
// for the g query heads that read that KV head, over K/V rows gathered
// through the block table as in Tutorial §4.2 (PagedKVCache.get_kv) --
// the "second-level addressing" nanoVLLM §4.2 says standard attention
// kernels lack.
//
// Mapping to gfx950:
//   * A token row of one KV head (D elements) is covered by LPR lanes, each
//     holding one 16-byte chunk; one buffer_load_dwordx4 per lane brings
//     RPI = 64 / LPR whole rows, so every load instruction reads complete
//     256-byte (bf16, D = 128) rows: full cache lines, no partial sectors.
//   * The partial dot product of each lane is summed over its row's LPR
//     lanes with four DPP adds (quad_perm, quad_perm, row_half_mirror,
//     row_mirror), leaving the score in every lane of the row.
//   * Each row position of the wave keeps its own online-softmax state (m,
//     l, o) over the tokens it sees, so the tile loop needs no cross-row
//     exchange; the RPI states are combined once, after the loop.
//   * The block id of a 16-token tile is wave-uniform (block_size >= 16),
//     fetched one tile ahead, and becomes the base of a buffer resource
//     limited to that block.
//   * Each wave keeps a ring of NB tiles in registers: the loads of tile
//     t + (NB - 1) W are issued before tile t is consumed.
//   * g <= 4 only (the plan sends larger groups to the MFMA kernel).
#include "pa_epilogue.h"

namespace pa {
namespace {

template <bool FP8, int EPL>
__device__ __forceinline__ void unpack(const u32x4& w, float (&f)[EPL]) {
    if constexpr (!FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16_lo(w[i]);
            f[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
            f[4 * i] = lo[0];
            f[4 * i + 1] = lo[1];
            f[4 * i + 2] = hi[0];
            f[4 * i + 3] = hi[1];
        }
    }
}

template <int D, bool FP8, int GM, int NB>
__global__ __launch_bounds__(512) void pa_decode_valu_kernel(DecodeArgs a) {
    constexpr int ESZ = FP8 ? 1 : 2;
    constexpr int EPL = 16 / ESZ;    // elements per lane per 16-byte load
    constexpr int LPR = D / EPL;     // lanes per token row
    constexpr int RPI = 64 / LPR;    // token rows per load instruction
    constexpr int NI = kTile / RPI;  // load instructions per 16-token tile
    static_assert(NI >= 1 && kTile % RPI == 0, "tile shape");

    extern __shared__ float smem[];
    for_each_item(a, reinterpret_cast<int*>(smem), [&](const WorkItem& wi) {
        const int W = (int)(blockDim.x >> 6);
        const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        const int lane = (int)(threadIdx.x & 63);
        const int r_in = lane / LPR;
        const int c = lane % LPR;
        const int g = a.group;

        // q for this lane's EPL dims of each head of the group, as float.
        float qf[GM][EPL];
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            if (h < g) {
                const uint16_t* qp = a.q + (int64_t)wi.seq * a.q_seq + (int64_t)(wi.kvh * g + h) * a.q_head + c * EPL;
#pragma unroll
                for (int e = 0; e < EPL; e += 8) {
                    const u32x4 w = *reinterpret_cast<const u32x4*>(qp + e);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        qf[h][e + 2 * i] = bf16_lo(w[i]);
                        qf[h][e + 2 * i + 1] = bf16_hi(w[i]);
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e) qf[h][e] = 0.0f;
            }
        }

        float m[GM], l[GM], o[GM][EPL];
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            m[h] = -INFINITY;
            l[h] = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[h][e] = 0.0f;
        }

        const int span = wi.t_end - wi.t_begin;
        const int ntiles = span > 0 ? (span + kTile - 1) / kTile : 0;
        // per-lane byte offsets inside a tile, fixed for the whole item; the
        // KV head is folded into each tile's descriptor base
        uint32_t lane_off[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) lane_off[i] = (uint32_t)(i * RPI + r_in) * a.cache.token + (uint32_t)c * 16u;
        const int64_t head_off = (int64_t)wi.kvh * a.cache.head;
        const int bs_mask = (1 << a.block_size_log2) - 1;
        const float qk = a.qk_scale_log2;

        u32x4 kb[NB][NI], vb[NB][NI];  // ring of NB tiles: NB - 1 in flight while one is consumed

        // Loads for tile t. A tile past the end (the prefetch after the last
        // one) still issues its loads, against a zero-byte buffer: they return
        // zeros without touching memory, and every path through the loop keeps
        // the same number of loads in flight, so the wait before a tile's use
        // never has to drain the prefetch behind it.
        auto issue = [&](int t, int64_t blk, u32x4 (&kb)[NI], u32x4 (&vb)[NI]) {
            const bool live = t < ntiles;
            const int t0 = wi.t_begin + (live ? t : ntiles - 1) * kTile;
            const uint32_t row0 = (uint32_t)(t0 & bs_mask);
            // the descriptor ends at the tile's last valid row: rows past the
            // context read as zero, so V needs no masking code
            const int valid = min(wi.t_end - t0, kTile);
            const uint32_t nbytes = live ? (row0 + (uint32_t)valid) * a.cache.token : 0u;
            const int64_t base = blk * a.cache.block + head_off;
            const auto rk = make_rsrc(a.k_cache + base, nbytes);
            const auto rv = make_rsrc(a.v_cache + base, nbytes);
            const uint32_t soff = row0 * a.cache.token;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                kb[i] = buf_load_b128_stream(rk, lane_off[i], soff);
                vb[i] = buf_load_b128_stream(rv, lane_off[i], soff);
            }
        };

        auto consume = [&](int t, const u32x4 (&kb)[NI], const u32x4 (&vb)[NI]) {
            const int t0 = wi.t_begin + t * kTile;
            const int valid = wi.t_end - t0;
            const bool full = valid >= kTile;
            float x[NI][GM];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                float kf[EPL];
                unpack<FP8, EPL>(kb[i], kf);
                const bool dead = !full && (i * RPI + r_in) >= valid;
#pragma unroll
                for (int h = 0; h < GM; ++h) {
                    float s = 0.0f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) s = fmaf(qf[h][e], kf[e], s);
                    s = group_sum<LPR>(s);
                    x[i][h] = dead ? -INFINITY : s * qk;
                }
            }
            float p[NI][GM];
#pragma unroll
            for (int h = 0; h < GM; ++h) {
                float mx = x[0][h];
#pragma unroll
                for (int i = 1; i < NI; ++i) mx = fmaxf(mx, x[i][h]);
                const float m_new = fmaxf(m[h], mx);
                const float ms = (m_new == -INFINITY) ? 0.0f : m_new;
                const float alpha = fast_exp2(m[h] - ms);
                m[h] = m_new;
                float lsum = 0.0f;
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    p[i][h] = fast_exp2(x[i][h] - ms);
                    lsum += p[i][h];
                }
                l[h] = fmaf(l[h], alpha, lsum);
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
            }
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                float vf[EPL];
                unpack<FP8, EPL>(vb[i], vf);
#pragma unroll
                for (int h = 0; h < GM; ++h) {
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(p[i][h], vf[e], o[h][e]);
                }
            }
        };

        if (ntiles > 0) {
            // The ring is unrolled so that every buffer index is a constant.
            // Each step issues the loads NB - 1 tiles ahead unconditionally
            // (past the end they are zero-byte no-ops) and consumes one tile
            // behind a uniform branch, so every path through the loop keeps
            // the same loads in flight and the waits before a tile's use
            // leave the prefetch behind it outstanding. sched_barrier keeps
            // the compiler from sinking the prefetch below those waits.
            // The table entry of each issued tile was fetched one step earlier.
            const TableReader tab = make_table_reader(a, wi, ntiles - 1);
            uint32_t entry = table_fetch(tab, wave);
#pragma unroll
            for (int b = 0; b < NB - 1; ++b) {
                const int64_t blk = table_block(tab, entry);
                entry = table_fetch(tab, wave + (b + 1) * W);
                __builtin_amdgcn_sched_barrier(0);
                issue(wave + b * W, blk, kb[b], vb[b]);
            }
            for (int t = wave; t < ntiles; t += NB * W) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int ti = t + (b + NB - 1) * W;
                    const int64_t blk = table_block(tab, entry);
                    entry = table_fetch(tab, ti + W);
                    __builtin_amdgcn_sched_barrier(0);
                    issue(ti, blk, kb[(b + NB - 1) % NB], vb[(b + NB - 1) % NB]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (t + b * W < ntiles) consume(t + b * W, kb[b], vb[b]);
                }
            }
        }

        // Combine the RPI row states of the wave (lanes differing in row bits).
        float* sm_ml = smem;
        float* sm_o = smem + W * g * 2;
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            float M = m[h];
#pragma unroll
            for (int mask = LPR; mask < 64; mask <<= 1) M = fmaxf(M, xor_shfl(M, mask));
            const float f = state_weight(m[h], M);
            float lh = l[h] * f;
#pragma unroll
            for (int mask = LPR; mask < 64; mask <<= 1) lh += xor_shfl(lh, mask);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float v = o[h][e] * f;
#pragma unroll
                for (int mask = LPR; mask < 64; mask <<= 1) v += xor_shfl(v, mask);
                o[h][e] = v;
            }
            if (h < g) {
                if (lane == 0) {
                    sm_ml[(wave * g + h) * 2] = M;
                    sm_ml[(wave * g + h) * 2 + 1] = lh;
                }
                if (r_in == 0) {
#pragma unroll
                    for (int e = 0; e < EPL; ++e) sm_o[(wave * g + h) * D + c * EPL + e] = o[h][e];
                }
            }
        }
        __syncthreads();
        combine_and_store<D>(a, sm_ml, sm_o, W, g, wi.seq, wi.kvh, wi.part, wi.final_out);
    });
}

template <int D, bool FP8, int GM, int NB>
hipError_t launch_k(const DecodeArgs& a, const LaunchShape& ls, hipStream_t s) {
    const dim3 block((unsigned)(64 * ls.waves));
    const size_t comb = (size_t)ls.waves * a.group * (D + 2) * sizeof(float);
    const size_t lds = comb > kSelfLdsInts * sizeof(int) ? comb : kSelfLdsInts * sizeof(int);
    const dim3 grid((unsigned)((int64_t)a.num_seqs * a.units_per_seq * a.num_items));
    hipLaunchKernelGGL((pa_decode_valu_kernel<D, FP8, GM, NB>), grid, block, lds, s, a);
    return hipGetLastError();
}

template <int D, bool FP8, int GM>
hipError_t launch_g(const DecodeArgs& a, const LaunchShape& ls, hipStream_t s) {
    if (ls.depth <= 2) return launch_k<D, FP8, GM, 2>(a, ls, s);
    if (ls.depth == 3) return launch_k<D, FP8, GM, 3>(a, ls, s);
    return launch_k<D, FP8, GM, 4>(a, ls, s);
}

template <int D, bool FP8>
hipError_t launch_d(const DecodeArgs& a, const LaunchShape& ls, hipStream_t s) {
    if (a.group <= 1) return launch_g<D, FP8, 1>(a, ls, s);
    if (a.group <= 2) return launch_g<D, FP8, 2>(a, ls, s);
    return launch_g<D, FP8, 4>(a, ls, s);
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs& a, int head_dim, bool fp8, const LaunchShape& ls, hipStream_t s) {
    if (head_dim == 64) return fp8 ? launch_d<64, true>(a, ls, s) : launch_d<64, false>(a, ls, s);
    return fp8 ? launch_d<128, true>(a, ls, s) : launch_d<128, false>(a, ls, s);
}

}  // namespace pa
