// pa_merge.h -- log-sum-exp merge of one output row's partial states by a
// whole workgroup.
//
// A state (m, l, o) over a token subset is the max score m (log2 units),
// l = sum 2^(x - m) and o = sum 2^(x - m) V over that subset; with M = max m
// over all states the row's output is sum 2^(m - M) o / sum 2^(m - M) l,
// the softmax-weighted sum of Tutorial «大模型推理优化与加速完全教程» §4.4
// over the union of the subsets.
//
// The merge is latency bound: a row has a few to a few hundred states of
// D + 2 floats. So every step issues all its loads at once instead of
// walking the states one by one: the 64 * W threads first read the m's
// spread over all threads (one round trip for up to 64 * W states), then
// thread t accumulates float4 column t % (D/4) of every G-th state starting
// at t / (D/4) (G = 64 * W / (D/4) groups, four states per group unrolled),
// and the groups' sums meet by shuffles inside a wave and through LDS
// across waves.
#pragma once

#include "pa_epilogue.h"

namespace pa {

// Waves per merge workgroup for `rows` rows of at most n states each: the
// fewest that keep all n states' loads of a row in flight in one unrolled
// pass (four per group), at most 8, and no more once the rows alone give
// about four waves per SIMD: then other rows hide the latency and wider
// groups only add barriers (measured: 8192 rows of 9 states, 2 waves 11.7
// us, 1 wave 10.3 us).
inline int merge_waves(int head_dim, int64_t n, int64_t rows) {
    int w = 1;
    while (w < 8 && (int64_t)4 * (64 * w / (head_dim / 4)) < n && rows * w * 2 <= 4096) w *= 2;
    return w;
}

// LDS floats merge_row<D, W> needs.
template <int D, int W>
constexpr int merge_lds_floats() { return W * (D + 4); }

// Merge n0 states (ml0 [n0][2] = (m, l), o0 [n0][D]) followed by n1 states
// (ml1, o1) into dst[0..D) as bf16 (round to nearest even); zeros when every
// state is empty (l sums to 0). Rows of o must be 16-byte aligned and rows
// of ml 8-byte aligned. Every thread of the 64 * W-thread workgroup calls it
// with the same arguments; red is LDS of merge_lds_floats<D, W>() floats.
template <int D, int W>
__device__ __forceinline__ void merge_row(const float* ml0, const float* o0, int n0, const float* ml1,
                                          const float* o1, int n1, uint16_t* dst, float* red) {
    constexpr int C = D / 4;      // float4 columns of a row
    constexpr int T = 64 * W;     // threads
    constexpr int G = T / C;      // state groups
    static_assert(D % 4 == 0 && 64 % C == 0, "a wave holds whole rows of float4 columns");
    const int t = (int)threadIdx.x, lane = t & 63, wave = t >> 6;
    const int n = n0 + n1;

    float M = -INFINITY;
    for (int s = t; s < n; s += T) M = fmaxf(M, s < n0 ? ml0[2 * s] : ml1[2 * (s - n0)]);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d, 64));
    if constexpr (W > 1) {
        if (lane == 0) red[wave] = M;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, red[w]);
        __syncthreads();  // red is rewritten below
    }

    const int c = t % C;
    float L = 0.0f, ox = 0.0f, oy = 0.0f, oz = 0.0f, ow = 0.0f;
#pragma unroll 4
    for (int s = t / C; s < n; s += G) {
        const bool first = s < n0;
        const float2 st = first ? *reinterpret_cast<const float2*>(ml0 + 2 * s)
                                : *reinterpret_cast<const float2*>(ml1 + 2 * (s - n0));
        const float4 v = first ? *reinterpret_cast<const float4*>(o0 + (int64_t)s * D + 4 * c)
                               : *reinterpret_cast<const float4*>(o1 + (int64_t)(s - n0) * D + 4 * c);
        const float f = state_weight(st.x, M);
        L = fmaf(st.y, f, L);
        ox = fmaf(v.x, f, ox);
        oy = fmaf(v.y, f, oy);
        oz = fmaf(v.z, f, oz);
        ow = fmaf(v.w, f, ow);
    }
#pragma unroll
    for (int d = C; d < 64; d <<= 1) {
        L += __shfl_xor(L, d, 64);
        ox += __shfl_xor(ox, d, 64);
        oy += __shfl_xor(oy, d, 64);
        oz += __shfl_xor(oz, d, 64);
        ow += __shfl_xor(ow, d, 64);
    }
    if constexpr (W > 1) {
        float* mine = red + wave * (D + 4);
        if (lane < C) *reinterpret_cast<float4*>(mine + 4 * lane) = make_float4(ox, oy, oz, ow);
        if (lane == 0) mine[D] = L;
        __syncthreads();
        if (t < C) {
            L = 0.0f;
            ox = oy = oz = ow = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float4 v = *reinterpret_cast<const float4*>(red + w * (D + 4) + 4 * t);
                L += red[w * (D + 4) + D];
                ox += v.x;
                oy += v.y;
                oz += v.z;
                ow += v.w;
            }
        }
    }
    if (t < C) {
        const bool live = L > 0.0f;
        uint2 packed;
        packed.x = (uint32_t)f32_to_bf16_rne(live ? ox / L : 0.0f) | ((uint32_t)f32_to_bf16_rne(live ? oy / L : 0.0f) << 16);
        packed.y = (uint32_t)f32_to_bf16_rne(live ? oz / L : 0.0f) | ((uint32_t)f32_to_bf16_rne(live ? ow / L : 0.0f) << 16);
        *reinterpret_cast<uint2*>(dst + 4 * c) = packed;
    }
}

// Rows with few states (at most NP): one thread per (row, float4 column)
// instead of a workgroup per row. A thread issues the loads of all the
// row's states at once -- every (m, l) and its column of every o -- so a
// row costs one memory round trip, and the C = D / 4 threads of a row each
// compute the same M and L. States are summed in order 0..n-1. With one
// workgroup per row the merge of hundreds of thousands of rows with 2
// states (32 query tokens per sequence on the mixed batch: 262,144 rows)
// was bound by that per-row latency: 142 us.
constexpr int kFlatMergeMaxStates = 8;

template <int D, int NP>
__device__ __forceinline__ void merge_column(const float* ml, const float* o, int n, int c, uint16_t* dst) {
    float m[NP], l[NP];
    float4 v[NP];
#pragma unroll
    for (int s = 0; s < NP; ++s) {
        m[s] = -INFINITY;
        l[s] = 0.0f;
        v[s] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (s < n) {
            const float2 st = *reinterpret_cast<const float2*>(ml + 2 * s);
            m[s] = st.x;
            l[s] = st.y;
            v[s] = *reinterpret_cast<const float4*>(o + (int64_t)s * D + 4 * c);
        }
    }
    float M = m[0];
#pragma unroll
    for (int s = 1; s < NP; ++s) M = fmaxf(M, m[s]);
    float L = 0.0f, ox = 0.0f, oy = 0.0f, oz = 0.0f, ow = 0.0f;
#pragma unroll
    for (int s = 0; s < NP; ++s) {
        const float f = state_weight(m[s], M);
        L = fmaf(l[s], f, L);
        ox = fmaf(v[s].x, f, ox);
        oy = fmaf(v[s].y, f, oy);
        oz = fmaf(v[s].z, f, oz);
        ow = fmaf(v[s].w, f, ow);
    }
    const bool live = L > 0.0f;
    uint2 packed;
    packed.x = (uint32_t)f32_to_bf16_rne(live ? ox / L : 0.0f) | ((uint32_t)f32_to_bf16_rne(live ? oy / L : 0.0f) << 16);
    packed.y = (uint32_t)f32_to_bf16_rne(live ? oz / L : 0.0f) | ((uint32_t)f32_to_bf16_rne(live ? ow / L : 0.0f) << 16);
    *reinterpret_cast<uint2*>(dst + 4 * c) = packed;
}

// Smallest unrolled state count of merge_column covering n states (n <= 8).
inline int flat_merge_states(int64_t n) { return n <= 2 ? 2 : (n <= 4 ? 4 : 8); }

}  // namespace pa
