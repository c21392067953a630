// decode_mfma.hip -- paged decode attention with q.K^T and P.V on the
// matrix cores; the kernel for GQA groups (g >= 4 query heads per KV head).
//
// Pages cited (titles as printed at the top of each page):
//   Tutorial = «大模型推理优化与加速完全教程» (LLM inference optimisation tutorial)
//   nanoVLLM = «大模型推理优化技术：从nano-vLLM到连续批处理»
//   ToPG     = «ToPG框架解析：大模型推理性能优化与三阶段流水线设计»
//
// What it computes: the same as the VALU kernel -- for the g query heads of
// one KV head (Tutorial §4.4, GroupedQueryAttention: the heads of a group
// share one K/V), softmax(q.K^T * scale).V over K/V rows reached through the
// block table (Tutorial §4.2, get_kv; nanoVLLM §4.2). With g query rows
// against a 16-token tile, q.K^T is a [g x D] x [D x 16] product and P.V a
// [g x 16] x [16 x D] one: real dense contractions, so they run as bf16
// MFMA with fp32 accumulation (ToPG §2: FP32 accumulation).
//
// Layout of one 16-token tile in a wave (lane l, c = l % 16, gq = l / 16):
//   * K and V rows go HBM -> registers -> LDS with 16-byte non-temporal
//     buffer loads in which every instruction covers whole 256-byte rows
//     (bf16, D = 128): the cache is read exactly once, as full lines. Loading
//     K straight into the MFMA operand layout instead (16 rows x 64 bytes
//     per instruction) was measured at ~70 % of peak against ~79 % this way.
//   * S = K Q^T by v_mfma_f32_16x16x32_bf16, D/32 times: the A operand is K
//     (row = token c, eight d values of chunk gq) read back from LDS; B is
//     Q^T (column = head c), kept in registers. Lane l receives
//     S[token 4*gq + r][head c], r = 0..3.
//   * The online softmax of head c needs the tile max over the four lane
//     groups: two cross-lane exchanges per tile.
//   * O^T = V^T P^T by v_mfma_f32_16x16x16_bf16, D/16 times: B is P^T
//     (token 4*gq + r, head c) -- exactly the lane's own four probabilities,
//     rounded to bf16 -- and A is V^T (row = d, token 4*gq + r), read from
//     the LDS copy with gfx950's transposing LDS load. Lane l accumulates
//     O[d = 16 j + 4 gq + r][head c], so the softmax rescale of head c stays
//     in-lane. The softmax denominator is one more such MFMA with A = ones:
//     every element of its tile is the column's sum of the same rounded
//     probabilities over all 16 tokens, with no VALU adds or cross-lane
//     sums (measured on fp8 caches, where the SIMDs' issue is the limit).
//   * fp8 caches: codes are widened to bf16 exactly (every e4m3fn value is a
//     bf16 value) with v_cvt_scalef32_pk_bf16_fp8 while staging; the scales
//     are folded into the score scale and the output.
//   * Each wave keeps a ring of NB tiles in registers: NB - 1 tiles are in
//     flight while one is consumed (the same scheme as the VALU kernel).
#include "pa_epilogue.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// 16 fp8 codes -> 16 bf16 (two 8-element halves), exact.
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4& w, u32x4& lo, u32x4& hi) {
    uint32_t r[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false);
        const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true);
        r[2 * i] = __builtin_bit_cast(uint32_t, a);
        r[2 * i + 1] = __builtin_bit_cast(uint32_t, b);
    }
    lo = u32x4{r[0], r[1], r[2], r[3]};
    hi = u32x4{r[4], r[5], r[6], r[7]};
}

// Occupancy the register allocator is asked to keep: 4 waves per SIMD (<= 128
// VGPRs) for the ring of 2 tiles, 3 (<= 168) for 3 tiles, 2 for 4 tiles; the
// bf16 kernel with packed heads keeps a per-head P.V path for non-finite V
// (about 35 more registers) and gets one wave per SIMD less.
template <int NB, int HP, bool FP8>
constexpr int mfma_waves_per_eu() {
    const int base = NB <= 2 ? 4 : (NB == 3 ? 3 : 2);
    return (HP > 1 && !FP8 && base > 2) ? base - 1 : base;
}

// WPP: each wave takes one whole partition of the item (wave w: partition
// item * W + w) and stores that partition's state itself; otherwise the
// waves share the item's tiles round robin and combine their states in LDS.
template <int D, bool FP8, int NB, int HP, bool WPP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(mfma_waves_per_eu<NB, HP, FP8>())))
void pa_decode_mfma_kernel(DecodeArgs a) {
    constexpr int ESZ = FP8 ? 1 : 2;
    constexpr int NQK = D / 32;         // q.K^T MFMAs per tile
    constexpr int NPV = D / 16;         // P.V MFMAs per tile
    constexpr int EPL = 16 / ESZ;       // elements per 16-byte lane load
    constexpr int LPR = D / EPL;        // lanes per KV head row
    // A tile is 16 MFMA rows: TPH tokens of each of HP adjacent KV heads
    // (row = head * TPH + token); their rows are HP * D contiguous elements
    // in the cache, so each token contributes one contiguous chunk.
    constexpr int TPH = kTile / HP;     // tokens per tile
    constexpr int LPC = HP * LPR;       // lanes per token chunk (HP heads)
    constexpr int RPI = 64 / LPC;       // tokens per load instruction
    constexpr int NI = TPH / RPI;       // loads per lane per tile, for each of K and V
    constexpr int RS = D + 8;           // LDS row stride (bf16 elements): +16 bytes per row
    static_assert(LPC <= 64 && NI >= 1 && TPH % RPI == 0, "tile shape");

    extern __shared__ float smem[];
    for_each_item(a, reinterpret_cast<int*>(smem), [&](const WorkItem& wi) {
        const int W = (int)(blockDim.x >> 6);
        const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        const int lane = (int)(threadIdx.x & 63);
        const int c = lane & 15;
        const int gq = lane >> 4;
        const int g = a.group;
        const int kvh0 = wi.kvh * HP;  // first KV head of this unit
        uint16_t* vs = reinterpret_cast<uint16_t*>(smem) + wave * 2 * kTile * RS;  // V tile
        uint16_t* ks = vs + kTile * RS;                                               // K tile
        const uint16_t* tr_base = vs + (4 * gq + (c >> 2)) * RS + 4 * (lane & 3);

        // Q^T operands: MFMA j takes d = 32 j + 8 gq + 0..7 of column c, the
        // d range of the lane's K operand of MFMA j. Column c is query head
        // c % TPH of KV head kvh0 + c / TPH (zero when c % TPH >= g). The q
        // rows are staged in LDS after the staging tiles; with one KV head
        // per tile (fewer registers in use) each lane then keeps its
        // fragments in registers, otherwise they are read per tile, which
        // keeps 16 registers per lane free for the load ring.
        uint16_t* qs = reinterpret_cast<uint16_t*>(smem) + W * 2 * kTile * RS;
        for (int i = (int)threadIdx.x; i < kTile * (D / 8); i += (int)blockDim.x) {
            const int col = i / (D / 8);
            const int d8 = i - col * (D / 8);
            const int qi = col % TPH;
            u32x4 w = u32x4{0u, 0u, 0u, 0u};
            if (qi < g)
                w = *reinterpret_cast<const u32x4*>(a.q + (int64_t)wi.seq * a.q_seq +
                                                    (int64_t)((kvh0 + col / TPH) * g + qi) * a.q_head + 8 * d8);
            *reinterpret_cast<u32x4*>(qs + col * RS + 8 * d8) = w;
        }
        __syncthreads();
        const uint16_t* q_row = qs + c * RS + 8 * gq;
        // q fragments in registers (one head per tile; not for the bf16
        // 2-tile ring at D = 128, whose 128-register budget they overflow)
        constexpr bool QR = HP == 1 && (FP8 || NB >= 3 || D == 64);
        bf16x8 qf[QR ? NQK : 1];
        if constexpr (QR) {
#pragma unroll
            for (int j = 0; j < NQK; ++j) qf[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q_row + 32 * j));
        }

        float m = -INFINITY;  // running max of head c (log2 units), same in all four lane groups
        // running sum of column c's probabilities over every token so far
        // (all four lane groups' rows), as an MFMA accumulator: each tile adds
        // ones(16 x 16) . P^T, so every element of the tile holds the sum
        f32x4 lacc = f32x4{0.f, 0.f, 0.f, 0.f};
        const bf16x4 ones = bf16x4{(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
        f32x4 o[NPV];
#pragma unroll
        for (int j = 0; j < NPV; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

        // The tokens this wave streams: the whole item's, shared round robin
        // with the other waves, or (WPP) its own partition's, in order.
        WorkItem wv = wi;
        int part_w = wi.part;
        if constexpr (WPP) {
            part_w = wi.part * W + wave;
            wv.t_begin = wi.t_begin + wave * a.partition_tokens;
            wv.t_end = min(wv.t_begin + a.partition_tokens, wi.t_end);
        }
        const int span = wv.t_end - wv.t_begin;
        const int ntiles = span > 0 ? (span + TPH - 1) / TPH : 0;
        // The unit's first KV head is folded into each tile's descriptor base,
        // so a row's bytes start at a multiple of the row stride from it
        // (with HP > 1 the HP heads of a row are adjacent in memory).
        const int64_t head_off = (int64_t)kvh0 * a.cache.head;
        // per-lane byte offset inside a tile (the same for K and V), fixed for
        // the whole item: load i of lane l covers token i * RPI + l / LPC,
        // bytes 16 (l % LPC) of its HP-head chunk; the i * RPI tokens go into
        // the wave-uniform offset
        const uint32_t roff = (uint32_t)(lane / LPC) * a.cache.token + 16u * (uint32_t)(lane % LPC);
        const uint32_t rstep = (uint32_t)RPI * a.cache.token;
        const int bs_mask = (1 << a.block_size_log2) - 1;
        const float qk = a.qk_scale_log2;

        u32x4 kb[NB][NI], vb[NB][NI];  // ring of NB tiles: NB - 1 in flight while one is consumed

        // Loads for tile t, through a buffer descriptor that ends at the
        // tile's last valid row: rows past the context read as zero (their
        // weight is 0, but 0 * NaN would not be), with no masking code. A tile
        // past the end (the prefetch after the last one) still issues its
        // loads, against a zero-byte descriptor: they return zeros without
        // touching memory, and every path through the loop keeps the same
        // number of loads in flight, so the wait before a tile's use never
        // has to drain the prefetch behind it.
        // Wave w takes tiles w, w + W, w + 2W, ... of the item.
        const int t_first = WPP ? 0 : wave, t_step = WPP ? 1 : W, t_stop = ntiles;

        auto issue = [&](int t, int64_t blk, u32x4 (&kb)[NI], u32x4 (&vb)[NI]) {
            const bool live = t < t_stop;
            const int t0 = wv.t_begin + (live ? t : t_stop - 1) * TPH;
            const uint32_t row0 = (uint32_t)(t0 & bs_mask) * a.cache.token;
            const int valid = min(wv.t_end - t0, TPH);
            const uint32_t nbytes = live ? row0 + (uint32_t)valid * a.cache.token : 0u;
            const int64_t base = blk * a.cache.block + head_off;
            const auto rk = make_rsrc(a.k_cache + base, nbytes);
            const auto rv = make_rsrc(a.v_cache + base, nbytes);
#pragma unroll
            for (int i = 0; i < NI; ++i) kb[i] = buf_load_b128_stream(rk, roff, row0 + i * rstep);
#pragma unroll
            for (int i = 0; i < NI; ++i) vb[i] = buf_load_b128_stream(rv, roff, row0 + i * rstep);
        };

        auto consume = [&](int t, const u32x4 (&kb)[NI], const u32x4 (&vb)[NI]) {
            const int t0 = wv.t_begin + t * TPH;
            const int valid = wv.t_end - t0;
            const bool full = valid >= TPH;

            // With HP > 1 the P.V MFMA also multiplies each V row by the zero
            // probabilities of the other heads' columns; 0 * Inf or 0 * NaN
            // would leak a non-finite V value into those heads. A tile whose V
            // holds one (never in practice) takes the per-head path below.
            bool v_nonfinite = false;
            if constexpr (HP > 1) {
                uint32_t flag = 0;
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if constexpr (!FP8)  // bf16: exponent field all ones, per 16-bit half
                            flag |= ((vb[i][q] & 0x7f807f80u) + 0x00800080u) & 0x80008000u;
                        else  // e4m3fn: S.1111.111 per byte
                            flag |= ((vb[i][q] & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u;
                    }
                v_nonfinite = __builtin_amdgcn_ballot_w64(flag != 0) != 0;
            }

            // K and V rows -> LDS as bf16 (rows past the context arrived as zeros)
            auto stage = [&](uint16_t* dst, const u32x4& w, int row) {
                if constexpr (!FP8) {
                    *reinterpret_cast<u32x4*>(dst + row * RS + (lane % LPR) * 8) = w;
                } else {
                    u32x4 lo, hi;
                    fp8x16_to_bf16(w, lo, hi);
                    *reinterpret_cast<u32x4*>(dst + row * RS + (lane % LPR) * 16) = lo;
                    *reinterpret_cast<u32x4*>(dst + row * RS + (lane % LPR) * 16 + 8) = hi;
                }
            };
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                // MFMA row of this chunk: head (l % LPC) / LPR, token i * RPI + l / LPC
                const int row = ((lane % LPC) / LPR) * TPH + i * RPI + lane / LPC;
                stage(ks, kb[i], row);
                stage(vs, vb[i], row);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

            // S = K Q^T
            f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NQK; ++j) {
                const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ks + c * RS + 32 * j + 8 * gq));
                bf16x8 qb;
                if constexpr (QR) qb = qf[j];
                else qb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q_row + 32 * j));
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb, s, 0, 0, 0);
            }

            // online softmax for column c over rows 4*gq + r: a row counts
            // when it is a token of the column's KV head inside the context
            float x[4];
            if (HP == 1 && full) {  // uniform: every row counts
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] = s[r] * qk;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * gq + r;
                    const bool mine = HP == 1 || (row / TPH) == (c / TPH);
                    x[r] = (!mine || (!full && row % TPH >= valid)) ? -INFINITY : s[r] * qk;
                }
            }
            float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            mx = fmaxf(mx, xor_shfl(mx, 16));
            mx = fmaxf(mx, xor_shfl(mx, 32));
            const float m_new = fmaxf(m, mx);
            const float ms = (m_new == -INFINITY) ? 0.0f : m_new;
            const float alpha = fast_exp2(m - ms);
            // Rescale only when some head's running max moved (after the first
            // tiles of a long context it rarely does).
            const bool moved = __builtin_amdgcn_ballot_w64(m_new != m) != 0;
            m = m_new;
            // probabilities rounded to bf16: the P.V operand, and what the
            // sum accumulates (so the normalisation matches the products)
            bf16x4 pb;
#pragma unroll
            for (int r = 0; r < 4; ++r) pb[r] = (__bf16)fast_exp2(x[r] - ms);
            if (moved) {
#pragma unroll
                for (int j = 0; j < NPV; ++j) o[j] *= alpha;
                lacc *= alpha;
            }
            lacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, pb, lacc, 0, 0, 0);

            // O^T += V^T P^T. ds_read_b64_tr_b16: within each 16-lane group,
            // lane i receives element i % 4 of the 8-byte rows addressed by
            // lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12. Lane (gq, s) addresses
            // V[4 gq + s/4][16 j + 4 (s % 4)], so lane (gq, c) receives
            // V[4 gq + k][16 j + c], k = 0..3: the A operand, one instruction
            // per MFMA.
            typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
            typedef __attribute__((address_space(3))) uint16_t lds_u16;
            if (!v_nonfinite) {
#pragma unroll
                for (int j = 0; j < NPV; ++j) {
                    lds_s16x4* src = (lds_s16x4*)((lds_u16*)const_cast<uint16_t*>(tr_base) + 16 * j);
                    const bf16x4 va = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(src));
                    o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[j], 0, 0, 0);
                }
            } else {
                // one MFMA per head with the other heads' V rows zeroed; a
                // lane keeps the result of its own column's head. Lane (gq, c)
                // supplies V rows 4 gq .. 4 gq + 3, all of head 4 gq / TPH.
                const int row_head = (4 * gq) / TPH, col_head = c / TPH;
#pragma unroll 1
                for (int h = 0; h < HP; ++h) {
                    const uint32_t keep = row_head == h ? 0xffffffffu : 0u;
#pragma unroll
                    for (int j = 0; j < NPV; ++j) {
                        // one MFMA at a time: this path is rare, keep its registers few
                        __builtin_amdgcn_sched_barrier(0);
                        lds_s16x4* src = (lds_s16x4*)((lds_u16*)const_cast<uint16_t*>(tr_base) + 16 * j);
                        const u32x2 vw = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(src));
                        const bf16x4 va = __builtin_bit_cast(bf16x4, u32x2{vw[0] & keep, vw[1] & keep});
                        const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, f32x4{0.f, 0.f, 0.f, 0.f},
                                                                                 0, 0, 0);
                        if (col_head == h) o[j] += t;
                    }
                }
            }
            // the next tile's staging overwrites this one
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };

        if (t_first < t_stop) {
            // The ring is unrolled so that every buffer index is a constant.
            // Each step issues the loads NB - 1 tiles ahead unconditionally
            // (past the end they are zero-byte no-ops) and consumes one tile
            // behind a uniform branch, so every path through the loop keeps
            // the same loads in flight and the waits before a tile's use
            // leave the prefetch behind it outstanding. sched_barrier keeps
            // the compiler from sinking the prefetch below those waits.
            // The table entry of each issued tile was fetched one step earlier.
            const TableReader tab = make_table_reader(a, wv, t_stop - 1, TPH);
            uint32_t entry = table_fetch(tab, t_first);
#pragma unroll
            for (int b = 0; b < NB - 1; ++b) {
                const int64_t blk = table_block(tab, entry);
                entry = table_fetch(tab, t_first + (b + 1) * t_step);
                __builtin_amdgcn_sched_barrier(0);
                issue(t_first + b * t_step, blk, kb[b], vb[b]);
            }
            for (int t = t_first; t < t_stop; t += NB * t_step) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int ti = t + (b + NB - 1) * t_step;
                    const int64_t blk = table_block(tab, entry);
                    entry = table_fetch(tab, ti + t_step);
                    __builtin_amdgcn_sched_barrier(0);
                    issue(ti, blk, kb[(b + NB - 1) % NB], vb[(b + NB - 1) % NB]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (t + b * t_step < t_stop) consume(t + b * t_step, kb[b], vb[b]);
                }
            }
        }

        // the sum over every token of column c, the same in all four lane groups
        const float l = lacc[0];

        if constexpr (WPP) {
            // This wave's state is a whole partition's: store it directly.
            // Partition 0 always stores (a zero-length context's zero row);
            // a partition past the context's end stores nothing (the merge
            // never reads it). Column c is query head (c / TPH) * g + c % TPH
            // of the unit's HP * g heads; lane (gq, c) holds d = 16 j + 4 gq + r.
            if ((wv.t_end > wv.t_begin || part_w == 0) && c % TPH < g) {
                const int hq = wi.kvh * HP * g + (c / TPH) * g + c % TPH;
                if (wi.final_out) {
                    const float inv = l > 0.0f ? a.v_scale / l : 0.0f;
                    uint16_t* dst = a.out + (int64_t)wi.seq * a.out_seq + (int64_t)hq * a.out_head;
#pragma unroll
                    for (int j = 0; j < NPV; ++j) {
                        const uint32_t lo = (uint32_t)f32_to_bf16_rne(o[j][0] * inv) |
                                            ((uint32_t)f32_to_bf16_rne(o[j][1] * inv) << 16);
                        const uint32_t hi = (uint32_t)f32_to_bf16_rne(o[j][2] * inv) |
                                            ((uint32_t)f32_to_bf16_rne(o[j][3] * inv) << 16);
                        *reinterpret_cast<u32x2*>(dst + 16 * j + 4 * gq) = u32x2{lo, hi};
                    }
                } else {
                    const int64_t prow = ((int64_t)wi.seq * a.num_q_heads + hq) * a.num_partitions + part_w;
#pragma unroll
                    for (int j = 0; j < NPV; ++j)
                        *reinterpret_cast<f32x4*>(a.part_o + prow * D + 16 * j + 4 * gq) = o[j] * a.v_scale;
                    if (gq == 0) {
                        a.part_ml[prow * 2] = m;
                        a.part_ml[prow * 2 + 1] = l;
                    }
                }
            }
            return;
        }

        __syncthreads();  // V staging is dead; reuse LDS for the combine
        // column c -> query head cc = (c / TPH) * g + c % TPH of the unit's
        // G = HP * g heads
        const int G = HP * g;
        float* sm_ml = smem;
        float* sm_o = smem + W * G * 2;
        if (c % TPH < g) {
            const int cc = (c / TPH) * g + c % TPH;
            if (gq == 0) {
                sm_ml[(wave * G + cc) * 2] = m;
                sm_ml[(wave * G + cc) * 2 + 1] = l;
            }
#pragma unroll
            for (int j = 0; j < NPV; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) sm_o[(wave * G + cc) * D + 16 * j + 4 * gq + r] = o[j][r];
        }
        __syncthreads();
        combine_and_store<D>(a, sm_ml, sm_o, W, G, wi.seq, wi.kvh, wi.part, wi.final_out);
    });
}

template <int D, bool FP8, int NB, int HP, bool WPP>
hipError_t launch_d(const DecodeArgs& a, const LaunchShape& ls, hipStream_t s) {
    const dim3 block((unsigned)(64 * ls.waves));
    const size_t stage = ((size_t)ls.waves * 2 + 1) * kTile * (D + 8) * sizeof(uint16_t);
    const size_t comb = (size_t)ls.waves * HP * a.group * (D + 2) * sizeof(float);
    static_assert(kSelfLdsInts * sizeof(int) <= kTile * (64 + 8) * sizeof(uint16_t), "item scratch fits the staging area");
    const size_t lds = stage > comb ? stage : comb;
    const dim3 grid((unsigned)((int64_t)a.num_seqs * a.units_per_seq * a.num_items));
    hipLaunchKernelGGL((pa_decode_mfma_kernel<D, FP8, NB, HP, WPP>), grid, block, lds, s, a);
    return hipGetLastError();
}

template <int D, bool FP8, int HP>
hipError_t launch_nb(const DecodeArgs& a, const LaunchShape& ls, hipStream_t s) {
    if (ls.wave_partitions) {  // one partition per wave: rings of 2 or 3 tiles, one or two heads per tile
        if constexpr (HP <= 2) {
            if (ls.depth <= 2) return launch_d<D, FP8, 2, HP, true>(a, ls, s);
            return launch_d<D, FP8, 3, HP, true>(a, ls, s);
        }
        return hipErrorInvalidValue;
    }
    if (ls.depth <= 2) return launch_d<D, FP8, 2, HP, false>(a, ls, s);
    if (ls.depth == 3) return launch_d<D, FP8, 3, HP, false>(a, ls, s);
    return launch_d<D, FP8, 4, HP, false>(a, ls, s);
}

template <int D, bool FP8>
hipError_t launch_hp(const DecodeArgs& a, const LaunchShape& ls, hipStream_t s) {
    if (ls.heads_per_unit == 4) return launch_nb<D, FP8, 4>(a, ls, s);
    if (ls.heads_per_unit == 2) return launch_nb<D, FP8, 2>(a, ls, s);
    return launch_nb<D, FP8, 1>(a, ls, s);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, int head_dim, bool fp8, const LaunchShape& ls, hipStream_t s) {
    if (head_dim == 64) return fp8 ? launch_hp<64, true>(a, ls, s) : launch_hp<64, false>(a, ls, s);
    return fp8 ? launch_hp<128, true>(a, ls, s) : launch_hp<128, false>(a, ls, s);
}

}  // namespace pa
