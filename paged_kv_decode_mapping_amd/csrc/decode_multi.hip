// decode_multi.hip -- paged attention for several query rows per KV head:
// multi-token queries (speculative verification, chunked prefill) and GQA
// groups wider than one 16-row matrix tile (MQA).
//
// Pages cited (titles as printed at the top of each page):
//   Tutorial = «大模型推理优化与加速完全教程» (LLM inference optimisation tutorial)
//   ToPG     = «ToPG框架解析：大模型推理性能优化与三阶段流水线设计»
//
// What it computes. Sequence i has context_lens[i] = L cached tokens; its
// last n = query_start[i+1] - query_start[i] are its query tokens (already
// written to the cache). Query r sits at position p = L - n + r and, for
// each query head h, attends over positions 0..p (causal) of KV head h / g:
// the target model's single verification pass over K draft tokens of
// Tutorial §5.1 (speculative decoding), a prefill chunk over its cached
// prefix as in Tutorial §6.2 (chunked prefill), and, with n = 1, the decode
// step of Tutorial §4.4 (GroupedQueryAttention) for any group size, MQA
// included. Gather through the block table as in Tutorial §4.2 (get_kv).
//
// Rows. The (query token r, head hh) pairs of one (sequence, KV head) are
// rows rho = r * g + hh; every wave of a workgroup owns RT 16-row tiles of
// them (W = 1, 2, 4 or 8 waves of one tile, or 4 waves of two: 16 W RT
// rows), so the online-softmax state of a row never leaves its lanes and a
// workgroup needs no combine step. Rows are the columns of the same MFMA tiles the decode
// kernel uses:
//   S = K Q^T   v_mfma_f32_16x16x32_bf16, A = K rows from LDS, B = Q^T rows
//               of this wave (in registers with 4 or 8 waves or two row
//               tiles, else LDS);
//   O^T += V^T P^T  A = V^T by the transposing LDS read, B = the lane's own
//               probabilities (bf16): v_mfma_f32_16x16x16_bf16 per tile, or
//               v_mfma_f32_16x16x32_bf16 per pair of tiles (below).
// Lane (c, gq) holds S[token 4 gq + r][row c]: the causal mask compares the
// token with the position of row c (skipped on tiles every row sees whole).
//
// Tiles. The workgroup walks its token range in 16-token tiles; all waves
// use every tile, so the tile is loaded once, cooperatively (each lane one
// or more 16-byte chunks of K and of V), and staged in LDS. Each lane keeps
// a ring of NB slots of its chunks in registers (NB - 1 in flight), and the
// LDS copy is double-buffered, so one workgroup barrier per slot orders
// both the staging before the reads and the reads before the next overwrite.
// With at least twice as many lanes as a tile has chunks, a slot holds two
// consecutive tiles (one per half of the workgroup) consumed as one 32-token
// step.
// fp8 codes are widened to bf16 while staging (exact); the scales are folded
// into the score scale and the output (ToPG §2: fp32 accumulation; ToPG §3:
// fp8 KV).
//
// Split-K. A workgroup covers one partition of at most P tokens; with more
// than one partition it stores unnormalised partial states (m, l, o) of the
// rows that see tokens past partition 0, and pa_multi_merge_kernel combines
// them by log-sum-exp; rows that see partition 0 only are finished here.
//
// Cascade prefix pass. Sequences that share a cached prefix (Tutorial §4.3,
// prefix caching: the same physical blocks in every sharer's table) attend
// to it here once per group instead of once per sequence: the grid's
// "sequences" are the prefix groups, each group's rows are the query heads
// of all its member sequences, the tiles come from the prefix's own table
// row, and a member attends the first min(its context, prefix length)
// tokens. The states are always stored as partials; the cascade merge adds
// the states of the suffix pass (the decode kernels over the rest of each
// context).
//
// Order. With a work list (the decode path's longest-first list of
// (sequence, KV head, partition) items), or with each workgroup ranking its
// block index in that order itself (batches of up to 256 sequences, no
// builder pass), workgroups take items longest first, so the longest
// contexts start first; one cooperative tile stream per workgroup makes a
// long item slow, and a long item started last would stretch the whole
// launch.
#include "pa_cascade.h"
#include "pa_merge.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void fp8x16_to_bf16_m(const u32x4& w, u32x4& lo, u32x4& hi) {
    uint32_t r[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
        r[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
    }
    lo = u32x4{r[0], r[1], r[2], r[3]};
    hi = u32x4{r[4], r[5], r[6], r[7]};
}

// Maximum over the four lanes c, c + 16, c + 32, c + 48 (one MFMA column),
// returned to all four: v_permlane16_swap exchanges lanes 16 apart and
// v_permlane32_swap lanes 32 apart, each result pair holding the lane's own
// value and its partner's. Both run on the VALU; a ds_bpermute exchange
// costs an LDS round trip per step, on the critical path of every tile.
__device__ __forceinline__ float column_max4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Work item of a workgroup: (sequence, KV head, row block, partition).
struct MultiItem {
    int seq, kvh, rb, part;
    int L;        // context length (clamped to the table row)
    int q0, n;    // first query row and number of query tokens
};

// Sum over the four lanes of one MFMA column, returned to all four.
__device__ __forceinline__ float column_sum4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Register budget of the multi-row kernel, as waves per SIMD: four (128
// registers) for 4 or 8 waves of one row tile; three (168) for two row tiles,
// whose accumulators and query fragments double, except fp8 at D = 128,
// whose staging conversion spills there (two, 256); unconstrained below 4
// waves.
constexpr int multi_waves_per_eu(int D, bool fp8, int W, int RT) {
    return RT == 2 ? ((fp8 && D == 128) ? 2 : 3) : (W >= 4 ? 4 : 1);
}

// RT: 16-row tiles per wave. Every wave reads each staged K fragment and
// each transposed V fragment from LDS once per tile and feeds it to RT
// MFMAs, one per row tile: with 128 rows per KV head, 4 waves of 32 rows
// read half the LDS bytes 8 waves of 16 rows do (the LDS, not HBM, bounds
// the 16-row form there: all waves read the whole tile). The row sums then
// stay per lane on the VALU (the matrix pipe is the busier one), reduced
// over the column's four lanes at the end.
template <int D, bool FP8, int W, int NB, int RT>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(multi_waves_per_eu(D, FP8, W, RT)))) void pa_multi_kernel(MultiArgs a) {
    constexpr int ESZ = FP8 ? 1 : 2;
    constexpr int NQK = D / 32;
    constexpr int NPV = D / 16;
    constexpr int EPL = 16 / ESZ;            // elements per 16-byte chunk
    constexpr int LPR = D / EPL;             // chunks per token row
    constexpr int CHUNKS = kTile * LPR;      // chunks per tile (of K, and of V)
    constexpr int LANES = 64 * W;
    // Tiles per ring slot. Every wave of the workgroup steps through the same
    // tiles, so what a slot holds is what hides latency and what one barrier
    // stages; two consecutive tiles are consumed as one 32-token step.
    //   mode 0: at least twice as many lanes as a tile has chunks: the two
    //           halves of the workgroup load one tile each (one chunk a lane);
    //   mode 1: exactly as many lanes as chunks, 4 or more waves: each lane
    //           loads one chunk of each tile (the ring then has 2 slots, so
    //           the registers stay those of 4 slots of one tile);
    //   mode 2: fewer lanes (1 or 2 waves): one tile a slot, several chunks
    //           a lane.
    constexpr int MODE = LANES >= 2 * CHUNKS ? 0 : ((W >= 4 && LANES == CHUNKS) ? 1 : 2);
    constexpr int TPS = MODE == 2 ? 1 : 2;
    constexpr int NI = MODE == 0 ? 1 : (MODE == 1 ? 2 : (CHUNKS + LANES - 1) / LANES);  // chunks a lane loads per slot
    constexpr int SROWS = TPS * kTile;       // token rows staged per LDS buffer
    constexpr int RS = D + 8;                // LDS row stride of q and K rows, bf16 elements
    // V rows: 16 more elements. A transposing read takes 4 rows x 32 bytes
    // per 16 lanes; rows 32 bytes apart in bank order (stride 288 bytes for
    // D = 128) keep those 4 segments on disjoint banks, where 272 bytes
    // overlaps them two-way. K rows keep 272 bytes: their 16-byte reads by
    // 16 lanes are conflict-free there and would collide at 288.
    constexpr int RSV = D + 16;
    static_assert(NB % 2 == 0, "the LDS buffer of a ring slot is its parity");
    static_assert(RT == 1 || RT == 2, "one or two row tiles per wave");
    constexpr int WROWS = 16 * RT;           // rows per wave
    constexpr int GROWS = WROWS * W;         // rows per workgroup

    // With 4 or 8 waves, or two row tiles a wave (many rows: LDS traffic
    // counts), this wave's query fragments, the B operands of every q.K^T
    // MFMA, stay in registers instead of being read from LDS for every tile,
    // and the query rows' LDS is then reused for the K/V buffers; with 1 or 2
    // waves of one tile (few rows, memory-bound) the 16 registers would cost
    // occupancy.
    constexpr bool kQInRegs = W >= 4 || RT == 2;
    extern __shared__ float smem[];
    uint16_t* qs = reinterpret_cast<uint16_t*>(smem);   // [GROWS][RS] query rows
    uint16_t* kbuf = kQInRegs ? qs : qs + GROWS * RS;    // [2][SROWS][RS]
    uint16_t* vbuf = kbuf + 2 * SROWS * RS;              // [2][SROWS][RSV]

    // ---- the work item
    int bid = (int)blockIdx.x;
    const int cap = a.max_blocks_per_seq << a.block_size_log2;
    MultiItem it;
    if (a.self_schedule) {
        // longest-first (sequence, partition) items, ranked by this workgroup
        // itself, expanded over (KV head, row block) units
        int unit;
        if (!rank_item_wave(a.context_lens, a.num_seqs, a.partition_tokens, cap, a.num_kv_heads * a.row_blocks, bid,
                            reinterpret_cast<int*>(smem), &it.seq, &it.part, &unit))
            return;
        it.kvh = unit / a.row_blocks;
        it.rb = unit - it.kvh * a.row_blocks;
    } else if (a.items != nullptr) {
        const int idx = bid / a.row_blocks;
        it.rb = bid - idx * a.row_blocks;
        const int count = *a.item_count;
        const int4 rec = a.items[idx];  // in bounds: the list has room for the whole grid
        if (idx >= count) return;
        it.seq = rec.x;
        it.kvh = rec.y & 0xffff;
        it.part = rec.y >> 16;
    } else {
        it.part = bid % a.num_partitions;
        bid /= a.num_partitions;
        it.rb = bid % a.row_blocks;
        bid /= a.row_blocks;
        it.kvh = bid % a.num_kv_heads;
        it.seq = bid / a.num_kv_heads;
    }
    // A cascade prefix pass: item "sequence" k is prefix group k, whose
    // member sequences are the query rows (one token each).
    const bool prefix_pass = a.cascade.group_start != nullptr;
    if (prefix_pass) {
        it.L = min(cascade_prefix_tokens(a.cascade, it.seq, a.block_size_log2), cap);
    } else {
        const int L = a.context_lens[it.seq];
        it.L = L < 0 ? 0 : (L > cap ? cap : L);
    }
    if (prefix_pass || a.query_start != nullptr) {
        const int32_t* starts = prefix_pass ? a.cascade.group_start : a.query_start;
        it.q0 = starts[it.seq];
        int n = starts[it.seq + 1] - it.q0;
        n = n > a.max_query_len ? a.max_query_len : n;
        // rows outside [0, num_query_rows) are never touched, whatever the offsets hold
        if (it.q0 < 0 || it.q0 > a.num_query_rows) n = 0;
        else if (n > a.num_query_rows - it.q0) n = a.num_query_rows - it.q0;
        it.n = n < 0 ? 0 : n;
    } else {
        it.q0 = it.seq;
        it.n = 1;
    }
    const int g = a.group;
    const int rows = it.n * g;
    const int row0 = it.rb * GROWS;
    if (row0 >= rows) return;
    // the last position any row of this block attends to
    const int last_row = min(rows, row0 + GROWS) - 1;
    const int pos_max = prefix_pass ? it.L - 1 : it.L - it.n + last_row / g;
    const int t_begin = it.part * a.partition_tokens;
    const int t_end = min(min(t_begin + a.partition_tokens, pos_max + 1), it.L);
    if (it.part > 0 && t_begin >= t_end) return;  // nothing of this block here (partition 0 always stores)

    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = (int)(threadIdx.x & 63);
    const int c = lane & 15;
    const int gq = lane >> 4;

    const int span = t_end - t_begin;
    const int ntiles = span > 0 ? (span + kTile - 1) / kTile : 0;
    // Block-table entries of the item, 64 at a time in one register (lane
    // l holds entry w_base + l), read with readlane; the next 64 are loaded
    // as soon as a window is entered, so the tile loop never waits on a
    // table load. (Fetching one entry per tile a tile ahead, as the decode
    // kernels do, made every iteration here wait for a load issued one
    // iteration earlier: all waves of a workgroup step through the tiles
    // together, so nothing hid that wait.) They go out before the query rows.
    const auto tab_rsrc = make_rsrc(a.block_tables + (int64_t)it.seq * a.table_stride,
                                    (uint32_t)a.max_blocks_per_seq * 4u);
    const int e_last = (t_begin + max(ntiles - 1, 0) * kTile) >> a.block_size_log2;
    auto table_load = [&](int base) {
        return __builtin_amdgcn_raw_buffer_load_b32(tab_rsrc, (uint32_t)min(base + lane, e_last) << 2, 0, 0);
    };
    int w_base = t_begin >> a.block_size_log2;
    uint32_t w_cur = 0u, w_next = 0u;
    if (ntiles > 0) {
        w_cur = table_load(w_base);
        w_next = table_load(w_base + 64);
    }

    // ---- query rows of this block -> LDS (zero rows past the block's rows):
    // every load first, then the stores
    constexpr int QPT = (GROWS * (D / 8)) / (64 * W);  // 16-byte chunks per thread
    u32x4 qv[QPT];
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
        const int i = (int)threadIdx.x + 64 * W * k;
        const int rr = i / (D / 8);
        const int d8 = i - rr * (D / 8);
        const int rho = row0 + rr;
        qv[k] = u32x4{0u, 0u, 0u, 0u};
        if (rho < rows) {
            const int r = rho / g, hh = rho - (rho / g) * g;
            qv[k] = *reinterpret_cast<const u32x4*>(a.q + (int64_t)(it.q0 + r) * a.q_row +
                                                    (int64_t)(it.kvh * g + hh) * a.q_head + 8 * d8);
        }
    }

    // this lane's rows (column c of each of the wave's tiles) and their
    // causal limits
    int my_rho[RT], my_pos[RT];
    bool my_valid[RT];
#pragma unroll
    for (int u = 0; u < RT; ++u) {
        my_rho[u] = row0 + (wave * RT + u) * 16 + c;
        my_valid[u] = my_rho[u] < rows;
        my_pos[u] = my_valid[u] ? it.L - it.n + my_rho[u] / g : -1;  // sees tokens <= my_pos
        if (prefix_pass && my_valid[u]) {
            // a member attends min(its context, the prefix) tokens here
            int ctx = a.context_lens[it.q0 + my_rho[u] / g];
            ctx = ctx < 0 ? 0 : (ctx > a.cascade.max_context ? a.cascade.max_context : ctx);
            my_pos[u] = min(ctx, it.L) - 1;
        }
    }
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
        const int i = (int)threadIdx.x + 64 * W * k;
        const int rr = i / (D / 8);
        *reinterpret_cast<u32x4*>(qs + rr * RS + 8 * (i - rr * (D / 8))) = qv[k];
    }
    const uint16_t* q_row = qs + (wave * WROWS + c) * RS + 8 * gq;  // row tile u at + 16 u RS
    // The last token every valid row of this wave sees (wave-uniform): tiles
    // that end at or before it, and before t_end, need no mask.
    int wave_pos = 0x7fffffff;
#pragma unroll
    for (int u = 0; u < RT; ++u) wave_pos = min(wave_pos, my_valid[u] ? my_pos[u] : 0x7fffffff);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) wave_pos = min(wave_pos, __shfl_xor(wave_pos, off, 64));
    wave_pos = __builtin_amdgcn_readfirstlane(wave_pos);

    float m[RT];
    // One row tile: the running sum of row c's probabilities over every
    // token so far, as an MFMA accumulator: each step adds ones . P^T, so
    // every element of the tile holds the row's sum of the same rounded
    // probabilities. Two: lsum, this lane's share of it (unrounded).
    f32x4 lacc = f32x4{0.f, 0.f, 0.f, 0.f};
    float lsum[RT];
    f32x4 o[RT][NPV];
#pragma unroll
    for (int u = 0; u < RT; ++u) {
        m[u] = -INFINITY;
        lsum[u] = 0.0f;
#pragma unroll
        for (int j = 0; j < NPV; ++j) o[u][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int64_t head_off = (int64_t)it.kvh * a.cache.head;  // folded into each tile's descriptor base
    const int bs_mask = (1 << a.block_size_log2) - 1;
    const float qk = a.qk_scale_log2;

    // Chunk i of this lane: tile cts[i] of the slot, chunk id cid[i] within
    // the tile (token row cid / LPR, 16-byte piece cid % LPR). The tile is
    // wave-uniform: CHUNKS is a multiple of 64.
    uint32_t coff[NI];
    bool cown[NI];
    int cid[NI], cts[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int tid = (int)threadIdx.x;
        int k, ts;
        bool own;
        if constexpr (MODE == 0) {
            ts = min(tid / CHUNKS, TPS - 1);
            k = tid - ts * CHUNKS;
            own = tid < TPS * CHUNKS;
        } else if constexpr (MODE == 1) {
            ts = i;
            k = tid;
            own = true;
        } else {
            ts = 0;
            k = tid + LANES * i;
            own = k < CHUNKS;
        }
        cown[i] = own;
        cts[i] = ts;
        const int kk = own ? k : 0;
        cid[i] = kk;
        // a lane past the tile's chunks reads past every descriptor (zeros)
        coff[i] = own ? (uint32_t)(kk / LPR) * a.cache.token + 16u * (uint32_t)(kk % LPR) : 0x7fffffffu;
    }
    const int nslots = (ntiles + TPS - 1) / TPS;

    u32x4 kb[NB][NI], vb[NB][NI];

    __syncthreads();  // query rows in LDS
    bf16x8 qf[RT][NQK];
    if constexpr (kQInRegs) {
#pragma unroll
        for (int u = 0; u < RT; ++u)
#pragma unroll
            for (int j = 0; j < NQK; ++j)
                qf[u][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q_row + 16 * u * RS + 32 * j));
        __syncthreads();  // every wave has its fragments: the K/V staging may overwrite the rows
    }
    // B operand of row tile u, fragment j
    auto qfrag = [&](int u, int j) -> bf16x8 {
        if constexpr (kQInRegs) return qf[u][j];
        else return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q_row + 16 * u * RS + 32 * j));
    };

    if (ntiles > 0) {
        // physical block of tile t (tiles past the last take the last one's),
        // clamped into the pool; a wave calls it with t growing by at most TPS
        auto block_of = [&](int t) -> int64_t {
            const int e = (t_begin + min(t, ntiles - 1) * kTile) >> a.block_size_log2;
            if (e >= w_base + 64) {
                w_base += 64;
                w_cur = w_next;
                w_next = table_load(w_base + 64);
            }
            int b = __builtin_amdgcn_readlane((int)w_cur, e - w_base);
            b = b < 0 ? 0 : b;
            b = b > a.last_block ? a.last_block : b;
            return (int64_t)b;
        };

        // loads of ring slot sl: chunk i of this lane belongs to tile sl * TPS + cts[i]
        auto issue = [&](int sl, u32x4 (&kr)[NI], u32x4 (&vr)[NI]) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int t = sl * TPS + cts[i];
                const int64_t blk = block_of(t);
                __builtin_amdgcn_sched_barrier(0);
                const bool live = t < ntiles;
                const int t0 = t_begin + (live ? t : ntiles - 1) * kTile;
                const uint32_t rowb = (uint32_t)(t0 & bs_mask) * a.cache.token;
                const int valid = min(t_end - t0, kTile);
                const uint32_t nbytes = live ? rowb + (uint32_t)valid * a.cache.token : 0u;
                const int64_t base = blk * a.cache.block + head_off;
                const auto rk = make_rsrc(a.k_cache + base, nbytes);
                const auto rv = make_rsrc(a.v_cache + base, nbytes);
                kr[i] = buf_load_b128_stream(rk, coff[i], rowb);
                vr[i] = buf_load_b128_stream(rv, coff[i], rowb);
            }
        };

        auto stage = [&](uint16_t* dst, int rs, const u32x4& w, int ts, int k) {
            const int row = ts * kTile + k / LPR, ch = k % LPR;
            if constexpr (!FP8) {
                *reinterpret_cast<u32x4*>(dst + row * rs + ch * 8) = w;
            } else {
                u32x4 lo, hi;
                fp8x16_to_bf16_m(w, lo, hi);
                *reinterpret_cast<u32x4*>(dst + row * rs + ch * 16) = lo;
                *reinterpret_cast<u32x4*>(dst + row * rs + ch * 16 + 8) = hi;
            }
        };

        // Online-softmax update of row tile u from its NX scores x (already
        // scaled and masked): new running max, rescale of the tile's output
        // and row sum when the max moved, probabilities returned in p.
        auto softmax_step = [&](int u, const float* x, float* p, auto nx_tag) {
            constexpr int NX = decltype(nx_tag)::value;
            float mx = fmaxf(x[0], x[1]);
#pragma unroll
            for (int r = 2; r < NX; ++r) mx = fmaxf(mx, x[r]);
            mx = column_max4(mx);
            const float m_new = fmaxf(m[u], mx);
            const float ms = (m_new == -INFINITY) ? 0.0f : m_new;
            const float alpha = fast_exp2(m[u] - ms);
            const bool moved = __builtin_amdgcn_ballot_w64(m_new != m[u]) != 0;
            m[u] = m_new;
            float ps = 0.0f;
#pragma unroll
            for (int r = 0; r < NX; ++r) {
                p[r] = fast_exp2(x[r] - ms);
                ps += p[r];
            }
            if (moved) {
#pragma unroll
                for (int j = 0; j < NPV; ++j) o[u][j] *= alpha;
                if constexpr (RT == 1) lacc *= alpha;
            }
            if constexpr (RT != 1) lsum[u] = lsum[u] * alpha + ps;
        };

        // one tile of a staged slot: scores, online softmax, P.V
        auto compute = [&](int t, const uint16_t* ks, const uint16_t* vs) {
            const int t0 = t_begin + t * kTile;
            f32x4 s[RT];
#pragma unroll
            for (int u = 0; u < RT; ++u) s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NQK; ++j) {
                const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ks + c * RS + 32 * j + 8 * gq));
#pragma unroll
                for (int u = 0; u < RT; ++u) s[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qfrag(u, j), s[u], 0, 0, 0);
            }
            const bool whole = t0 + kTile - 1 <= wave_pos && t0 + kTile <= t_end;  // uniform: every row sees the whole tile
            bf16x4 pb[RT];
#pragma unroll
            for (int u = 0; u < RT; ++u) {
                float x[4], p[4];
                if (whole) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[r] = s[u][r] * qk;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int tok = t0 + 4 * gq + r;
                        x[r] = (tok > my_pos[u] || tok >= t_end) ? -INFINITY : s[u][r] * qk;
                    }
                }
                softmax_step(u, x, p, std::integral_constant<int, 4>{});
#pragma unroll
                for (int r = 0; r < 4; ++r) pb[u][r] = (__bf16)p[r];
            }
            if constexpr (RT == 1) {
                const bf16x4 ones = bf16x4{(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
                lacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, pb[0], lacc, 0, 0, 0);
            }
            // V^T by ds_read_b64_tr_b16: lane (gq, c) receives V[4 gq + k][16 j + c]
            const uint16_t* tr_base = vs + (4 * gq + (c >> 2)) * RSV + 4 * (lane & 3);
#pragma unroll
            for (int j = 0; j < NPV; ++j) {
                typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
                typedef __attribute__((address_space(3))) uint16_t lds_u16;
                lds_s16x4* src = (lds_s16x4*)((lds_u16*)const_cast<uint16_t*>(tr_base) + 16 * j);
                const bf16x4 va = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(src));
#pragma unroll
                for (int u = 0; u < RT; ++u) o[u][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[u], o[u][j], 0, 0, 0);
            }
        };

        // Two consecutive tiles t and t + 1 as one step of 32 tokens (the
        // second may lie past the item: its scores are masked and its V rows
        // were loaded as zeros): one softmax update, and P.V as
        // v_mfma_f32_16x16x32_bf16, half as many as 16x16x16 steps. Its K
        // index 8 gq + j stands for token 4 gq + j of the first tile (j < 4)
        // and 4 gq + j - 4 of the second (j >= 4): the lane's own eight
        // probabilities in that order, and V^T as the two tiles' transposed
        // reads side by side.
        auto compute_pair = [&](int t, const uint16_t* ks, const uint16_t* vs) {
            const int t0 = t_begin + t * kTile;
            f32x4 sa[RT], sb[RT];
#pragma unroll
            for (int u = 0; u < RT; ++u) {
                sa[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                sb[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int j = 0; j < NQK; ++j) {
                const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ks + c * RS + 32 * j + 8 * gq));
                const bf16x8 kb2 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ks + (kTile + c) * RS + 32 * j + 8 * gq));
#pragma unroll
                for (int u = 0; u < RT; ++u) {
                    const bf16x8 qb = qfrag(u, j);
                    sa[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb, sa[u], 0, 0, 0);
                    sb[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb2, qb, sb[u], 0, 0, 0);
                }
            }
            const bool whole = t0 + 2 * kTile - 1 <= wave_pos && t0 + 2 * kTile <= t_end;  // uniform: nothing to mask
            bf16x8 pb[RT];
#pragma unroll
            for (int u = 0; u < RT; ++u) {
                float x[8], p[8];
                if (whole) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        x[r] = sa[u][r] * qk;
                        x[4 + r] = sb[u][r] * qk;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int ta = t0 + 4 * gq + r, tb = ta + kTile;
                        x[r] = (ta > my_pos[u] || ta >= t_end) ? -INFINITY : sa[u][r] * qk;
                        x[4 + r] = (tb > my_pos[u] || tb >= t_end) ? -INFINITY : sb[u][r] * qk;
                    }
                }
                softmax_step(u, x, p, std::integral_constant<int, 8>{});
#pragma unroll
                for (int r = 0; r < 8; ++r) pb[u][r] = (__bf16)p[r];
            }
            if constexpr (RT == 1) {
                // two 16-token halves against a 2-register ones operand (the
                // 4- and 8-wave kernels sit at their 128-register budget)
                const bf16x4 ones = bf16x4{(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
                lacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, __builtin_shufflevector(pb[0], pb[0], 0, 1, 2, 3),
                                                                 lacc, 0, 0, 0);
                lacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, __builtin_shufflevector(pb[0], pb[0], 4, 5, 6, 7),
                                                                 lacc, 0, 0, 0);
            }
            // V^T by ds_read_b64_tr_b16: lane (gq, c) receives V[4 gq + k][16 j + c] of each tile
            const uint16_t* tr_a = vs + (4 * gq + (c >> 2)) * RSV + 4 * (lane & 3);
            const uint16_t* tr_b = tr_a + kTile * RSV;
#pragma unroll
            for (int j = 0; j < NPV; ++j) {
                typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
                typedef __attribute__((address_space(3))) uint16_t lds_u16;
                const bf16x4 va = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)((lds_u16*)const_cast<uint16_t*>(tr_a) + 16 * j)));
                const bf16x4 vb2 = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)((lds_u16*)const_cast<uint16_t*>(tr_b) + 16 * j)));
                const bf16x8 v8 = __builtin_shufflevector(va, vb2, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int u = 0; u < RT; ++u) o[u][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, pb[u], o[u][j], 0, 0, 0);
            }
        };

        auto consume = [&](int sl, const u32x4 (&kr)[NI], const u32x4 (&vr)[NI], int buf) {
            uint16_t* ks = kbuf + buf * SROWS * RS;
            uint16_t* vs = vbuf + buf * SROWS * RSV;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                if (cown[i]) {
                    stage(ks, RS, kr[i], cts[i], cid[i]);
                    stage(vs, RSV, vr[i], cts[i], cid[i]);
                }
            }
            __syncthreads();  // the slot is in LDS; the other buffer's readers are done
            if constexpr (TPS == 2) {
                compute_pair(sl * 2, ks, vs);
            } else {
                compute(sl, ks, vs);
            }
        };

#pragma unroll
        for (int b = 0; b < NB - 1; ++b) issue(b, kb[b], vb[b]);
        for (int sl = 0; sl < nslots; sl += NB) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                issue(sl + b + NB - 1, kb[(b + NB - 1) % NB], vb[(b + NB - 1) % NB]);
                __builtin_amdgcn_sched_barrier(0);
                if (sl + b < nslots) consume(sl + b, kb[b], vb[b], b & 1);  // uniform over the workgroup
            }
        }
    }

    // ---- store this lane's rows (each row's sum over every token, in all
    // four lanes of its column)
#pragma unroll
    for (int u = 0; u < RT; ++u) {
        const float l = RT == 1 ? lacc[0] : column_sum4(lsum[u]);
        if (!my_valid[u]) continue;
        // A split plan still finishes here every row whose positions all lie
        // in partition 0 (the merge skips rows of one partition: the same
        // test on the same clamped lengths), and stores no state for a
        // partition that holds none of a row's tokens (the merge reads
        // states 0 .. (position / P) only).
        if (!prefix_pass && it.part > 0 && my_pos[u] < t_begin) continue;
        const bool direct = !prefix_pass && (a.num_partitions == 1 || my_pos[u] < a.partition_tokens);
        const int r = my_rho[u] / g, hh = my_rho[u] - (my_rho[u] / g) * g;
        const int64_t row = (int64_t)(it.q0 + r) * a.num_q_heads + it.kvh * g + hh;
        if (direct) {
            uint16_t* dst = a.out + (int64_t)(it.q0 + r) * a.out_row + (int64_t)(it.kvh * g + hh) * a.out_head;
            const float inv = l > 0.0f ? a.v_scale / l : 0.0f;
#pragma unroll
            for (int j = 0; j < NPV; ++j) {
                const uint32_t lo = (uint32_t)f32_to_bf16_rne(o[u][j][0] * inv) |
                                    ((uint32_t)f32_to_bf16_rne(o[u][j][1] * inv) << 16);
                const uint32_t hi = (uint32_t)f32_to_bf16_rne(o[u][j][2] * inv) |
                                    ((uint32_t)f32_to_bf16_rne(o[u][j][3] * inv) << 16);
                *reinterpret_cast<u32x2*>(dst + 16 * j + 4 * gq) = u32x2{lo, hi};
            }
        } else {
            const int64_t prow = row * a.num_partitions + it.part;
#pragma unroll
            for (int j = 0; j < NPV; ++j)
                *reinterpret_cast<f32x4*>(a.part_o + prow * D + 16 * j + 4 * gq) = o[u][j] * a.v_scale;
            if (gq == 0) {
                a.part_ml[prow * 2] = m[u];
                a.part_ml[prow * 2 + 1] = l;
            }
        }
    }
}

// The sequence, first query row and query count of query row `qrow`: the
// last i with query_start[i] <= qrow (n = 0 for rows no sequence owns).
__device__ __forceinline__ void multi_row_owner(const MultiArgs& a, int qrow, int* seq, int* q0, int* n) {
    if (a.query_start != nullptr) {
        int lo = 0, hi = a.num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.query_start[mid] <= qrow) lo = mid;
            else hi = mid - 1;
        }
        *seq = lo;
        *q0 = a.query_start[lo];
        int k = a.query_start[lo + 1] - *q0;
        k = k > a.max_query_len ? a.max_query_len : k;
        if (*q0 < 0 || *q0 > a.num_query_rows) k = 0;
        else if (k > a.num_query_rows - *q0) k = a.num_query_rows - *q0;
        *n = k < 0 ? 0 : k;
    } else {
        *seq = qrow;
        *q0 = qrow;
        *n = 1;
    }
}

// Partitions holding tokens query row r (of n) of a sequence with context L
// attends to (positions 0..L - n + r).
__device__ __forceinline__ int multi_row_partitions(const MultiArgs& a, int seq, int n, int r) {
    const int cap = a.max_blocks_per_seq << a.block_size_log2;
    int L = a.context_lens[seq];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int pos = L - n + r;
    return pos < 0 ? 1 : (pos + a.partition_tokens) / a.partition_tokens;
}

// One workgroup of 64 * W threads per (query row, query head): log-sum-exp
// merge of the partitions that hold tokens the row attends to (positions
// 0..p).
template <int D, int W>
__global__ __launch_bounds__(64 * W) void pa_multi_merge_kernel(MultiArgs a) {
    __shared__ __align__(16) float red[merge_lds_floats<D, W>()];
    const int64_t wid = (int64_t)blockIdx.x;  // query row * Hq + query head
    const int qrow = (int)(wid / a.num_q_heads);
    int seq, q0, n;
    multi_row_owner(a, qrow, &seq, &q0, &n);
    const int r = qrow - q0;
    if (r < 0 || r >= n) return;  // not a row of this sequence's queries (malformed query_start)
    const int np = multi_row_partitions(a, seq, n, r);
    if (np <= 1) return;  // finished by pa_multi_kernel
    const int head = (int)(wid - (int64_t)qrow * a.num_q_heads);
    merge_row<D, W>(a.part_ml + wid * a.num_partitions * 2, a.part_o + wid * a.num_partitions * D, np,
                    nullptr, nullptr, 0, a.out + (int64_t)qrow * a.out_row + (int64_t)head * a.out_head, red);
}

// Few partitions: one thread per (query row, query head, float4 column).
template <int D, int NP>
__global__ __launch_bounds__(256) void pa_multi_merge_flat_kernel(MultiArgs a) {
    constexpr int C = D / 4;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t wid = gid / C;  // query row * Hq + query head
    const int c = (int)(gid - wid * C);
    if (wid >= (int64_t)a.num_query_rows * a.num_q_heads) return;
    const int qrow = (int)(wid / a.num_q_heads);
    int seq, q0, n;
    multi_row_owner(a, qrow, &seq, &q0, &n);
    const int r = qrow - q0;
    if (r < 0 || r >= n) return;
    const int np = multi_row_partitions(a, seq, n, r);
    if (np <= 1) return;  // finished by pa_multi_kernel
    const int head = (int)(wid - (int64_t)qrow * a.num_q_heads);
    merge_column<D, NP>(a.part_ml + wid * a.num_partitions * 2, a.part_o + wid * a.num_partitions * D, np, c,
                        a.out + (int64_t)qrow * a.out_row + (int64_t)head * a.out_head);
}

// Few partitions, with query offsets: the grid walks (sequence, query head,
// block of R = 256 / (D / 4) query rows), one thread per float4 column of a
// row, so the sequence comes from the block index (no search of the
// offsets) and a sequence whose context lies in partition 0, every row of
// it finished by pa_multi_kernel, costs one load.
template <int D, int NP>
__global__ __launch_bounds__(256) void pa_multi_merge_flat_seq_kernel(MultiArgs a, int row_chunks) {
    constexpr int C = D / 4;
    constexpr int R = 256 / C;
    int b = (int)blockIdx.x;
    const int rc = b % row_chunks;
    b /= row_chunks;
    const int head = b % a.num_q_heads;
    const int seq = b / a.num_q_heads;
    const int cap = a.max_blocks_per_seq << a.block_size_log2;
    int L = a.context_lens[seq];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    if (L <= a.partition_tokens) return;
    // the query rows of the sequence, clamped as multi_row_owner clamps them
    const int q0 = a.query_start[seq];
    int n = a.query_start[seq + 1] - q0;
    n = n > a.max_query_len ? a.max_query_len : n;
    if (q0 < 0 || q0 > a.num_query_rows) n = 0;
    else if (n > a.num_query_rows - q0) n = a.num_query_rows - q0;
    const int r = rc * R + (int)threadIdx.x / C;
    if (r >= n) return;
    const int pos = L - n + r;
    const int np = pos < 0 ? 1 : (pos + a.partition_tokens) / a.partition_tokens;
    if (np <= 1) return;  // finished by pa_multi_kernel
    const int64_t wid = (int64_t)(q0 + r) * a.num_q_heads + head;
    merge_column<D, NP>(a.part_ml + wid * a.num_partitions * 2, a.part_o + wid * a.num_partitions * D, np,
                        (int)threadIdx.x % C, a.out + (int64_t)(q0 + r) * a.out_row + (int64_t)head * a.out_head);
}

template <int D, int W>
void launch_merge_w(const MultiArgs& a, int64_t rows, hipStream_t s) {
    hipLaunchKernelGGL((pa_multi_merge_kernel<D, W>), dim3((unsigned)rows), dim3(64 * W), 0, s, a);
}

template <int D>
void launch_multi_merge(const MultiArgs& a, hipStream_t s) {
    const int64_t rows = (int64_t)a.num_query_rows * a.num_q_heads;
    if (a.num_partitions <= kFlatMergeMaxStates) {
        const int64_t row_blocks = (rows * (D / 4) + 255) / 256;
        const int np = flat_merge_states(a.num_partitions);
        constexpr int R = 256 / (D / 4);
        const int chunks = (a.max_query_len + R - 1) / R;
        const int64_t seq_blocks = (int64_t)a.num_seqs * a.num_q_heads * chunks;
        if (a.query_start != nullptr && chunks > 0 && seq_blocks <= 2 * row_blocks) {
            const dim3 grid((unsigned)seq_blocks);
            if (np == 2) hipLaunchKernelGGL((pa_multi_merge_flat_seq_kernel<D, 2>), grid, dim3(256), 0, s, a, chunks);
            else if (np == 4) hipLaunchKernelGGL((pa_multi_merge_flat_seq_kernel<D, 4>), grid, dim3(256), 0, s, a, chunks);
            else hipLaunchKernelGGL((pa_multi_merge_flat_seq_kernel<D, 8>), grid, dim3(256), 0, s, a, chunks);
            return;
        }
        const dim3 grid((unsigned)row_blocks);
        if (np == 2) hipLaunchKernelGGL((pa_multi_merge_flat_kernel<D, 2>), grid, dim3(256), 0, s, a);
        else if (np == 4) hipLaunchKernelGGL((pa_multi_merge_flat_kernel<D, 4>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((pa_multi_merge_flat_kernel<D, 8>), grid, dim3(256), 0, s, a);
        return;
    }
    const int w = merge_waves(D, a.num_partitions, rows);
    if (w <= 1) launch_merge_w<D, 1>(a, rows, s);
    else if (w == 2) launch_merge_w<D, 2>(a, rows, s);
    else if (w == 4) launch_merge_w<D, 4>(a, rows, s);
    else launch_merge_w<D, 8>(a, rows, s);
}

template <int D, bool FP8, int W, int RT>
hipError_t launch_w(const MultiArgs& a, hipStream_t s) {
    // as in the kernel: tiles per ring slot (two unless 1 or 2 waves fall
    // short of a tile's chunks; with one row tile a wave, a 2-slot ring when
    // each lane loads one chunk of each: the 128-register budget; two row
    // tiles have 256 registers and keep 4 slots), query rows' LDS reused by
    // the K/V buffers at 4 or 8 waves or two row tiles
    constexpr int CHUNKS = kTile * (D / (FP8 ? 16 : 8));
    constexpr int MODE = 64 * W >= 2 * CHUNKS ? 0 : ((W >= 4 && 64 * W == CHUNKS) ? 1 : 2);
    constexpr int TPS = MODE == 2 ? 1 : 2;
    constexpr int NB = (W == 1 || MODE == 1 || RT == 2) ? 2 : 4;
    const size_t q_elems = (size_t)16 * W * RT * (D + 8);
    const size_t kv_elems = (size_t)2 * TPS * kTile * (D + 8) + (size_t)2 * TPS * kTile * (D + 16);
    const bool reuse = W >= 4 || RT == 2;
    const size_t lds = (reuse ? (q_elems > kv_elems ? q_elems : kv_elems) : q_elems + kv_elems) * sizeof(uint16_t);
    const dim3 grid((unsigned)((int64_t)a.num_seqs * a.num_kv_heads * a.row_blocks * a.num_partitions));
    hipLaunchKernelGGL((pa_multi_kernel<D, FP8, W, NB, RT>), grid, dim3(64 * W), lds, s, a);
    return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch_df(const MultiArgs& a, int waves, int row_tiles, hipStream_t s) {
    if (row_tiles == 2) return launch_w<D, FP8, 4, 2>(a, s);
    if (waves <= 1) return launch_w<D, FP8, 1, 1>(a, s);
    if (waves == 2) return launch_w<D, FP8, 2, 1>(a, s);
    if (waves == 4) return launch_w<D, FP8, 4, 1>(a, s);
    return launch_w<D, FP8, 8, 1>(a, s);
}

}  // namespace

hipError_t launch_multi(const MultiArgs& a, int head_dim, bool fp8, int waves, int row_tiles, hipStream_t s) {
    hipError_t e;
    if (head_dim == 64)
        e = fp8 ? launch_df<64, true>(a, waves, row_tiles, s) : launch_df<64, false>(a, waves, row_tiles, s);
    else
        e = fp8 ? launch_df<128, true>(a, waves, row_tiles, s) : launch_df<128, false>(a, waves, row_tiles, s);
    if (e != hipSuccess || a.num_partitions == 1 || a.cascade.group_start != nullptr) return e;
    if (head_dim == 64) launch_multi_merge<64>(a, s);
    else launch_multi_merge<128>(a, s);
    return hipGetLastError();
}

}  // namespace pa
