// pa_api.hip -- the C ABI of libpa: argument checks, launch planning and
// kernel dispatch. Host code only; nothing here reads device memory or
// synchronises (unless PA_DEBUG_VALIDATE asks for the checks of validate.hip).
//
// Pages cited (titles as printed at the top of each page):
//   Tutorial = «大模型推理优化与加速完全教程» (LLM inference optimisation tutorial)
//   nanoVLLM = «大模型推理优化技术：从nano-vLLM到连续批处理»
#include <atomic>
#include <climits>
#include <cmath>
#include <cstring>

#include "../../include/pa.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device (cached per device).
int current_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    if (dev < kMaxDevices) {
        const int c = g_cu_count[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return -1;
    if (dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
    return n;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int64_t x) {
    int r = 0;
    while ((int64_t(1) << r) < x) ++r;
    return r;
}
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Plan {
    int variant = PA_VARIANT_VALU;
    int waves = 4;
    int depth = 3;  // register-ring tiles per wave (prefetch distance + 1)
    int partition_tokens = 0;
    int num_partitions = 1;
    bool scheduled = true;
    bool multi = false;          // the multi-row kernel (more than 16 query rows per KV head)
    int heads_per_unit = 1;      // MFMA kernel: adjacent KV heads sharing a 16-row tile
    int row_blocks = 1;          // multi: blocks of 16 * waves rows per (sequence, KV head)
    int64_t num_workgroups = 0;  // direct grid size, or the item bound when scheduled
    // workspace layout (byte offsets); total = workspace
    bool partials = false;       // split-K partial states in the workspace
    size_t items_off = 0, ml_off = 0, o_off = 0;
    size_t workspace = 0;
};

constexpr size_t kHeaderBytes = 256;  // scheduled: item count

int check_sizes(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t MB,
                int32_t kv_dtype) {
    if (S < 0 || Hq <= 0 || Hkv <= 0 || MB <= 0 || bs <= 0 || D <= 0) return PA_ERR_SHAPE;
    if (Hq % Hkv != 0) return PA_ERR_SHAPE;
    if (kv_dtype != PA_KV_BF16 && kv_dtype != PA_KV_FP8_E4M3FN) return PA_ERR_DTYPE;
    if (D != 64 && D != 128) return PA_ERR_UNSUPPORTED;
    const int g = Hq / Hkv;
    if (g > 1024) return PA_ERR_UNSUPPORTED;
    if (!is_pow2(bs) || bs < pa::kTile || bs > 1024) return PA_ERR_UNSUPPORTED;
    const int64_t esz = kv_dtype == PA_KV_BF16 ? 2 : 1;
    if ((int64_t)bs * Hkv * D * esz >= (int64_t(1) << 31)) return PA_ERR_UNSUPPORTED;
    if ((int64_t)MB * bs >= (int64_t(1) << 30)) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

// Tokens per partition for `units` independent workgroup groups over
// contexts of at most `cap` tokens: enough workgroups to fill every
// resident slot (groups_per_cu per CU) twice over, but no split while whole
// contexts already give two per CU and stay short. partition_tokens: 0 =
// choose, -1 = never split, > 0 = forced (a multiple of the tile).
int choose_partition(int64_t units, int64_t cap, int32_t partition_tokens, int groups_per_cu, int64_t* P_out) {
    const int64_t cap16 = align_up((size_t)cap, pa::kTile);
    int64_t P;
    if (partition_tokens > 0) {
        if (partition_tokens % pa::kTile) return PA_ERR_SHAPE;
        P = partition_tokens;
    } else if (partition_tokens < 0) {
        P = cap16;
    } else {
        const int cus = current_cu_count();
        if (cus <= 0) return PA_ERR_DEVICE;
        if (cap <= 4096 && units >= 2 * cus) {
            P = cap16;
        } else {
            P = 4096;
            while (P > 512 && units * ((cap + P - 1) / P) < 2 * (int64_t)groups_per_cu * cus) P /= 2;
        }
    }
    if (P >= cap16) P = cap16;
    *P_out = P;
    return PA_OK;
}

// Plan of the multi-row kernel: Tq query rows in all, at most maxq per
// sequence, g = Hq / Hkv heads per KV head, so at most maxq * g rows per
// (sequence, KV head); one wave per 16 of them, up to 8 waves a workgroup
// (more rows take more workgroups, each reading the K/V again).
int make_multi_plan(int32_t S, int32_t Tq, int32_t maxq, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs,
                    int32_t MB, int32_t partition_tokens, Plan* plan) {
    if (Tq < 0 || maxq < 0) return PA_ERR_SHAPE;
    Plan p;
    p.variant = PA_VARIANT_MFMA;
    p.multi = true;
    p.scheduled = false;
    const int g = Hq / Hkv;
    const int64_t rows = (int64_t)(maxq > 0 ? maxq : 1) * g;
    p.waves = rows <= 16 ? 1 : (rows <= 32 ? 2 : (rows <= 64 ? 4 : 8));
    p.depth = p.waves == 1 ? 2 : 4;  // register ring of the cooperative tile loads
    const int64_t rb = (rows + 16 * p.waves - 1) / (16 * p.waves);
    if (rb >= (int64_t(1) << 20)) return PA_ERR_UNSUPPORTED;
    p.row_blocks = (int)rb;
    const int64_t cap = (int64_t)MB * bs;
    int64_t P = 0;
    // A workgroup of four or more waves already spans the four SIMDs of a
    // CU: one resident group per CU is the target there (measured on 64
    // heads sharing one KV head, 4096 tokens: 1024-token partitions 68 us,
    // 512-token ones 83 us), two for the narrower ones.
    const int st = choose_partition((int64_t)S * Hkv * rb, cap, partition_tokens, p.waves >= 4 ? 1 : 2, &P);
    if (st != PA_OK) return st;
    p.partition_tokens = (int)P;
    p.num_partitions = (int)((cap + P - 1) / P);
    if (p.num_partitions < 1) p.num_partitions = 1;
    p.num_workgroups = (int64_t)S * Hkv * rb * p.num_partitions;
    if (!pa::grid_fits(p.num_workgroups, 64 * p.waves)) return PA_ERR_UNSUPPORTED;
    // Split contexts (long or ragged ones): take items longest first from the
    // device work list. A workgroup here is one cooperative tile stream, so a
    // long item started last would stretch the launch (measured: 8 queries
    // per sequence on a ragged batch, 531 -> 384 us). Unsplit, the direct
    // grid keeps the KV heads of a sequence adjacent, which measured faster.
    p.scheduled = p.num_partitions > 1 && p.num_partitions < 32768 && Hkv < 65536;
    size_t off = 0;
    if (p.scheduled) {
        p.items_off = kHeaderBytes;
        off = p.items_off + align_up((size_t)S * Hkv * p.num_partitions * 4 * sizeof(int32_t), 256);
    }
    if (p.num_partitions > 1) {
        if (!pa::grid_fits((int64_t)Tq * Hq, 512)) return PA_ERR_UNSUPPORTED;  // merge grid: a workgroup of <= 8 waves per row
        const size_t prow = (size_t)Tq * Hq * p.num_partitions;
        p.partials = true;
        p.ml_off = off;
        p.o_off = off + align_up(prow * 2 * sizeof(float), 256);
        off = p.o_off + prow * D * sizeof(float);
    }
    p.workspace = off;
    *plan = p;
    return PA_OK;
}

int make_plan(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t MB, int32_t kv_dtype,
              const pa_decode_opts* opts, Plan* plan) {
    int st = check_sizes(S, Hq, Hkv, D, bs, MB, kv_dtype);
    if (st != PA_OK) return st;
    pa_decode_opts o{};
    if (opts) o = *opts;
    if (o.reserved != 0) return PA_ERR_SHAPE;
    const int g = Hq / Hkv;
    Plan p;
    // Family: matrix tiles once the GQA group fills a useful part of a
    // 16-row tile (g >= 4); below that the dot products stay on the VALU.
    if (o.variant != PA_VARIANT_AUTO && o.variant != PA_VARIANT_VALU && o.variant != PA_VARIANT_MFMA)
        return PA_ERR_SHAPE;
    p.variant = o.variant != PA_VARIANT_AUTO ? o.variant : (g >= 4 ? PA_VARIANT_MFMA : PA_VARIANT_VALU);
    if (p.variant == PA_VARIANT_VALU && g > 4) return PA_ERR_UNSUPPORTED;
    if (o.prefetch_tiles < 0 || o.prefetch_tiles > 3) return PA_ERR_SHAPE;
    if (o.schedule < -1 || o.schedule > 1) return PA_ERR_SHAPE;
    if (o.waves_per_group != 0 && o.waves_per_group != 1 && o.waves_per_group != 2 &&
        o.waves_per_group != 4 && o.waves_per_group != 8)
        return PA_ERR_SHAPE;
    // More query heads per KV head than one 16-row tile holds (MQA): the
    // multi-row kernel, one wave per 16 heads (waves, prefetch and schedule
    // options do not apply to it).
    if (g > 16) return make_multi_plan(S, S, 1, Hq, Hkv, D, bs, MB, o.partition_tokens, plan);
    // Defaults measured on MI355X: the MFMA kernel's tiles are 16 whole K
    // and V rows (8 KiB per wave for bf16, D = 128), so one tile in flight
    // per wave already covers the memory latency; the VALU kernel for g = 1
    // holds fewer bytes per wave and does best with 8 waves, 2 tiles ahead.
    if (p.variant == PA_VARIANT_MFMA) {
        p.waves = 4;
        p.depth = 2;
    } else {
        p.waves = g == 1 ? 8 : 4;
        p.depth = 3;
    }
    if (o.prefetch_tiles < 0 || o.prefetch_tiles > 3) return PA_ERR_SHAPE;
    if (o.prefetch_tiles > 0) p.depth = o.prefetch_tiles + 1;
    if (o.waves_per_group != 0) {
        if (o.waves_per_group != 1 && o.waves_per_group != 2 && o.waves_per_group != 4 &&
            o.waves_per_group != 8)
            return PA_ERR_SHAPE;
        p.waves = o.waves_per_group;
    }
    // MFMA tiles are 16 rows by 16 query-head columns. With g <= 8 a KV
    // head fills at most half of the columns, so 2 adjacent KV heads share a
    // tile, 8 tokens each, and each token's two rows are read as one
    // contiguous chunk (512 bytes for bf16, 256 for fp8, D = 128). Measured
    // on MI355X: 70B batch (g = 8) bf16 79 -> 84 % of peak, fp8 68 -> 74 %;
    // mixed batch (g = 4) bf16 81 -> 86 %; long contexts (g = 4) bf16
    // 72 -> 75 %. fp8 with g = 4 packed gained on long contexts but lost on
    // the mixed batch, and 4 heads of 4-token tiles measured slower than 1:
    // those are only used when asked for. Packed bf16 does best two tiles
    // ahead, packed fp8 one.
    if (o.heads_per_tile != 0 && o.heads_per_tile != 1 && o.heads_per_tile != 2 && o.heads_per_tile != 4)
        return PA_ERR_SHAPE;
    if (p.variant == PA_VARIANT_MFMA) {
        int hp = 1;
        if (o.heads_per_tile != 0) {
            hp = o.heads_per_tile;
            if (g * hp > 16 || Hkv % hp != 0) return PA_ERR_UNSUPPORTED;
        } else if (g <= 8 && Hkv % 2 == 0 && (kv_dtype == PA_KV_BF16 ? g >= 4 : g >= 5)) {
            hp = 2;
            if (o.prefetch_tiles == 0) p.depth = kv_dtype == PA_KV_BF16 ? 3 : 2;
        }
        p.heads_per_unit = hp;
    } else if (o.heads_per_tile > 1) {
        return PA_ERR_UNSUPPORTED;
    }
    const int G = g * p.heads_per_unit;  // query heads per work unit
    // The epilogue stages W * G * (D + 2) floats in LDS; stay within 64 KiB.
    while (p.waves > 1 && (size_t)p.waves * G * (D + 2) * sizeof(float) > 65536) p.waves /= 2;
    const int64_t cap = (int64_t)MB * bs;  // longest context the tables can hold
    const int64_t units = (int64_t)S * (Hkv / p.heads_per_unit);
    int64_t P = 0;
    // Resident workgroups per CU: the MFMA kernel's register budget targets
    // waves per SIMD by ring depth (decode_mfma.hip, mfma_waves_per_eu), one
    // wave per SIMD for 4 waves a workgroup. Measured on the long-context
    // batch (fp8, one KV head per tile, 4 resident): 2048-token partitions
    // 138 us against 151 us for 4096, which a target of 2 per CU kept.
    int groups_per_cu = 2;
    if (p.variant == PA_VARIANT_MFMA) {
        const int base = p.depth <= 2 ? 4 : (p.depth == 3 ? 3 : 2);
        const int wpe = (p.heads_per_unit > 1 && kv_dtype == PA_KV_BF16 && base > 2) ? base - 1 : base;
        groups_per_cu = wpe * 4 / p.waves > 1 ? wpe * 4 / p.waves : 1;
    }
    st = choose_partition(units, cap, o.partition_tokens, groups_per_cu, &P);
    if (st != PA_OK) return st;
    p.partition_tokens = (int)P;
    p.num_partitions = (int)((cap + P - 1) / P);
    if (p.num_partitions < 1) p.num_partitions = 1;
    p.num_workgroups = units * p.num_partitions;
    if (!pa::grid_fits(p.num_workgroups, 64 * p.waves)) return PA_ERR_UNSUPPORTED;
    if (o.schedule < -1 || o.schedule > 1) return PA_ERR_SHAPE;
    // Device work list: by default only when contexts are split. Then most
    // (sequence, partition) pairs of a ragged batch are empty and the real
    // ones differ in length, so a compact longest-first list pays for its
    // pre-pass; an unsplit grid has one workgroup per (sequence, KV head)
    // and no empty ones. Items pack (partition << 16 | KV head) into 32 bits.
    const bool want = o.schedule == 1 || (o.schedule == 0 && p.num_partitions > 1);
    p.scheduled = want && p.num_partitions < 32768 && Hkv / p.heads_per_unit < 65536;
    size_t off = 0;
    if (p.scheduled) {
        p.items_off = kHeaderBytes;
        off = p.items_off + align_up((size_t)p.num_workgroups * 4 * sizeof(int32_t), 256);
    }
    if (p.num_partitions > 1) {
        if (!pa::grid_fits((int64_t)S * Hq, 512)) return PA_ERR_UNSUPPORTED;  // merge grid: a workgroup of <= 8 waves per row
        const size_t rows = (size_t)S * Hq * p.num_partitions;
        p.partials = true;
        p.ml_off = off;
        p.o_off = off + align_up(rows * 2 * sizeof(float), 256);
        off = p.o_off + rows * D * sizeof(float);
    }
    p.workspace = off;
    *plan = p;
    return PA_OK;
}

// Plan of a cascade call: the decode plan for the suffix pass, on the
// device work list (its items start after each sequence's prefix tokens)
// and always with partial states (a sequence with prefix tokens is merged
// even when its suffix is one partition); and, when there are groups, a
// multi-row plan for the prefix pass over G groups of at most maxg member
// sequences, whose states (prefix_partitions slots per row) follow the
// suffix partials in the workspace.
struct CascadePlan {
    Plan suffix;
    Plan prefix;
    bool has_prefix = false;
    size_t pre_ml_off = 0, pre_o_off = 0;
    size_t workspace = 0;
};

int make_cascade_plan(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t MB, int32_t kv_dtype,
                      int32_t G, int32_t maxg, int32_t PMB, const pa_decode_opts* opts, CascadePlan* out) {
    CascadePlan c;
    int st = make_plan(S, Hq, Hkv, D, bs, MB, kv_dtype, opts, &c.suffix);
    if (st != PA_OK) return st;
    if (G < 0 || maxg < 0 || PMB < 0) return PA_ERR_SHAPE;
    if (G >= (int64_t(1) << 30) || (int64_t)PMB * bs >= (int64_t(1) << 30)) return PA_ERR_UNSUPPORTED;
    Plan& p = c.suffix;
    // the suffix pass runs on the decode kernels (at most 16 query heads per KV head)
    if (p.multi) return PA_ERR_UNSUPPORTED;
    if (p.num_partitions >= 32768 || Hkv / p.heads_per_unit >= 65536) return PA_ERR_UNSUPPORTED;
    if (!pa::grid_fits((int64_t)S * Hq, 512)) return PA_ERR_UNSUPPORTED;  // merge grid: a workgroup of <= 8 waves per row
    p.scheduled = true;
    p.partials = true;
    size_t off = kHeaderBytes;
    p.items_off = off;
    off += align_up((size_t)p.num_workgroups * 4 * sizeof(int32_t), 256);
    const size_t rows = (size_t)S * Hq;
    p.ml_off = off;
    p.o_off = off + align_up(rows * p.num_partitions * 2 * sizeof(float), 256);
    off = align_up(p.o_off + rows * p.num_partitions * D * sizeof(float), 256);
    p.workspace = off;
    c.has_prefix = G > 0 && maxg > 0 && PMB > 0;
    if (c.has_prefix) {
        // The groups are few, so the prefix is split into short partitions
        // (down to 64 tokens) until there are about two workgroups per
        // compute unit; each partition adds one state per member row.
        const int cus = current_cu_count();
        if (cus <= 0) return PA_ERR_DEVICE;
        Plan& q = c.prefix;
        st = make_multi_plan(G, S, maxg, Hq, Hkv, D, bs, PMB, -1, &q);
        if (st != PA_OK) return st;
        const int64_t units = (int64_t)G * Hkv * q.row_blocks;
        const int64_t cap = align_up((size_t)PMB * bs, pa::kTile);
        int64_t P = cap;
        while (P > 64 && units * ((cap + P - 1) / P) < 2 * cus) P = align_up((size_t)(P / 2), pa::kTile);
        q.partition_tokens = (int)P;
        q.num_partitions = (int)((cap + P - 1) / P);
        q.num_workgroups = units * q.num_partitions;
        if (!pa::grid_fits(q.num_workgroups, 64 * q.waves)) return PA_ERR_UNSUPPORTED;
        q.scheduled = false;
        q.partials = true;
        q.items_off = 0;
        c.pre_ml_off = off;
        c.pre_o_off = off + align_up(rows * q.num_partitions * 2 * sizeof(float), 256);
        off = c.pre_o_off + rows * q.num_partitions * D * sizeof(float);
        q.ml_off = c.pre_ml_off;
        q.o_off = c.pre_o_off;
        q.workspace = 0;
    }
    c.workspace = off;
    *out = c;
    return PA_OK;
}

int32_t last_block_id(int64_t num_blocks) {
    return (int32_t)((num_blocks > INT32_MAX ? (int64_t)INT32_MAX + 1 : num_blocks) - 1);
}

// Arguments of the multi-row kernel for a plan made by make_multi_plan
// (partials at the plan's workspace offsets when it splits).
pa::MultiArgs multi_args(const Plan& p, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                         float scale, void* out, int32_t S, int32_t Tq, int32_t maxq, int32_t Hq, int32_t Hkv,
                         int32_t D, int32_t bs, int32_t MB, int64_t num_blocks, int32_t kv_dtype, float k_scale,
                         float v_scale, void* workspace) {
    const bool fp8 = kv_dtype == PA_KV_FP8_E4M3FN;
    const int64_t esz = fp8 ? 1 : 2;
    pa::MultiArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k_cache = static_cast<const uint8_t*>(k_cache);
    a.v_cache = static_cast<const uint8_t*>(v_cache);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.query_start = query_start;
    a.out = static_cast<uint16_t*>(out);
    if (p.partials) {
        char* ws = static_cast<char*>(workspace);
        a.part_ml = reinterpret_cast<float*>(ws + p.ml_off);
        a.part_o = reinterpret_cast<float*>(ws + p.o_off);
    }
    a.num_seqs = S;
    a.num_query_rows = Tq;
    a.max_query_len = maxq;
    a.num_q_heads = Hq;
    a.num_kv_heads = Hkv;
    a.group = Hq / Hkv;
    a.block_size_log2 = log2i(bs);
    a.max_blocks_per_seq = MB;
    a.partition_tokens = p.partition_tokens;
    a.num_partitions = p.num_partitions;
    a.row_blocks = p.row_blocks;
    a.last_block = last_block_id(num_blocks);
    a.head_bytes = (uint32_t)(D * esz);
    a.slot_bytes = (uint32_t)((int64_t)Hkv * D * esz);
    a.block_bytes = (uint32_t)((int64_t)bs * Hkv * D * esz);
    a.qk_scale_log2 = scale * (fp8 ? k_scale : 1.0f) * pa::kLog2e;
    a.v_scale = fp8 ? v_scale : 1.0f;
    return a;
}

// Launch the multi-row kernel for a plan made by make_multi_plan.
int run_multi(const Plan& p, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
              float scale, void* out, int32_t S, int32_t Tq, int32_t maxq, int32_t Hq, int32_t Hkv,
              int32_t D, int32_t bs, int32_t MB, int64_t num_blocks, int32_t kv_dtype, float k_scale,
              float v_scale, void* workspace, void* stream) {
    const bool fp8 = kv_dtype == PA_KV_FP8_E4M3FN;
    pa::MultiArgs a = multi_args(p, q, k_cache, v_cache, block_tables, context_lens, query_start, scale, out, S,
                                 Tq, maxq, Hq, Hkv, D, bs, MB, num_blocks, kv_dtype, k_scale, v_scale, workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.scheduled) {
        char* ws = static_cast<char*>(workspace);
        pa::ScheduleArgs sa{};
        sa.context_lens = context_lens;
        sa.items = reinterpret_cast<int4*>(ws + p.items_off);
        sa.item_count = reinterpret_cast<int*>(ws);
        sa.num_seqs = S;
        sa.num_kv_heads = Hkv;
        sa.partition_tokens = p.partition_tokens;
        sa.num_partitions = p.num_partitions;
        sa.max_context = MB * bs;
        if (pa::launch_schedule(sa, s) != hipSuccess) return PA_ERR_LAUNCH;
        a.items = sa.items;
        a.item_count = sa.item_count;
    }
    const hipError_t e = pa::launch_multi(a, D, fp8, p.waves, s);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

// Arguments of the decode kernels for a plan made by make_plan (partials
// and work list at the plan's workspace offsets).
pa::DecodeArgs decode_args(const Plan& p, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens, float scale, void* out,
                           int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t MB,
                           int64_t num_blocks, int32_t kv_dtype, float k_scale, float v_scale, void* workspace) {
    const bool fp8 = kv_dtype == PA_KV_FP8_E4M3FN;
    const int64_t esz = fp8 ? 1 : 2;
    pa::DecodeArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k_cache = static_cast<const uint8_t*>(k_cache);
    a.v_cache = static_cast<const uint8_t*>(v_cache);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = static_cast<uint16_t*>(out);
    char* ws = static_cast<char*>(workspace);
    if (p.partials) {
        a.part_ml = reinterpret_cast<float*>(ws + p.ml_off);
        a.part_o = reinterpret_cast<float*>(ws + p.o_off);
    }
    if (p.scheduled) {
        a.item_count = reinterpret_cast<int*>(ws);
        a.items = reinterpret_cast<const int4*>(ws + p.items_off);
    }
    a.num_seqs = S;
    a.num_q_heads = Hq;
    a.num_kv_heads = Hkv;
    a.group = Hq / Hkv;
    a.units_per_seq = Hkv / p.heads_per_unit;
    a.block_size_log2 = log2i(bs);
    a.max_blocks_per_seq = MB;
    a.partition_tokens = p.partition_tokens;
    a.num_partitions = p.num_partitions;
    a.last_block = last_block_id(num_blocks);
    a.head_bytes = (uint32_t)(D * esz);
    a.slot_bytes = (uint32_t)((int64_t)Hkv * D * esz);
    a.block_bytes = (uint32_t)((int64_t)bs * Hkv * D * esz);
    a.qk_scale_log2 = scale * (fp8 ? k_scale : 1.0f) * pa::kLog2e;
    a.v_scale = fp8 ? v_scale : 1.0f;
    return a;
}

// Arguments of the work-list builder for the decode kernels' items.
pa::ScheduleArgs schedule_args(const Plan& p, const pa::DecodeArgs& a, const int32_t* context_lens,
                               int32_t max_context) {
    pa::ScheduleArgs sa{};
    sa.context_lens = context_lens;
    sa.items = const_cast<int4*>(a.items);
    sa.item_count = const_cast<int*>(a.item_count);
    sa.num_seqs = a.num_seqs;
    sa.num_kv_heads = a.units_per_seq;  // items are (sequence, unit, partition)
    sa.partition_tokens = p.partition_tokens;
    sa.num_partitions = p.num_partitions;
    sa.max_context = max_context;
    sa.block_size_log2 = a.block_size_log2;
    return sa;
}

}  // namespace

extern "C" {

int pa_cache_write(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
                   void* v_cache, int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int64_t num_blocks, int32_t kv_dtype, float k_scale,
                   float v_scale, void* stream) {
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
    if (kv_dtype != PA_KV_BF16 && kv_dtype != PA_KV_FP8_E4M3FN) return PA_ERR_DTYPE;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (!is_pow2(block_size) || block_size > 1024) return PA_ERR_UNSUPPORTED;
    if (kv_dtype == PA_KV_FP8_E4M3FN &&
        (!std::isfinite(k_scale) || !std::isfinite(v_scale) || k_scale <= 0.f || v_scale <= 0.f))
        return PA_ERR_DTYPE;
    if (num_tokens == 0) return PA_OK;
    if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(slot_mapping) & 7u) != 0) return PA_ERR_ALIGN;
    // one thread per 16-byte chunk in a single launch, whose grid counts
    // work-items in 32 bits; divided, not multiplied, so that nothing overflows
    const int64_t chunks_per_token = (int64_t)num_kv_heads * (head_dim / 8);
    if (num_tokens > ((int64_t(1) << 32) - 256) / chunks_per_token) return PA_ERR_UNSUPPORTED;
    if (pa::debug_validate_enabled()) {
        const int vs = pa_check_cache_write_inputs(slot_mapping, num_tokens, block_size, num_blocks, stream);
        if (vs != PA_OK) return vs;
    }
    pa::CacheWriteArgs a{};
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.slot_mapping = slot_mapping;
    a.k_cache = static_cast<uint8_t*>(k_cache);
    a.v_cache = static_cast<uint8_t*>(v_cache);
    a.num_tokens = num_tokens;
    a.num_slots = num_blocks * block_size;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.k_scale = kv_dtype == PA_KV_FP8_E4M3FN ? k_scale : 1.0f;
    a.v_scale = kv_dtype == PA_KV_FP8_E4M3FN ? v_scale : 1.0f;
    const hipError_t e =
        pa::launch_cache_write(a, kv_dtype == PA_KV_FP8_E4M3FN, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int64_t num_pairs,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                   int32_t kv_dtype, void* stream) {
    if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
    if (kv_dtype != PA_KV_BF16 && kv_dtype != PA_KV_FP8_E4M3FN) return PA_ERR_DTYPE;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (!is_pow2(block_size) || block_size > 1024) return PA_ERR_UNSUPPORTED;
    if (!pa::grid_fits(num_pairs, pa::kCopyThreads)) return PA_ERR_UNSUPPORTED;
    if (num_pairs == 0) return PA_OK;
    if (!k_cache || !v_cache || !block_mapping) return PA_ERR_NULL;
    if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(block_mapping) & 7u) != 0) return PA_ERR_ALIGN;
    pa::CopyBlocksArgs a{};
    a.k_cache = static_cast<uint8_t*>(k_cache);
    a.v_cache = static_cast<uint8_t*>(v_cache);
    a.pairs = block_mapping;
    a.num_pairs = num_pairs;
    a.num_blocks = num_blocks;
    a.block_bytes = (int64_t)block_size * num_kv_heads * head_dim * (kv_dtype == PA_KV_BF16 ? 2 : 1);
    const hipError_t e = pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_decode_get_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t max_blocks_per_seq, int32_t kv_dtype,
                       const pa_decode_opts* opts, pa_decode_plan* plan) {
    if (!plan) return PA_ERR_NULL;
    Plan p;
    const int st = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                             max_blocks_per_seq, kv_dtype, opts, &p);
    if (st != PA_OK) return st;
    plan->variant = p.variant;
    plan->waves_per_group = p.waves;
    plan->partition_tokens = p.partition_tokens;
    plan->num_partitions = p.num_partitions;
    plan->prefetch_tiles = p.depth - 1;
    plan->scheduled = p.scheduled ? 1 : 0;
    plan->num_workgroups = p.num_workgroups;
    plan->workspace_bytes = p.workspace;
    plan->heads_per_tile = p.heads_per_unit;
    return PA_OK;
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t kv_dtype, const pa_decode_opts* opts) {
    Plan p;
    if (make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                  kv_dtype, opts, &p) != PA_OK)
        return 0;
    return p.workspace;
}

int pa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
              const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
              int32_t max_blocks_per_seq, int64_t num_blocks, int32_t kv_dtype, float k_scale,
              float v_scale, void* workspace, size_t workspace_bytes, const pa_decode_opts* opts,
              void* stream) {
    Plan p;
    int st = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                       kv_dtype, opts, &p);
    if (st != PA_OK) return st;
    if (num_blocks <= 0) return PA_ERR_SHAPE;
    if (!std::isfinite(scale)) return PA_ERR_SHAPE;
    const bool fp8 = kv_dtype == PA_KV_FP8_E4M3FN;
    if (fp8 && (!std::isfinite(k_scale) || !std::isfinite(v_scale) || k_scale <= 0.f || v_scale <= 0.f))
        return PA_ERR_DTYPE;
    if (num_seqs == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return PA_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(block_tables) & 3u) || (reinterpret_cast<uintptr_t>(context_lens) & 3u))
        return PA_ERR_ALIGN;
    if (p.workspace > 0) {
        if (!workspace || workspace_bytes < p.workspace) return PA_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_ALIGN;
    }
    if (pa::debug_validate_enabled()) {
        const int vs = pa_check_decode_inputs(block_tables, context_lens, num_seqs, block_size,
                                              max_blocks_per_seq, num_blocks, stream);
        if (vs != PA_OK) return vs;
    }
    if (p.multi)
        return run_multi(p, q, k_cache, v_cache, block_tables, context_lens, nullptr, scale, out, num_seqs,
                         num_seqs, 1, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                         num_blocks, kv_dtype, k_scale, v_scale, workspace, stream);
    pa::DecodeArgs a = decode_args(p, q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                                   num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                   num_blocks, kv_dtype, k_scale, v_scale, workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (p.scheduled) {
        const pa::ScheduleArgs sa = schedule_args(p, a, context_lens, max_blocks_per_seq * block_size);
        e = pa::launch_schedule(sa, s);
        if (e != hipSuccess) return PA_ERR_LAUNCH;
    }
    const pa::LaunchShape ls{p.waves, p.depth, p.heads_per_unit};
    e = p.variant == PA_VARIANT_MFMA ? pa::launch_decode_mfma(a, head_dim, fp8, ls, s)
                                     : pa::launch_decode_valu(a, head_dim, fp8, ls, s);
    if (e != hipSuccess) return PA_ERR_LAUNCH;
    if (p.num_partitions > 1) {
        pa::MergeArgs m{};
        m.context_lens = context_lens;
        m.part_ml = a.part_ml;
        m.part_o = a.part_o;
        m.out = a.out;
        m.num_seqs = num_seqs;
        m.num_q_heads = num_q_heads;
        m.head_dim = head_dim;
        m.partition_tokens = p.partition_tokens;
        m.num_partitions = p.num_partitions;
        m.max_context = max_blocks_per_seq * block_size;
        e = pa::launch_merge(m, s);
        if (e != hipSuccess) return PA_ERR_LAUNCH;
    }
    return PA_OK;
}

size_t pa_decode_cascade_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                        int32_t num_groups, int32_t max_group_size, int32_t max_prefix_blocks,
                                        int32_t kv_dtype, const pa_decode_opts* opts) {
    CascadePlan c;
    if (make_cascade_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                          kv_dtype, num_groups, max_group_size, max_prefix_blocks, opts, &c) != PA_OK)
        return 0;
    return c.workspace;
}

int pa_decode_cascade(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, const int32_t* prefix_tables, const int32_t* prefix_lens,
                      const int32_t* group_start, float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                      int64_t num_blocks, int32_t num_groups, int32_t max_group_size, int32_t max_prefix_blocks,
                      int32_t kv_dtype, float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                      const pa_decode_opts* opts, void* stream) {
    CascadePlan c;
    int st = make_cascade_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                               kv_dtype, num_groups, max_group_size, max_prefix_blocks, opts, &c);
    if (st != PA_OK) return st;
    if (num_blocks <= 0) return PA_ERR_SHAPE;
    if (!std::isfinite(scale)) return PA_ERR_SHAPE;
    const bool fp8 = kv_dtype == PA_KV_FP8_E4M3FN;
    if (fp8 && (!std::isfinite(k_scale) || !std::isfinite(v_scale) || k_scale <= 0.f || v_scale <= 0.f))
        return PA_ERR_DTYPE;
    if (num_seqs == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PA_ERR_NULL;
    if (c.has_prefix && (!prefix_tables || !prefix_lens || !group_start)) return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return PA_ERR_ALIGN;
    const auto mis4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) != 0; };
    if (mis4(block_tables) || mis4(context_lens) || mis4(prefix_tables) || mis4(prefix_lens) || mis4(group_start))
        return PA_ERR_ALIGN;
    if (!workspace || workspace_bytes < c.workspace) return PA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_ALIGN;
    if (pa::debug_validate_enabled()) {
        int vs = pa_check_decode_inputs(block_tables, context_lens, num_seqs, block_size, max_blocks_per_seq,
                                        num_blocks, stream);
        if (vs == PA_OK && c.has_prefix)
            vs = pa_check_cascade_inputs(prefix_tables, prefix_lens, group_start, num_groups, max_group_size,
                                         max_prefix_blocks, num_seqs, block_size, num_blocks, stream);
        if (vs != PA_OK) return vs;
    }
    pa::CascadeGroups groups{};
    if (c.has_prefix) {
        groups.group_start = group_start;
        groups.prefix_lens = prefix_lens;
        groups.num_groups = num_groups;
        groups.max_group_size = max_group_size;
        groups.max_prefix_tokens = max_prefix_blocks * block_size;
        groups.max_context = max_blocks_per_seq * block_size;
    }
    const Plan& p = c.suffix;
    const pa::DecodeArgs a = decode_args(p, q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                                         num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                         num_blocks, kv_dtype, k_scale, v_scale, workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // 1. suffix work list
    pa::ScheduleArgs sa = schedule_args(p, a, context_lens, max_blocks_per_seq * block_size);
    sa.cascade = groups;
    if (pa::launch_schedule(sa, s) != hipSuccess) return PA_ERR_LAUNCH;
    // 2. prefix pass: each group's prefix once for all its members
    pa::MultiArgs m{};
    if (c.has_prefix) {
        m = multi_args(c.prefix, q, k_cache, v_cache, prefix_tables, context_lens, nullptr, scale, out,
                       num_groups, num_seqs, max_group_size, num_q_heads, num_kv_heads, head_dim, block_size,
                       max_prefix_blocks, num_blocks, kv_dtype, k_scale, v_scale, workspace);
        m.cascade = groups;
        if (pa::launch_multi(m, head_dim, fp8, c.prefix.waves, s) != hipSuccess) return PA_ERR_LAUNCH;
    }
    // 3. suffix pass
    const pa::LaunchShape ls{p.waves, p.depth, p.heads_per_unit};
    const hipError_t e = p.variant == PA_VARIANT_MFMA ? pa::launch_decode_mfma(a, head_dim, fp8, ls, s)
                                                      : pa::launch_decode_valu(a, head_dim, fp8, ls, s);
    if (e != hipSuccess) return PA_ERR_LAUNCH;
    // 4. merge both passes' states
    pa::CascadeMergeArgs mg{};
    mg.context_lens = context_lens;
    mg.cascade = groups;
    mg.pre_ml = m.part_ml;
    mg.pre_o = m.part_o;
    mg.part_ml = a.part_ml;
    mg.part_o = a.part_o;
    mg.out = a.out;
    mg.num_seqs = num_seqs;
    mg.num_q_heads = num_q_heads;
    mg.head_dim = head_dim;
    mg.prefix_partition_tokens = c.has_prefix ? c.prefix.partition_tokens : 1;
    mg.prefix_partitions = c.has_prefix ? c.prefix.num_partitions : 0;
    mg.partition_tokens = p.partition_tokens;
    mg.num_partitions = p.num_partitions;
    mg.max_context = max_blocks_per_seq * block_size;
    mg.block_size_log2 = a.block_size_log2;
    return pa::launch_cascade_merge(mg, s) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

size_t pa_decode_multi_workspace_size(int32_t num_seqs, int32_t num_query_tokens, int32_t max_query_len,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq, int32_t kv_dtype,
                                      int32_t partition_tokens) {
    if (check_sizes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, kv_dtype) != PA_OK)
        return 0;
    Plan p;
    if (make_multi_plan(num_seqs, num_query_tokens, max_query_len, num_q_heads, num_kv_heads, head_dim,
                        block_size, max_blocks_per_seq, partition_tokens, &p) != PA_OK)
        return 0;
    return p.workspace;
}

int pa_decode_multi(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                    const int32_t* context_lens, const int32_t* query_start, float scale, void* out,
                    int32_t num_seqs, int32_t num_query_tokens, int32_t max_query_len, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                    int64_t num_blocks, int32_t kv_dtype, float k_scale, float v_scale, void* workspace,
                    size_t workspace_bytes, int32_t partition_tokens, void* stream) {
    int st = check_sizes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, kv_dtype);
    if (st != PA_OK) return st;
    if (num_query_tokens < 0 || max_query_len < 0) return PA_ERR_SHAPE;
    if (num_blocks <= 0 || !std::isfinite(scale)) return PA_ERR_SHAPE;
    const bool fp8 = kv_dtype == PA_KV_FP8_E4M3FN;
    if (fp8 && (!std::isfinite(k_scale) || !std::isfinite(v_scale) || k_scale <= 0.f || v_scale <= 0.f))
        return PA_ERR_DTYPE;
    Plan p;
    st = make_multi_plan(num_seqs, num_query_tokens, max_query_len, num_q_heads, num_kv_heads, head_dim,
                         block_size, max_blocks_per_seq, partition_tokens, &p);
    if (st != PA_OK) return st;
    if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out) return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return PA_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(block_tables) & 3u) || (reinterpret_cast<uintptr_t>(context_lens) & 3u) ||
        (reinterpret_cast<uintptr_t>(query_start) & 3u))
        return PA_ERR_ALIGN;
    if (p.workspace > 0) {
        if (!workspace || workspace_bytes < p.workspace) return PA_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_ALIGN;
    }
    if (pa::debug_validate_enabled()) {
        const int vs = pa_check_decode_inputs(block_tables, context_lens, num_seqs, block_size,
                                              max_blocks_per_seq, num_blocks, stream);
        if (vs != PA_OK) return vs;
    }
    return run_multi(p, q, k_cache, v_cache, block_tables, context_lens, query_start, scale, out, num_seqs,
                     num_query_tokens, max_query_len, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, num_blocks, kv_dtype, k_scale, v_scale, workspace, stream);
}

int pa_probe_stream_read(const void* buf, int64_t bytes, int32_t nontemporal, uint32_t* sink, void* stream) {
    if (bytes < 0 || (bytes & 15) != 0) return PA_ERR_SHAPE;
    if (bytes == 0) return PA_OK;
    if (!buf || !sink) return PA_ERR_NULL;
    if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return PA_ERR_ALIGN;
    const int cus = current_cu_count();
    if (cus <= 0) return PA_ERR_DEVICE;
    const hipError_t e = pa::launch_probe_read(buf, bytes, nontemporal != 0, sink, cus, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

void pa_fp8_e4m3fn_encode_host(const float* x, uint8_t* codes, int64_t n) {
    if (!x || !codes) return;
    for (int64_t i = 0; i < n; ++i) codes[i] = pa::fp8_e4m3fn_encode(x[i]);
}

const char* pa_strerror(int status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_NULL: return "a required pointer is NULL";
        case PA_ERR_SHAPE: return "a size is out of range or inconsistent";
        case PA_ERR_UNSUPPORTED: return "valid but not supported by the kernels";
        case PA_ERR_ALIGN: return "a pointer is not suitably aligned";
        case PA_ERR_DTYPE: return "unknown kv dtype or bad fp8 scale";
        case PA_ERR_WORKSPACE: return "workspace missing or too small";
        case PA_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
        case PA_ERR_DEVICE: return "the current HIP device could not be queried";
        case PA_ERR_PRECONDITION: return "a device-side input violates a precondition (slots, tables or lengths)";
        default: return "unknown status";
    }
}

int pa_version(void) { return 100; }

}  // extern "C"
