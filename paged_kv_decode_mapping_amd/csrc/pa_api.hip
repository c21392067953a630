// pa_api.hip -- the C ABI of libpa: argument checks, launch planning and
// kernel dispatch. Host code only; nothing here reads device memory or
// synchronises (unless PA_DEBUG_VALIDATE asks for the checks of validate.hip).
// The pa_tensor arguments are read by pa_abi.h.
//
// Pages cited (titles as printed at the top of each page):
//   Tutorial = «大模型推理优化与加速完全教程» (LLM inference optimisation tutorial)
//   nanoVLLM = «大模型推理优化技术：从nano-vLLM到连续批处理»
#include <atomic>
#include <climits>
#include <cmath>
#include <cstring>

#include "pa_abi.h"
#include "pa_device.h"

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

using pa::abi::is_pow2;
using pa::abi::log2i;
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Plan {
    int variant = PA_VARIANT_VALU;
    int waves = 4;
    int depth = 3;  // register-ring tiles per wave (prefetch distance + 1)
    int partition_tokens = 0;
    int num_partitions = 1;
    bool scheduled = true;
    bool self_scheduled = false; // scheduled, each workgroup finding its own item (no builder pass)
    bool multi = false;          // the multi-row kernel (more than 16 query rows per KV head)
    int heads_per_unit = 1;      // MFMA kernel: adjacent KV heads sharing a 16-row tile
    bool wave_partitions = false; // MFMA kernel: each wave takes one whole partition
    int num_items = 1;           // work items per (sequence, unit): partitions, or groups of W
    int row_tiles = 1;           // multi: 16-row matrix tiles per wave (1 or 2)
    int row_blocks = 1;          // multi: blocks of 16 * waves * row_tiles rows per (sequence, KV head)
    int64_t num_workgroups = 0;  // direct grid size, or the item bound when scheduled
    // workspace layout (byte offsets); total = workspace
    bool partials = false;       // split-K partial states in the workspace
    size_t items_off = 0, ml_off = 0, o_off = 0;
    size_t workspace = 0;
};

constexpr size_t kHeaderBytes = 256;  // scheduled: item count
constexpr int64_t kSelfMaxPairs = 1024;  // default self-scheduling: grid size bound (see make_plan)

int check_sizes(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t MB,
                int32_t kv_dtype) {
    if (S < 0 || Hq <= 0 || Hkv <= 0 || MB <= 0 || bs <= 0 || D <= 0) return PA_ERR_SHAPE;
    if (Hq % Hkv != 0) return PA_ERR_SHAPE;
    if (kv_dtype != PA_DTYPE_BF16 && kv_dtype != PA_DTYPE_FP8_E4M3FN) return PA_ERR_DTYPE;
    if (D != 64 && D != 128) return PA_ERR_UNSUPPORTED;
    const int g = Hq / Hkv;
    if (g > 1024) return PA_ERR_UNSUPPORTED;
    if (!is_pow2(bs) || bs < pa::kTile || bs > 1024) return PA_ERR_UNSUPPORTED;
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
// (sequence, KV head); one wave per 16 of them up to 64 rows, one per 32
// beyond (every wave reads the whole staged tile from LDS, so fewer, wider
// waves read less of it), up to 8 waves a workgroup (more rows take more
// workgroups, each reading the K/V again).
int make_multi_plan(int32_t S, int32_t Tq, int32_t maxq, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs,
                    int32_t MB, int32_t partition_tokens, Plan* plan, int32_t schedule = 0) {
    if (Tq < 0 || maxq < 0) return PA_ERR_SHAPE;
    Plan p;
    p.variant = PA_VARIANT_MFMA;
    p.multi = true;
    p.scheduled = false;
    const int g = Hq / Hkv;
    const int64_t rows = (int64_t)(maxq > 0 ? maxq : 1) * g;
    p.row_tiles = rows > 64 ? 2 : 1;
    p.waves = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
    p.depth = p.waves == 1 ? 2 : 4;  // register ring of the cooperative tile loads
    const int64_t block_rows = (int64_t)16 * p.waves * p.row_tiles;
    const int64_t rb = (rows + block_rows - 1) / block_rows;
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
    p.scheduled = p.num_partitions > 1 && p.num_partitions < 32768 && Hkv < 65536 && schedule >= 0;
    // The longest-first order without the builder pass, by the rule of the
    // decode kernels (make_plan): one wave ranks the batch, small grids.
    // Measured on MQA (128 sequences of 4096 tokens, one KV head, 64 query
    // heads, 1024-token partitions): the builder pass and its launch gap
    // cost more than the workgroups' own search.
    const bool self_ok = S <= pa::kSelfWaveSeqs && P / pa::kTile + 1 <= pa::kSelfBuckets;
    p.self_scheduled = p.scheduled && self_ok &&
                       (schedule == 2 || (schedule == 0 && (int64_t)S * p.num_partitions <= kSelfMaxPairs));
    size_t off = 0;
    if (p.scheduled && !p.self_scheduled) {
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

// heads_adjacent: a token row's KV heads are one contiguous run (the head
// stride is head_dim), which packing several KV heads into a tile needs.
int make_plan(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t MB, int32_t kv_dtype,
              bool heads_adjacent, const pa_decode_opts* opts, Plan* plan, bool allow_wave_partitions = true) {
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
    if (o.schedule < -1 || o.schedule > 2) return PA_ERR_SHAPE;
    if (o.waves_per_group != 0 && o.waves_per_group != 1 && o.waves_per_group != 2 &&
        o.waves_per_group != 4 && o.waves_per_group != 8)
        return PA_ERR_SHAPE;
    // More query heads per KV head than one 16-row tile holds (MQA): the
    // multi-row kernel, one wave per 16 heads (waves, prefetch and schedule
    // options do not apply to it).
    if (g > 16) return make_multi_plan(S, S, 1, Hq, Hkv, D, bs, MB, o.partition_tokens, plan, o.schedule);
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
            if (g * hp > 16 || Hkv % hp != 0 || (hp > 1 && !heads_adjacent)) return PA_ERR_UNSUPPORTED;
        } else if (g <= 8 && Hkv % 2 == 0 && heads_adjacent && (kv_dtype == PA_DTYPE_BF16 ? g >= 4 : g >= 5)) {
            hp = 2;
            if (o.prefetch_tiles == 0) p.depth = kv_dtype == PA_DTYPE_BF16 ? 3 : 2;
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
        const int wpe = (p.heads_per_unit > 1 && kv_dtype == PA_DTYPE_BF16 && base > 2) ? base - 1 : base;
        groups_per_cu = wpe * 4 / p.waves > 1 ? wpe * 4 / p.waves : 1;
    }
    st = choose_partition(units, cap, o.partition_tokens, groups_per_cu, &P);
    if (st != PA_OK) return st;
    p.partition_tokens = (int)P;
    p.num_partitions = (int)((cap + P - 1) / P);
    if (p.num_partitions < 1) p.num_partitions = 1;
    // One partition per wave: a workgroup covers W consecutive partitions,
    // each wave streaming one of them and storing its state, instead of
    // the W waves sharing one partition's tiles and combining in LDS. This
    // amortises a workgroup's set-up (query rows, first loads, combine) over
    // W times the bytes. Measured on MI355X: fp8 caches with 512-token
    // partitions gain 4-6 % (long contexts 137.6 -> 131.6 us, mixed batch
    // 169.0 -> 158.3 us); bf16 at 512 tokens is unchanged, and with longer
    // partitions (1024-4096 tokens) it loses, as one wave then streams a
    // whole long partition by itself.
    if (o.wave_partitions < -1 || o.wave_partitions > 1) return PA_ERR_SHAPE;
    const bool wpp_ok = p.variant == PA_VARIANT_MFMA && p.heads_per_unit <= 2 && p.depth <= 3 &&
                        allow_wave_partitions;
    if (o.wave_partitions == 1 && !wpp_ok) return PA_ERR_UNSUPPORTED;
    p.wave_partitions = p.num_partitions > 1 && p.waves > 1 && wpp_ok &&
                        (o.wave_partitions == 1 ||
                         (o.wave_partitions == 0 && kv_dtype == PA_DTYPE_FP8_E4M3FN && P <= 512));
    p.num_items = p.wave_partitions ? (p.num_partitions + p.waves - 1) / p.waves : p.num_partitions;
    p.num_workgroups = units * p.num_items;
    if (!pa::grid_fits(p.num_workgroups, 64 * p.waves)) return PA_ERR_UNSUPPORTED;
    if (o.schedule < -1 || o.schedule > 2) return PA_ERR_SHAPE;
    // Longest-first items: by default only when contexts are split. Then
    // most (sequence, partition) pairs of a ragged batch are empty and the
    // real ones differ in length, so a compact longest-first order pays for
    // finding it; an unsplit grid has one workgroup per (sequence, KV head)
    // and no empty ones. The order comes either from a one-workgroup builder
    // pass that writes the list to the workspace (items pack partition << 16
    // | KV head into 32 bits), or from each decode workgroup itself, which
    // counts the items of context_lens by length in LDS and ranks its block
    // index among them -- no extra launch, at the cost of reading
    // context_lens in every workgroup, so only for batches of up to
    // kSelfMaxSeqs sequences.
    const bool want = o.schedule >= 1 || (o.schedule == 0 && p.num_partitions > 1);
    p.scheduled = want && p.num_partitions < 32768 && Hkv / p.heads_per_unit < 65536;
    const int64_t span = P * (p.wave_partitions ? p.waves : 1);
    const bool self_ok = S <= pa::kSelfMaxSeqs && span % pa::kTile == 0 && span / pa::kTile + 1 <= pa::kSelfBuckets;
    if (o.schedule == 2 && !self_ok) return PA_ERR_UNSUPPORTED;
    // By default when one wave ranks the batch (at most kSelfWaveSeqs
    // sequences) and the grid holds at most kSelfMaxPairs (sequence, item)
    // pairs: every workgroup of the grid, real item or not, first reads
    // context_lens, so the search pays where the grid is small against the
    // work. Measured on MI355X (decode + merge, % of 8 TB/s, list -> self):
    // long contexts (4 sequences) bf16 at 2048-token partitions 75.7 -> 76.9,
    // at 512 71.9 -> 73.4, fp8 69.3 -> 70.5; mixed batch (256 sequences, 2
    // partitions) bf16 85.7 -> 86.3, fp8 71-78 -> 77.8; the 70B batch at 512
    // tokens (1024 pairs) even; but the mixed batch at 512-token partitions
    // (4096 pairs, ~3800 real items) 75.0 -> 68.6.
    const int64_t pairs = (int64_t)S * p.num_items;
    p.self_scheduled = p.scheduled && self_ok &&
                       (o.schedule == 2 || (o.schedule == 0 && S <= pa::kSelfWaveSeqs && pairs <= kSelfMaxPairs));
    size_t off = 0;
    if (p.scheduled && !p.self_scheduled) {
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
                      bool heads_adjacent, int32_t G, int32_t maxg, int32_t PMB, const pa_decode_opts* opts,
                      CascadePlan* out) {
    CascadePlan c;
    int st = make_plan(S, Hq, Hkv, D, bs, MB, kv_dtype, heads_adjacent, opts, &c.suffix, false);
    if (st != PA_OK) return st;
    if (G < 0 || maxg < 0 || PMB < 0) return PA_ERR_SHAPE;
    if (G >= (int64_t(1) << 30) || (int64_t)PMB * bs >= (int64_t(1) << 30)) return PA_ERR_UNSUPPORTED;
    Plan& p = c.suffix;
    // the suffix pass runs on the decode kernels (at most 16 query heads per KV head)
    if (p.multi) return PA_ERR_UNSUPPORTED;
    if (p.num_partitions >= 32768 || Hkv / p.heads_per_unit >= 65536) return PA_ERR_UNSUPPORTED;
    if (!pa::grid_fits((int64_t)S * Hq, 512)) return PA_ERR_UNSUPPORTED;  // merge grid: a workgroup of <= 8 waves per row
    p.scheduled = true;
    p.self_scheduled = false;  // the builder also offsets items past each sequence's prefix
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

bool scales_ok(int kv_dtype, float k_scale, float v_scale) {
    return kv_dtype != PA_DTYPE_FP8_E4M3FN ||
           (std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f);
}

int check_workspace(size_t need, const void* workspace, size_t workspace_bytes) {
    if (need == 0) return PA_OK;
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_ALIGN;
    return PA_OK;
}

// What a decode-family call reads from its tensors: the query rows (and the
// output rows, for the calls that run), the paged caches, the tables and
// the context lengths.
struct Geom {
    pa::abi::Rows q{}, out{};
    pa::abi::Cache cache{};
    const uint8_t* v_cache = nullptr;
    pa::abi::Table tables{};
    const int32_t* context_lens = nullptr;
    int32_t S = 0, Hq = 0, Hkv = 0, D = 0, bs = 0, MB = 0;
    int64_t N = 0;
};

// The shapes a plan needs: q [S (or query rows), Hq, D], the K cache and
// the tables [S, MB]. num_seqs is the tables' row count. need_data: the
// call runs (a plan reads shapes, types and strides only).
int plan_geom(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* block_tables, Geom* g,
              bool need_data = false) {
    int st = pa::abi::rows(q, false, &g->q, need_data);
    if (st != PA_OK) return st;
    st = pa::abi::cache(k_cache, &g->cache, need_data);
    if (st != PA_OK) return st;
    st = pa::abi::table(block_tables, &g->tables, need_data);
    if (st != PA_OK) return st;
    g->S = (int32_t)g->tables.rows;
    g->Hq = g->q.heads;
    g->D = g->q.dim;
    g->Hkv = g->cache.Hkv;
    g->bs = g->cache.bs;
    g->MB = g->tables.cols;
    g->N = g->cache.N;
    if (g->D != g->cache.D) return PA_ERR_SHAPE;
    return PA_OK;
}

// Everything a running call needs: plan_geom, the V cache (same layout),
// context_lens [S] and out (q's shape, written).
int run_geom(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache, const pa_tensor* block_tables,
             const pa_tensor* context_lens, const pa_tensor* out, Geom* g) {
    int st = plan_geom(q, k_cache, block_tables, g, true);
    if (st != PA_OK) return st;
    st = pa::abi::caches(k_cache, v_cache, &g->cache);
    if (st != PA_OK) return st;
    g->v_cache = static_cast<const uint8_t*>(v_cache->data);
    int64_t n = 0;
    st = pa::abi::vec(context_lens, PA_DTYPE_I32, &g->context_lens, &n);
    if (st != PA_OK) return st;
    if (n != g->S) return PA_ERR_SHAPE;
    st = pa::abi::rows(out, true, &g->out);
    if (st != PA_OK) return st;
    if (g->out.rows != g->q.rows || g->out.heads != g->q.heads || g->out.dim != g->q.dim) return PA_ERR_SHAPE;
    return PA_OK;
}

// Arguments of the multi-row kernel for a plan made by make_multi_plan
// (partials at the plan's workspace offsets when it splits). `tables` and
// `S` are the pass's own: the batch's, or the prefix groups' in a cascade.
pa::MultiArgs multi_args(const Plan& p, const Geom& g, const pa::abi::Table& tables, int32_t S,
                         const int32_t* query_start, int32_t Tq, int32_t maxq, float scale, int32_t kv_dtype,
                         float k_scale, float v_scale, void* workspace) {
    const bool fp8 = kv_dtype == PA_DTYPE_FP8_E4M3FN;
    pa::MultiArgs a{};
    a.q = static_cast<const uint16_t*>(g.q.data);
    a.k_cache = g.cache.data;
    a.v_cache = g.v_cache;
    a.block_tables = tables.data;
    a.table_stride = tables.stride;
    a.context_lens = g.context_lens;
    a.query_start = query_start;
    a.out = static_cast<uint16_t*>(g.out.data);
    a.q_row = g.q.s_row;
    a.q_head = g.q.s_head;
    a.out_row = g.out.s_row;
    a.out_head = g.out.s_head;
    if (p.partials) {
        char* ws = static_cast<char*>(workspace);
        a.part_ml = reinterpret_cast<float*>(ws + p.ml_off);
        a.part_o = reinterpret_cast<float*>(ws + p.o_off);
    }
    a.num_seqs = S;
    a.num_query_rows = Tq;
    a.max_query_len = maxq;
    a.num_q_heads = g.Hq;
    a.num_kv_heads = g.Hkv;
    a.group = g.Hq / g.Hkv;
    a.block_size_log2 = log2i(g.bs);
    a.max_blocks_per_seq = tables.cols;
    a.partition_tokens = p.partition_tokens;
    a.num_partitions = p.num_partitions;
    a.row_blocks = p.row_blocks;
    a.last_block = last_block_id(g.N);
    a.cache = g.cache.lay;
    a.qk_scale_log2 = scale * (fp8 ? k_scale : 1.0f) * pa::kLog2e;
    a.v_scale = fp8 ? v_scale : 1.0f;
    return a;
}

// Launch the multi-row kernel for a plan made by make_multi_plan.
int run_multi(const Plan& p, const Geom& g, const int32_t* query_start, int32_t Tq, int32_t maxq, float scale,
              int32_t kv_dtype, float k_scale, float v_scale, void* workspace, void* stream) {
    pa::MultiArgs a =
        multi_args(p, g, g.tables, g.S, query_start, Tq, maxq, scale, kv_dtype, k_scale, v_scale, workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    a.self_schedule = p.self_scheduled ? 1 : 0;
    if (p.scheduled && !p.self_scheduled) {
        char* ws = static_cast<char*>(workspace);
        pa::ScheduleArgs sa{};
        sa.context_lens = g.context_lens;
        sa.items = reinterpret_cast<int4*>(ws + p.items_off);
        sa.item_count = reinterpret_cast<int*>(ws);
        sa.num_seqs = g.S;
        sa.num_kv_heads = g.Hkv;
        sa.partition_tokens = p.partition_tokens;
        sa.num_partitions = p.num_partitions;
        sa.split_tokens = p.partition_tokens;
        sa.split_count = p.num_partitions;
        sa.max_context = g.MB * g.bs;
        if (pa::launch_schedule(sa, s) != hipSuccess) return PA_ERR_LAUNCH;
        a.items = sa.items;
        a.item_count = sa.item_count;
    }
    const hipError_t e = pa::launch_multi(a, g.D, kv_dtype == PA_DTYPE_FP8_E4M3FN, p.waves, p.row_tiles, s);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

// Arguments of the decode kernels for a plan made by make_plan (partials
// and work list at the plan's workspace offsets).
pa::DecodeArgs decode_args(const Plan& p, const Geom& g, float scale, int32_t kv_dtype, float k_scale,
                           float v_scale, void* workspace) {
    const bool fp8 = kv_dtype == PA_DTYPE_FP8_E4M3FN;
    pa::DecodeArgs a{};
    a.q = static_cast<const uint16_t*>(g.q.data);
    a.k_cache = g.cache.data;
    a.v_cache = g.v_cache;
    a.block_tables = g.tables.data;
    a.table_stride = g.tables.stride;
    a.context_lens = g.context_lens;
    a.out = static_cast<uint16_t*>(g.out.data);
    a.q_seq = g.q.s_row;
    a.q_head = g.q.s_head;
    a.out_seq = g.out.s_row;
    a.out_head = g.out.s_head;
    char* ws = static_cast<char*>(workspace);
    if (p.partials) {
        a.part_ml = reinterpret_cast<float*>(ws + p.ml_off);
        a.part_o = reinterpret_cast<float*>(ws + p.o_off);
    }
    if (p.scheduled && !p.self_scheduled) {
        a.item_count = reinterpret_cast<int*>(ws);
        a.items = reinterpret_cast<const int4*>(ws + p.items_off);
    }
    a.self_schedule = p.self_scheduled ? 1 : 0;
    a.num_seqs = g.S;
    a.num_q_heads = g.Hq;
    a.num_kv_heads = g.Hkv;
    a.group = g.Hq / g.Hkv;
    a.units_per_seq = g.Hkv / p.heads_per_unit;
    a.block_size_log2 = log2i(g.bs);
    a.max_blocks_per_seq = g.MB;
    a.partition_tokens = p.partition_tokens;
    a.num_partitions = p.num_partitions;
    a.wave_partitions = p.wave_partitions ? p.waves : 1;
    a.num_items = p.num_items;
    a.last_block = last_block_id(g.N);
    a.cache = g.cache.lay;
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
    sa.num_kv_heads = a.units_per_seq;  // items are (sequence, unit, partition or group of partitions)
    sa.partition_tokens = p.partition_tokens * a.wave_partitions;
    sa.num_partitions = p.num_items;
    sa.split_tokens = p.partition_tokens;
    sa.split_count = p.num_partitions;
    sa.max_context = max_context;
    sa.block_size_log2 = a.block_size_log2;
    return sa;
}

int decode_plan(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* block_tables,
                const pa_decode_opts* opts, Geom* g, Plan* p) {
    int st = plan_geom(q, k_cache, block_tables, g);
    if (st != PA_OK) return st;
    if (g->q.rows != g->S) return PA_ERR_SHAPE;
    return make_plan(g->S, g->Hq, g->Hkv, g->D, g->bs, g->MB, g->cache.dtype, g->cache.heads_adjacent, opts, p);
}

// The cascade's group tensors: none (NULL or zero groups), or
// prefix_tables [G, PMB], prefix_lens [G], group_start [G + 1].
struct Groups {
    pa::abi::Table prefix{};
    const int32_t* prefix_lens = nullptr;
    const int32_t* group_start = nullptr;
    int32_t G = 0, PMB = 0;
};

int group_geom(const pa_tensor* prefix_tables, const pa_tensor* prefix_lens, const pa_tensor* group_start,
               bool need_arrays, Groups* gr) {
    if (prefix_tables == nullptr) return PA_OK;
    int st = pa::abi::table(prefix_tables, &gr->prefix, need_arrays);
    if (st != PA_OK) return st;
    gr->G = (int32_t)gr->prefix.rows;
    gr->PMB = gr->prefix.cols;
    if (!need_arrays) return PA_OK;
    if (gr->G == 0) return PA_OK;
    int64_t n = 0;
    st = pa::abi::vec(prefix_lens, PA_DTYPE_I32, &gr->prefix_lens, &n);
    if (st != PA_OK) return st;
    if (n != gr->G) return PA_ERR_SHAPE;
    st = pa::abi::vec(group_start, PA_DTYPE_I32, &gr->group_start, &n);
    if (st != PA_OK) return st;
    if (n != (int64_t)gr->G + 1) return PA_ERR_SHAPE;
    return PA_OK;
}

}  // namespace

extern "C" {

int pa_cache_write(const pa_tensor* k, const pa_tensor* v, const pa_tensor* slot_mapping, const pa_tensor* k_cache,
                   const pa_tensor* v_cache, float k_scale, float v_scale, void* stream) {
    pa::abi::Rows kr, vr;
    pa::abi::Cache c;
    int st = pa::abi::rows(k, false, &kr);
    if (st != PA_OK) return st;
    st = pa::abi::rows(v, false, &vr);
    if (st != PA_OK) return st;
    st = pa::abi::caches(k_cache, v_cache, &c);
    if (st != PA_OK) return st;
    const int64_t* slots = nullptr;
    int64_t T = 0;
    st = pa::abi::vec(slot_mapping, PA_DTYPE_I64, &slots, &T);
    if (st != PA_OK) return st;
    if (kr.rows != T || vr.rows != T || kr.heads != c.Hkv || vr.heads != c.Hkv || kr.dim != c.D || vr.dim != c.D)
        return PA_ERR_SHAPE;
    if (!scales_ok(c.dtype, k_scale, v_scale)) return PA_ERR_DTYPE;
    if (T == 0) return PA_OK;
    // one thread per 8-element chunk in a single launch, whose grid counts
    // work-items in 32 bits; divided, not multiplied, so that nothing overflows
    const int64_t chunks_per_token = (int64_t)c.Hkv * (c.D / 8);
    if (T > ((int64_t(1) << 32) - 256) / chunks_per_token) return PA_ERR_UNSUPPORTED;
    if (pa::debug_validate_enabled()) {
        const int vs = pa_check_cache_write_inputs(slot_mapping, k_cache, stream);
        if (vs != PA_OK) return vs;
    }
    pa::CacheWriteArgs a{};
    a.k = static_cast<const uint16_t*>(kr.data);
    a.v = static_cast<const uint16_t*>(vr.data);
    a.k_token = kr.s_row;
    a.k_head = kr.s_head;
    a.v_token = vr.s_row;
    a.v_head = vr.s_head;
    a.slot_mapping = slots;
    a.k_cache = c.data;
    a.v_cache = static_cast<uint8_t*>(v_cache->data);
    a.num_tokens = T;
    a.num_slots = c.N * c.bs;
    a.num_kv_heads = c.Hkv;
    a.head_dim = c.D;
    a.block_size_log2 = log2i(c.bs);
    a.cache = c.lay;
    a.k_scale = c.dtype == PA_DTYPE_FP8_E4M3FN ? k_scale : 1.0f;
    a.v_scale = c.dtype == PA_DTYPE_FP8_E4M3FN ? v_scale : 1.0f;
    const hipError_t e =
        pa::launch_cache_write(a, c.dtype == PA_DTYPE_FP8_E4M3FN, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_copy_blocks(const pa_tensor* k_cache, const pa_tensor* v_cache, const pa_tensor* block_mapping,
                   void* stream) {
    pa::abi::Cache c;
    int st = pa::abi::caches(k_cache, v_cache, &c);
    if (st != PA_OK) return st;
    st = pa::abi::basic(block_mapping, 2, PA_DTYPE_I64);
    if (st != PA_OK) return st;
    if (block_mapping->shape[1] != 2) return PA_ERR_SHAPE;
    const int64_t n = block_mapping->shape[0];
    if (n > 1 && block_mapping->stride[0] != 2) return PA_ERR_LAYOUT;
    if (!c.blocks_contiguous) return PA_ERR_LAYOUT;
    if (!pa::grid_fits(n, pa::kCopyThreads) || n >= (int64_t(1) << 31)) return PA_ERR_UNSUPPORTED;
    if (n == 0) return PA_OK;
    if (!pa::abi::aligned(block_mapping->data, 8)) return PA_ERR_ALIGN;
    pa::CopyBlocksArgs a{};
    a.k_cache = c.data;
    a.v_cache = static_cast<uint8_t*>(v_cache->data);
    a.pairs = static_cast<const int64_t*>(block_mapping->data);
    a.num_pairs = n;
    a.num_blocks = c.N;
    a.block_stride = c.lay.block;
    a.block_bytes = c.block_bytes;
    const hipError_t e = pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_decode_get_plan(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* block_tables,
                       const pa_decode_opts* opts, pa_decode_plan* plan) {
    if (!plan) return PA_ERR_NULL;
    Geom g;
    Plan p;
    const int st = decode_plan(q, k_cache, block_tables, opts, &g, &p);
    if (st != PA_OK) return st;
    plan->variant = p.variant;
    plan->waves_per_group = p.waves;
    plan->partition_tokens = p.partition_tokens;
    plan->num_partitions = p.num_partitions;
    plan->prefetch_tiles = p.depth - 1;
    plan->scheduled = p.self_scheduled ? 2 : (p.scheduled ? 1 : 0);
    plan->num_workgroups = p.num_workgroups;
    plan->workspace_bytes = p.workspace;
    plan->heads_per_tile = p.heads_per_unit;
    plan->wave_partitions = p.wave_partitions ? 1 : 0;
    return PA_OK;
}

size_t pa_decode_workspace_size(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* block_tables,
                                const pa_decode_opts* opts) {
    Geom g;
    Plan p;
    if (decode_plan(q, k_cache, block_tables, opts, &g, &p) != PA_OK) return 0;
    return p.workspace;
}

int pa_decode(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
              const pa_tensor* block_tables, const pa_tensor* context_lens, float scale, const pa_tensor* out,
              float k_scale, float v_scale, void* workspace, size_t workspace_bytes, const pa_decode_opts* opts,
              void* stream) {
    Geom g;
    int st = run_geom(q, k_cache, v_cache, block_tables, context_lens, out, &g);
    if (st != PA_OK) return st;
    if (g.q.rows != g.S) return PA_ERR_SHAPE;
    Plan p;
    st = make_plan(g.S, g.Hq, g.Hkv, g.D, g.bs, g.MB, g.cache.dtype, g.cache.heads_adjacent, opts, &p);
    if (st != PA_OK) return st;
    if (!std::isfinite(scale)) return PA_ERR_SHAPE;
    const int kvd = g.cache.dtype;
    if (!scales_ok(kvd, k_scale, v_scale)) return PA_ERR_DTYPE;
    if (g.S == 0) return PA_OK;
    st = check_workspace(p.workspace, workspace, workspace_bytes);
    if (st != PA_OK) return st;
    if (pa::debug_validate_enabled()) {
        const int vs = pa_check_decode_inputs(block_tables, context_lens, k_cache, stream);
        if (vs != PA_OK) return vs;
    }
    if (p.multi) return run_multi(p, g, nullptr, g.S, 1, scale, kvd, k_scale, v_scale, workspace, stream);
    pa::DecodeArgs a = decode_args(p, g, scale, kvd, k_scale, v_scale, workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (p.scheduled && !p.self_scheduled) {
        const pa::ScheduleArgs sa = schedule_args(p, a, g.context_lens, g.MB * g.bs);
        e = pa::launch_schedule(sa, s);
        if (e != hipSuccess) return PA_ERR_LAUNCH;
    }
    const pa::LaunchShape ls{p.waves, p.depth, p.heads_per_unit, p.wave_partitions};
    const bool fp8 = kvd == PA_DTYPE_FP8_E4M3FN;
    e = p.variant == PA_VARIANT_MFMA ? pa::launch_decode_mfma(a, g.D, fp8, ls, s)
                                     : pa::launch_decode_valu(a, g.D, fp8, ls, s);
    if (e != hipSuccess) return PA_ERR_LAUNCH;
    if (p.num_partitions > 1) {
        pa::MergeArgs m{};
        m.context_lens = g.context_lens;
        m.part_ml = a.part_ml;
        m.part_o = a.part_o;
        m.out = a.out;
        m.out_seq = a.out_seq;
        m.out_head = a.out_head;
        m.num_seqs = g.S;
        m.num_q_heads = g.Hq;
        m.head_dim = g.D;
        m.partition_tokens = p.partition_tokens;
        m.num_partitions = p.num_partitions;
        m.max_context = g.MB * g.bs;
        e = pa::launch_merge(m, s);
        if (e != hipSuccess) return PA_ERR_LAUNCH;
    }
    return PA_OK;
}

size_t pa_decode_cascade_workspace_size(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* block_tables,
                                        const pa_tensor* prefix_tables, int32_t max_group_size,
                                        const pa_decode_opts* opts) {
    Geom g;
    Groups gr;
    if (plan_geom(q, k_cache, block_tables, &g) != PA_OK || g.q.rows != g.S) return 0;
    if (group_geom(prefix_tables, nullptr, nullptr, false, &gr) != PA_OK) return 0;
    CascadePlan c;
    if (make_cascade_plan(g.S, g.Hq, g.Hkv, g.D, g.bs, g.MB, g.cache.dtype, g.cache.heads_adjacent, gr.G,
                          max_group_size, gr.PMB, opts, &c) != PA_OK)
        return 0;
    return c.workspace;
}

int pa_decode_cascade(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                      const pa_tensor* block_tables, const pa_tensor* context_lens, const pa_tensor* prefix_tables,
                      const pa_tensor* prefix_lens, const pa_tensor* group_start, float scale, const pa_tensor* out,
                      int32_t max_group_size, float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                      const pa_decode_opts* opts, void* stream) {
    Geom g;
    int st = run_geom(q, k_cache, v_cache, block_tables, context_lens, out, &g);
    if (st != PA_OK) return st;
    if (g.q.rows != g.S) return PA_ERR_SHAPE;
    Groups gr;
    st = group_geom(prefix_tables, prefix_lens, group_start, true, &gr);
    if (st != PA_OK) return st;
    CascadePlan c;
    st = make_cascade_plan(g.S, g.Hq, g.Hkv, g.D, g.bs, g.MB, g.cache.dtype, g.cache.heads_adjacent, gr.G,
                           max_group_size, gr.PMB, opts, &c);
    if (st != PA_OK) return st;
    if (!std::isfinite(scale)) return PA_ERR_SHAPE;
    const int kvd = g.cache.dtype;
    if (!scales_ok(kvd, k_scale, v_scale)) return PA_ERR_DTYPE;
    if (g.S == 0) return PA_OK;
    if (!workspace || workspace_bytes < c.workspace) return PA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_ALIGN;
    if (pa::debug_validate_enabled()) {
        int vs = pa_check_decode_inputs(block_tables, context_lens, k_cache, stream);
        if (vs == PA_OK && c.has_prefix)
            vs = pa_check_cascade_inputs(prefix_tables, prefix_lens, group_start, max_group_size, g.S, k_cache,
                                         stream);
        if (vs != PA_OK) return vs;
    }
    pa::CascadeGroups groups{};
    if (c.has_prefix) {
        groups.group_start = gr.group_start;
        groups.prefix_lens = gr.prefix_lens;
        groups.num_groups = gr.G;
        groups.max_group_size = max_group_size;
        groups.max_prefix_tokens = gr.PMB * g.bs;
        groups.max_context = g.MB * g.bs;
    }
    const Plan& p = c.suffix;
    const pa::DecodeArgs a = decode_args(p, g, scale, kvd, k_scale, v_scale, workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool fp8 = kvd == PA_DTYPE_FP8_E4M3FN;
    // 1. suffix work list
    pa::ScheduleArgs sa = schedule_args(p, a, g.context_lens, g.MB * g.bs);
    sa.cascade = groups;
    if (pa::launch_schedule(sa, s) != hipSuccess) return PA_ERR_LAUNCH;
    // 2. prefix pass: each group's prefix once for all its members
    pa::MultiArgs m{};
    if (c.has_prefix) {
        m = multi_args(c.prefix, g, gr.prefix, gr.G, nullptr, g.S, max_group_size, scale, kvd, k_scale, v_scale,
                       workspace);
        m.cascade = groups;
        if (pa::launch_multi(m, g.D, fp8, c.prefix.waves, c.prefix.row_tiles, s) != hipSuccess) return PA_ERR_LAUNCH;
    }
    // 3. suffix pass
    const pa::LaunchShape ls{p.waves, p.depth, p.heads_per_unit, false};
    const hipError_t e = p.variant == PA_VARIANT_MFMA ? pa::launch_decode_mfma(a, g.D, fp8, ls, s)
                                                      : pa::launch_decode_valu(a, g.D, fp8, ls, s);
    if (e != hipSuccess) return PA_ERR_LAUNCH;
    // 4. merge both passes' states
    pa::CascadeMergeArgs mg{};
    mg.context_lens = g.context_lens;
    mg.cascade = groups;
    mg.pre_ml = m.part_ml;
    mg.pre_o = m.part_o;
    mg.part_ml = a.part_ml;
    mg.part_o = a.part_o;
    mg.out = a.out;
    mg.out_seq = a.out_seq;
    mg.out_head = a.out_head;
    mg.num_seqs = g.S;
    mg.num_q_heads = g.Hq;
    mg.head_dim = g.D;
    mg.prefix_partition_tokens = c.has_prefix ? c.prefix.partition_tokens : 1;
    mg.prefix_partitions = c.has_prefix ? c.prefix.num_partitions : 0;
    mg.partition_tokens = p.partition_tokens;
    mg.num_partitions = p.num_partitions;
    mg.max_context = g.MB * g.bs;
    mg.block_size_log2 = a.block_size_log2;
    return pa::launch_cascade_merge(mg, s) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

size_t pa_decode_multi_workspace_size(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* block_tables,
                                      int32_t max_query_len, int32_t partition_tokens) {
    Geom g;
    if (plan_geom(q, k_cache, block_tables, &g) != PA_OK) return 0;
    if (g.q.rows > INT32_MAX) return 0;
    if (check_sizes(g.S, g.Hq, g.Hkv, g.D, g.bs, g.MB, g.cache.dtype) != PA_OK) return 0;
    Plan p;
    if (make_multi_plan(g.S, (int32_t)g.q.rows, max_query_len, g.Hq, g.Hkv, g.D, g.bs, g.MB, partition_tokens, &p) !=
        PA_OK)
        return 0;
    return p.workspace;
}

int pa_decode_multi(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                    const pa_tensor* block_tables, const pa_tensor* context_lens, const pa_tensor* query_start,
                    float scale, const pa_tensor* out, int32_t max_query_len, float k_scale, float v_scale,
                    void* workspace, size_t workspace_bytes, int32_t partition_tokens, void* stream) {
    Geom g;
    int st = run_geom(q, k_cache, v_cache, block_tables, context_lens, out, &g);
    if (st != PA_OK) return st;
    const int32_t* qs = nullptr;
    int64_t nqs = 0;
    st = pa::abi::vec(query_start, PA_DTYPE_I32, &qs, &nqs);
    if (st != PA_OK) return st;
    if (nqs != (int64_t)g.S + 1) return PA_ERR_SHAPE;
    st = check_sizes(g.S, g.Hq, g.Hkv, g.D, g.bs, g.MB, g.cache.dtype);
    if (st != PA_OK) return st;
    const int32_t Tq = (int32_t)g.q.rows;
    if (max_query_len < 0) return PA_ERR_SHAPE;
    if (!std::isfinite(scale)) return PA_ERR_SHAPE;
    const int kvd = g.cache.dtype;
    if (!scales_ok(kvd, k_scale, v_scale)) return PA_ERR_DTYPE;
    Plan p;
    st = make_multi_plan(g.S, Tq, max_query_len, g.Hq, g.Hkv, g.D, g.bs, g.MB, partition_tokens, &p);
    if (st != PA_OK) return st;
    if (g.S == 0 || Tq == 0 || max_query_len == 0) return PA_OK;
    st = check_workspace(p.workspace, workspace, workspace_bytes);
    if (st != PA_OK) return st;
    if (pa::debug_validate_enabled()) {
        const int vs = pa_check_multi_inputs(block_tables, context_lens, query_start, max_query_len, k_cache, stream);
        if (vs != PA_OK) return vs;
    }
    return run_multi(p, g, qs, Tq, max_query_len, scale, kvd, k_scale, v_scale, workspace, stream);
}

int pa_probe_stream_read(const void* buf, int64_t bytes, int32_t nontemporal, uint32_t* sink, void* stream) {
    if (bytes < 0 || (bytes & 15) != 0) return PA_ERR_SHAPE;
    if (bytes == 0) return PA_OK;
    if (!buf || !sink) return PA_ERR_NULL;
    if (!pa::abi::aligned(buf, 16) || !pa::abi::aligned(sink, 4)) return PA_ERR_ALIGN;
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
        case PA_ERR_ALIGN: return "a device address is not suitably aligned";
        case PA_ERR_DTYPE: return "wrong element type, or a bad fp8 scale";
        case PA_ERR_WORKSPACE: return "workspace missing or too small";
        case PA_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch or a copy";
        case PA_ERR_DEVICE: return "the current HIP device could not be queried";
        case PA_ERR_PRECONDITION: return "a device-side input violates a precondition (slots, tables or lengths)";
        case PA_ERR_SCRATCH: return "the plan needs more workspace than pa_decode_no_alloc's static scratch holds";
        case PA_ERR_LAYOUT: return "unsupported strides (innermost dimension not contiguous, not 16-byte multiples, "
                                   "overlapping, or a block too large)";
        default: return "unknown status";
    }
}

int pa_version(void) { return 200; }

}  // extern "C"
