/*
 * pa_oracle.c -- plain, slow, obviously correct CPU oracle for paged decode
 * attention and the paged KV-cache write. TEST INFRASTRUCTURE ONLY: it is
 * called by the tests, by the smoke check and by the benchmark's CPU
 * baseline leg; the product library never links, loads or calls it, and it
 * shares no code, header or table with that library.
 *
 * Pages cited (titles as printed at the top of each page):
 *   Tutorial = «大模型推理优化与加速完全教程» (LLM inference optimisation tutorial)
 *   ToPG     = «ToPG框架解析：大模型推理性能优化与三阶段流水线设计»
 *
 * What each function follows:
 *   oracle_decode_units  Tutorial §4.2 "PagedAttention" (PagedKVCache.get_kv:
 *                        walk the block table, keep `actual_len` rows of the
 *                        last block) followed by Tutorial §4.4 (GroupedQuery-
 *                        Attention.forward: query head h reads KV head
 *                        h div (Hq/Hkv), the repeat_interleave; scores
 *                        q.K^T * scale, softmax over the context, times V).
 *                        Everything in double precision.
 *   oracle_cache_write   Tutorial §4.2 (PagedKVCache.append_token: the row
 *                        `offset` of physical block `block` receives the new
 *                        token's K and V; here the slot id names that row as
 *                        block * block_size + offset).
 *   oracle_multi_units   Tutorial §5.1 (speculative decoding verifies the K
 *                        draft tokens in one pass) and §6.2 (chunked
 *                        prefill): several query tokens per sequence, each
 *                        attending causally over the paged context.
 *   oracle_copy_blocks   Tutorial §4.2 (copy-on-write named by PagedKVCache)
 *                        and §4.3 "Prefix Caching" (shared blocks): a block
 *                        is duplicated into a free one, every byte unchanged.
 *   fp8 e4m3fn codec     Tutorial §3.1 "量化基础" (symmetric_quantize:
 *                        value / scale, rounded, clamped to the code range;
 *                        dequantize: code * scale) with the OCP FP8 E4M3FN
 *                        format (1 sign, 4 exponent bits with bias 7, 3
 *                        mantissa bits, no infinities, S.1111.111 = NaN,
 *                        largest finite 448). ToPG names fp8 as the KV-cache
 *                        compression format.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - a slot id s < 0 is padding: nothing is written for that token;
 *   - context length 0 gives an all-zero output row;
 *   - fp8 quantisation divides in float32 (correctly rounded), rounds to the
 *     nearest e4m3fn value with ties to the even code, saturates magnitudes
 *     above 448 to 448 and maps NaN to NaN (0x7F with the sign);
 *   - fp8 values are decoded exactly and multiplied by the per-tensor scale
 *     in double before use.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no fast-math: the division and the
 * rounding above must be the IEEE operations).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_KV_BF16 = 1, ORACLE_KV_FP8_E4M3FN = 2 };

/* bfloat16 -> double: the 16 bits are the high half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* e4m3fn code -> double, from the field definition. */
double oracle_e4m3fn_to_f64(uint8_t c) {
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double v;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, 1 - 7);          /* subnormal: 0.m * 2^-6 */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);     /* normal: 1.m * 2^(e-7) */
    return sign ? -v : v;
}

/* Nearest e4m3fn code to x (float32), ties to the even code, saturating.
 * Plain search over the 127 non-negative finite codes, in increasing value. */
uint8_t oracle_f32_to_e4m3fn(float x) {
    if (isnan(x)) return (uint8_t)(signbit(x) ? 0xFF : 0x7F);
    int neg = signbit(x) ? 1 : 0;
    double a = fabs((double)x);
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double err = fabs(oracle_e4m3fn_to_f64((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(best | (neg << 7));
}

/* The quantised code of one bf16 input under a per-tensor scale. */
uint8_t oracle_quantize_bf16(uint16_t xb, float scale) {
    float x = (float)oracle_bf16_to_f64(xb);
    float y = x / scale;  /* binary32 division, correctly rounded */
    return oracle_f32_to_e4m3fn(y);
}

/*
 * Cache write. k, v: [T, Hkv, D] bf16 bits. caches: [N, bs, Hkv, D] of
 * bf16 bits (kv_dtype 1) or e4m3fn codes (kv_dtype 2). Returns the number
 * of tokens written, or -1 if a slot is outside the pool.
 */
int64_t oracle_cache_write(const uint16_t* k, const uint16_t* v, const int64_t* slot_mapping,
                           int64_t T, int64_t Hkv, int64_t D, int64_t bs, int64_t N,
                           int kv_dtype, float k_scale, float v_scale,
                           void* k_cache, void* v_cache) {
    int64_t written = 0;
    /* fp8: the code of a bf16 input depends only on its 16 bits, so tabulate
     * oracle_quantize_bf16 over all 65536 inputs once per call (same values,
     * computed once instead of once per element). */
    uint8_t* kq = NULL;
    uint8_t* vq = NULL;
    if (kv_dtype != ORACLE_KV_BF16) {
        kq = (uint8_t*)malloc(65536);
        vq = (uint8_t*)malloc(65536);
        for (int b = 0; b < 65536; ++b) {
            kq[b] = oracle_quantize_bf16((uint16_t)b, k_scale);
            vq[b] = oracle_quantize_bf16((uint16_t)b, v_scale);
        }
    }
    for (int64_t t = 0; t < T; ++t) {
        int64_t s = slot_mapping[t];
        if (s < 0) continue;
        if (s >= N * bs) { written = -1; break; }
        int64_t block = s / bs, offset = s % bs;
        for (int64_t h = 0; h < Hkv; ++h) {
            for (int64_t d = 0; d < D; ++d) {
                int64_t src = (t * Hkv + h) * D + d;
                int64_t dst = ((block * bs + offset) * Hkv + h) * D + d;
                if (kv_dtype == ORACLE_KV_BF16) {
                    ((uint16_t*)k_cache)[dst] = k[src];
                    ((uint16_t*)v_cache)[dst] = v[src];
                } else {
                    ((uint8_t*)k_cache)[dst] = kq[k[src]];
                    ((uint8_t*)v_cache)[dst] = vq[v[src]];
                }
            }
        }
        ++written;
    }
    free(kq);
    free(vq);
    return written;
}

static double load_kv(const void* cache, int kv_dtype, int64_t idx, double s) {
    if (kv_dtype == ORACLE_KV_BF16) return oracle_bf16_to_f64(((const uint16_t*)cache)[idx]);
    return oracle_e4m3fn_to_f64(((const uint8_t*)cache)[idx]) * s;
}

/*
 * Decode attention for selected (sequence, KV head) units.
 *   q            [S, Hq, D] bf16 bits
 *   caches       [N, bs, Hkv, D] bf16 bits or e4m3fn codes
 *   block_tables [S, MB] int32, context_lens [S] int32
 *   units        n_units ids u = seq * Hkv + kv_head
 *   out          [n_units, g, D] doubles, g = Hq / Hkv, for query heads
 *                kv_head * g .. kv_head * g + g - 1 of that sequence
 * Returns 0, or -1 on a block id outside the pool or a context longer than
 * the table row.
 */
int oracle_decode_units(const uint16_t* q, const void* k_cache, const void* v_cache,
                        int kv_dtype, double k_scale, double v_scale,
                        const int32_t* block_tables, const int32_t* context_lens,
                        int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t bs,
                        int64_t N, int64_t MB, double scale,
                        const int64_t* units, int64_t n_units, double* out, int num_threads) {
    int64_t g = Hq / Hkv;
    int bad = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t u = 0; u < n_units; ++u) {
        int64_t seq = units[u] / Hkv, kvh = units[u] % Hkv;
        double* o = out + u * g * D;
        if (units[u] < 0 || seq >= S) { bad = 1; continue; }
        int64_t L = context_lens[seq];
        if (L <= 0) {
            for (int64_t x = 0; x < g * D; ++x) o[x] = 0.0;
            continue;
        }
        if (L > MB * bs) { bad = 1; continue; }
        /* gather through the block table: token j -> (table[j / bs], j % bs) */
        double* K = (double*)malloc(sizeof(double) * L * D);
        double* V = (double*)malloc(sizeof(double) * L * D);
        double* sc = (double*)malloc(sizeof(double) * L);
        for (int64_t j = 0; j < L; ++j) {
            int64_t block = block_tables[seq * MB + j / bs];
            int64_t offset = j % bs;
            if (block < 0 || block >= N) { bad = 1; block = 0; }
            for (int64_t d = 0; d < D; ++d) {
                int64_t idx = ((block * bs + offset) * Hkv + kvh) * D + d;
                K[j * D + d] = load_kv(k_cache, kv_dtype, idx, k_scale);
                V[j * D + d] = load_kv(v_cache, kv_dtype, idx, v_scale);
            }
        }
        for (int64_t r = 0; r < g; ++r) {
            int64_t h = kvh * g + r;  /* query head h reads KV head h / g */
            const uint16_t* qh = q + (seq * Hq + h) * D;
            double m = -INFINITY;
            for (int64_t j = 0; j < L; ++j) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += oracle_bf16_to_f64(qh[d]) * K[j * D + d];
                sc[j] = dot * scale;
                if (sc[j] > m) m = sc[j];
            }
            double den = 0.0;
            for (int64_t j = 0; j < L; ++j) {
                sc[j] = exp(sc[j] - m);
                den += sc[j];
            }
            for (int64_t d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int64_t j = 0; j < L; ++j) acc += sc[j] * V[j * D + d];
                o[r * D + d] = acc / den;
            }
        }
        free(K);
        free(V);
        free(sc);
    }
    return bad ? -1 : 0;
}

/*
 * Multi-token paged attention: several query tokens per sequence, each
 * attending causally over the paged context. This is the attention of the
 * target model's single pass that verifies K draft tokens (Tutorial §5.1,
 * speculative decoding: the draft tokens are appended and scored together)
 * and of a prefill chunk over a sequence whose earlier chunks are already
 * cached (Tutorial §6.2, chunked prefill in 512-token chunks).
 * Sequence i has context_lens[i] = L cached tokens whose last
 * n = query_start[i+1] - query_start[i] are its query tokens (already
 * written to the cache): query r (0 <= r < n) is the token at position
 * p = L - n + r and attends to positions 0..p (the causal mask), through the
 * block table exactly as in oracle_decode_units.
 *   q            [T_q, Hq, D] bf16 bits; row query_start[i] + r
 *   query_start  [S + 1] int32, non-decreasing, query_start[0] = 0
 *   units        n_units ids u = seq * Hkv + kv_head
 *   out          [T_q, Hq, D] doubles; the rows of the requested units are
 *                written (query heads kv_head * g .. kv_head * g + g - 1)
 * Returns 0, or -1 on a block id outside the pool, a context longer than the
 * table row, or more query tokens than context.
 */
int oracle_multi_units(const uint16_t* q, const void* k_cache, const void* v_cache,
                       int kv_dtype, double k_scale, double v_scale,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* query_start,
                       int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t bs,
                       int64_t N, int64_t MB, double scale,
                       const int64_t* units, int64_t n_units, double* out, int num_threads) {
    int64_t g = Hq / Hkv;
    int bad = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t u = 0; u < n_units; ++u) {
        int64_t seq = units[u] / Hkv, kvh = units[u] % Hkv;
        if (units[u] < 0 || seq >= S) { bad = 1; continue; }
        int64_t L = context_lens[seq];
        int64_t q0 = query_start[seq], n = query_start[seq + 1] - query_start[seq];
        if (n <= 0) continue;
        if (L < n || L > MB * bs) { bad = 1; continue; }
        /* gather the context through the block table */
        double* K = (double*)malloc(sizeof(double) * L * D);
        double* V = (double*)malloc(sizeof(double) * L * D);
        double* sc = (double*)malloc(sizeof(double) * L);
        for (int64_t j = 0; j < L; ++j) {
            int64_t block = block_tables[seq * MB + j / bs];
            int64_t offset = j % bs;
            if (block < 0 || block >= N) { bad = 1; block = 0; }
            for (int64_t d = 0; d < D; ++d) {
                int64_t idx = ((block * bs + offset) * Hkv + kvh) * D + d;
                K[j * D + d] = load_kv(k_cache, kv_dtype, idx, k_scale);
                V[j * D + d] = load_kv(v_cache, kv_dtype, idx, v_scale);
            }
        }
        for (int64_t r = 0; r < n; ++r) {
            int64_t p = L - n + r;  /* position of query r; it sees tokens 0..p */
            for (int64_t hh = 0; hh < g; ++hh) {
                int64_t h = kvh * g + hh;
                const uint16_t* qh = q + ((q0 + r) * Hq + h) * D;
                double* o = out + ((q0 + r) * Hq + h) * D;
                double m = -INFINITY;
                for (int64_t j = 0; j <= p; ++j) {
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += oracle_bf16_to_f64(qh[d]) * K[j * D + d];
                    sc[j] = dot * scale;
                    if (sc[j] > m) m = sc[j];
                }
                double den = 0.0;
                for (int64_t j = 0; j <= p; ++j) {
                    sc[j] = exp(sc[j] - m);
                    den += sc[j];
                }
                for (int64_t d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int64_t j = 0; j <= p; ++j) acc += sc[j] * V[j * D + d];
                    o[d] = acc / den;
                }
            }
        }
        free(K);
        free(V);
        free(sc);
    }
    return bad ? -1 : 0;
}

/*
 * Block copy, the copy half of copy-on-write (Tutorial §4.2, PagedKVCache
 * lists copy-on-write for beam search; Tutorial §4.3 "Prefix Caching" shares
 * a prefix's blocks between sequences until one of them must write): for
 * every pair (src, dst) of `pairs` ([n_pairs][2] int64), every element of
 * physical block dst -- all block_size rows, all KV heads, all head_dim
 * values -- becomes the element of block src, in both caches. Element size
 * `elem` bytes (2 for bf16, 1 for fp8); the bytes are copied unchanged.
 * A pair with a negative id is padding and is skipped. Sources are read as
 * they were before the call (the destinations are copied into a separate
 * buffer first), so the result does not depend on the order of the pairs.
 * Returns the number of pairs copied, or -1 if an id is outside the pool or
 * two pairs name the same destination.
 */
int64_t oracle_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int64_t n_pairs,
                           int64_t N, int64_t bs, int64_t Hkv, int64_t D, int64_t elem) {
    const int64_t row_elems = Hkv * D;
    const int64_t block_elems = bs * row_elems;
    for (int64_t p = 0; p < n_pairs; ++p) {
        int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
        if (src < 0 || dst < 0) continue;
        if (src >= N || dst >= N) return -1;
        for (int64_t p2 = 0; p2 < p; ++p2)
            if (pairs[2 * p2] >= 0 && pairs[2 * p2 + 1] == dst) return -1;
    }
    void* caches[2] = {k_cache, v_cache};
    int64_t copied = 0;
    for (int c = 0; c < 2; ++c) {
        unsigned char* base = (unsigned char*)caches[c];
        /* snapshot of every source block, element by element */
        unsigned char* snap = (unsigned char*)malloc((size_t)(n_pairs > 0 ? n_pairs : 1) * block_elems * elem);
        for (int64_t p = 0; p < n_pairs; ++p) {
            int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
            if (src < 0 || dst < 0) continue;
            for (int64_t r = 0; r < bs; ++r)
                for (int64_t h = 0; h < Hkv; ++h)
                    for (int64_t d = 0; d < D; ++d) {
                        int64_t from = ((src * bs + r) * Hkv + h) * D + d;
                        int64_t to = (p * bs + r) * row_elems + h * D + d;
                        memcpy(snap + to * elem, base + from * elem, (size_t)elem);
                    }
        }
        for (int64_t p = 0; p < n_pairs; ++p) {
            int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
            if (src < 0 || dst < 0) continue;
            for (int64_t r = 0; r < bs; ++r)
                for (int64_t h = 0; h < Hkv; ++h)
                    for (int64_t d = 0; d < D; ++d) {
                        int64_t from = (p * bs + r) * row_elems + h * D + d;
                        int64_t to = ((dst * bs + r) * Hkv + h) * D + d;
                        memcpy(base + to * elem, snap + from * elem, (size_t)elem);
                    }
            if (c == 0) ++copied;
        }
        free(snap);
    }
    return copied;
}

/* Number of OpenMP threads a parallel region would use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
