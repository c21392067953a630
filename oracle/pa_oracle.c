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

/* Number of OpenMP threads a parallel region would use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
