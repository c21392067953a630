/*
 * pa.h -- paged KV-cache decode attention on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels. Every tensor is passed as a
 * pa_tensor: a device address plus element type, shape and element strides.
 * Every call is asynchronous on `stream` (a hipStream_t passed as void*,
 * NULL = the default stream) and returns once its launches are queued. The
 * caller owns every buffer, including the split-K workspace; apart from
 * pa_decode_no_alloc's static scratch (below) the library allocates no
 * device memory and keeps no state between calls beyond a per-device CU
 * count.
 *
 * Pages cited (titles as printed at the top of each page):
 *   Tutorial = «大模型推理优化与加速完全教程» (LLM inference optimisation tutorial)
 *   nanoVLLM = «大模型推理优化技术：从nano-vLLM到连续批处理»
 *   TGI      = «TGI技术解析：大规模语言模型高效推理实践»
 *   ToPG     = «ToPG框架解析：大模型推理性能优化与三阶段流水线设计»
 *
 * Logical shapes (the strides say where each element lives):
 *   q, out        [num_seqs, num_q_heads, head_dim]             bf16
 *   k, v          [num_tokens, num_kv_heads, head_dim]          bf16
 *   k_cache,      [num_blocks, block_size, num_kv_heads, head_dim]
 *   v_cache         bf16 or fp8 e4m3fn codes. This is the physical block
 *                 pool of Tutorial §4.2 "PagedAttention" (PagedKVCache's
 *                 block pool) for one layer and one of K/V; nanoVLLM §4.3
 *                 sizes a block the same way. The page stores the pool in
 *                 this order; any other order of the first three dimensions
 *                 is passed as strides, e.g. a head-major pool allocated as
 *                 [num_blocks, num_kv_heads, block_size, head_dim] and
 *                 described with shape [N, bs, Hkv, D] and strides
 *                 [Hkv*bs*D, D, bs*D, 1]. K and V must share one layout.
 *   block_tables  [num_seqs, max_blocks_per_seq] int32: entry b of row i is
 *                 the physical block holding tokens b*block_size ..
 *                 b*block_size + block_size - 1 of sequence i (Tutorial §4.2,
 *                 block_tables; nanoVLLM §4.2 logical-to-physical map).
 *   context_lens  [num_seqs] int32: cached tokens sequence i attends to.
 *   slot_mapping  [num_tokens] int64: slot s names row s % block_size of
 *                 physical block s / block_size (Tutorial §4.2, append_token's
 *                 block index and offset, flattened).
 *
 * Layout rules, checked on the host before anything is launched:
 *   - the last dimension is contiguous (stride 1); no stride is negative;
 *   - bf16 and fp8 tensors: data 16-byte aligned and every stride a
 *     multiple of 16 bytes (8 bf16 elements, 16 fp8 codes);
 *   - int32 / int64 index tensors: data aligned to the element size; 1-D
 *     ones contiguous; block tables may have any row stride >= their width;
 *   - tensors the call writes (out, the caches of pa_cache_write and
 *     pa_copy_blocks) and every cache do not overlap themselves;
 *   - a cache block spans less than 2^31 bytes (its rows' byte offsets are
 *     32-bit).
 * A violation returns PA_ERR_LAYOUT (PA_ERR_ALIGN for a misaligned address).
 *
 * Status: every entry point returns PA_OK (0) or a negative PA_ERR_* code.
 * Arguments are checked on the host; nothing is read back from the device.
 * Device-side contents (slot ids, block ids, context lengths) are
 * preconditions: the kernels clamp block ids into the pool and ignore
 * out-of-pool slots so that a bad table cannot fault the GPU, but the
 * results are then unspecified. The pa_check_* calls verify them
 * (synchronising); with the environment variable PA_DEBUG_VALIDATE set to
 * anything but "0", the hot-path calls run those checks first and return
 * PA_ERR_PRECONDITION instead of launching.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_OK 0
#define PA_ERR_NULL (-1)        /* a required pointer is NULL */
#define PA_ERR_SHAPE (-2)       /* a size is negative, zero where it may not be, or inconsistent */
#define PA_ERR_UNSUPPORTED (-3) /* valid, but outside what the kernels implement */
#define PA_ERR_ALIGN (-4)       /* a device address is not suitably aligned */
#define PA_ERR_DTYPE (-5)       /* wrong element type, or a bad fp8 scale */
#define PA_ERR_WORKSPACE (-6)   /* workspace missing or smaller than the call needs */
#define PA_ERR_LAUNCH (-7)      /* the HIP runtime rejected a launch or a copy */
#define PA_ERR_DEVICE (-8)      /* the current device could not be queried */
#define PA_ERR_PRECONDITION (-9) /* a device-side input breaks a precondition (checked calls only) */
#define PA_ERR_LAYOUT (-10)     /* strides outside the layout rules above */
#define PA_ERR_SCRATCH (-11)    /* pa_decode_no_alloc: the plan needs more than the static scratch */

/* Element types of a pa_tensor. */
#define PA_DTYPE_BF16 1
#define PA_DTYPE_FP8_E4M3FN 2 /* OCP FP8 E4M3FN codes, per-tensor scale (ToPG §3: fp8 KV compression) */
#define PA_DTYPE_I32 4
#define PA_DTYPE_I64 5

/* A strided view of device memory. Dimensions past ndim are ignored. */
typedef struct pa_tensor {
    void* data;        /* device address; may be NULL when the tensor has no elements */
    int32_t dtype;     /* PA_DTYPE_* */
    int32_t ndim;      /* 1..4, as each argument requires */
    int64_t shape[4];  /* sizes */
    int64_t stride[4]; /* element strides */
} pa_tensor;

/* Decode kernel families. */
#define PA_VARIANT_AUTO 0
#define PA_VARIANT_VALU 1 /* dot products on the vector ALUs, DPP row reductions (g <= 4) */
#define PA_VARIANT_MFMA 2 /* q.K^T and P.V as 16x16 bf16 MFMA tiles (GQA groups) */

/* Optional decode tuning; pass NULL for the defaults. */
typedef struct pa_decode_opts {
    int32_t partition_tokens; /* 0 = chosen by the library; -1 = never split the
                                 context; >0 = split every context into
                                 partitions of this many tokens (multiple of 16),
                                 merged by log-sum-exp. */
    int32_t variant;          /* PA_VARIANT_* */
    int32_t waves_per_group;  /* 0 = chosen; else 1, 2, 4 or 8 wavefronts per
                                 workgroup */
    int32_t prefetch_tiles;   /* 0 = chosen; else 1..3: 16-token tiles each
                                 wavefront keeps in flight ahead of the one it
                                 consumes */
    int32_t schedule;         /* 1 = first build the work list on the device
                                 from context_lens: real (sequence, KV head,
                                 partition) items only, longest first, so
                                 workgroups are dispatched in that order;
                                 2 = the same order without the builder
                                 pass: each workgroup ranks its block index
                                 among the items of context_lens itself (at
                                 most 4096 sequences, PA_ERR_UNSUPPORTED
                                 beyond; with more than 16 query heads per
                                 KV head at most 256, as 1 beyond);
                                 -1 = one workgroup per (sequence, KV head,
                                 partition) in index order, empty ones
                                 included;
                                 0 = chosen: when the plan splits contexts,
                                 2 for batches of at most 256 sequences
                                 whose grid holds at most 1024 (sequence,
                                 item) pairs, else 1; when it does not
                                 split, -1 */
    int32_t heads_per_tile;   /* MFMA kernel: 0 = chosen (2 for bf16 caches
                                 when g is 4..8, 2 for fp8 when g is 5..8,
                                 given an even num_kv_heads and adjacent KV
                                 heads in memory; else 1); else 1, 2 or 4
                                 adjacent KV heads sharing one 16-row matrix
                                 tile (g * heads_per_tile <= 16, head stride
                                 == head_dim) */
    int32_t wave_partitions;  /* split contexts, MFMA kernel: 1 = each wave
                                 of a workgroup takes one whole partition (a
                                 workgroup covers W consecutive partitions and
                                 stores W states); -1 = the waves share one
                                 partition's tiles and combine their states;
                                 0 = chosen (1 for fp8 caches and partitions
                                 of at most 512 tokens) */
    int32_t reserved;         /* must be 0 */
} pa_decode_opts;

/* What pa_decode will launch for a given set of arguments (for tests and
 * profiling). */
typedef struct pa_decode_plan {
    int32_t variant;          /* PA_VARIANT_VALU or PA_VARIANT_MFMA */
    int32_t waves_per_group;
    int32_t partition_tokens; /* tokens per partition */
    int32_t num_partitions;   /* partitions per (sequence, KV head); 1 = no split */
    int32_t prefetch_tiles;
    int32_t scheduled;        /* 0 = direct grid; 1 = device-built work list;
                                 2 = longest-first items found by each
                                 workgroup (no list, no builder pass) */
    int64_t num_workgroups;   /* decode kernel grid size (with a work list, the
                                 ones past its end exit at once) */
    size_t workspace_bytes;   /* bytes of workspace pa_decode needs */
    int32_t heads_per_tile;   /* KV heads per matrix tile (1 for the VALU kernel) */
    int32_t wave_partitions;  /* 1 = each wave takes its own partition */
} pa_decode_plan;

/*
 * pa_cache_write -- store num_tokens new tokens' K and V rows in the paged
 * caches (Tutorial §4.2, PagedKVCache.append_token: the new K/V row goes to
 * row `offset` of physical block `block`).
 *
 *   k, v           [num_tokens, num_kv_heads, head_dim] bf16 (read)
 *   slot_mapping   [num_tokens] int64; slot < 0 = skip this token; slots
 *                  must be distinct (concurrent writers otherwise race)
 *   k_cache,       [num_blocks, block_size, num_kv_heads, head_dim], bf16 or
 *   v_cache          fp8 e4m3fn (written: only the addressed rows)
 *   For bf16 caches rows are copied bit for bit. For fp8 caches each
 *   element x becomes the e4m3fn code nearest to float32(x) / scale
 *   (correctly rounded division, ties to the even code, magnitudes above
 *   448 saturate to 448, NaN stays NaN), scale = k_scale for K and v_scale
 *   for V (Tutorial §3.1 "量化基础", symmetric_quantize: value / scale,
 *   rounded and clamped to the code range).
 *   k_scale,       fp8 only: finite and > 0 (ignored for bf16)
 *   v_scale
 * head_dim in {64, 128}; block_size a power of two in [16, 1024] (the range
 * pa_decode reads). num_tokens == 0 returns PA_OK with no launch;
 * num_tokens * num_kv_heads * head_dim / 8 must stay below 2^32 - 256 (one
 * launch), else PA_ERR_UNSUPPORTED.
 */
int pa_cache_write(const pa_tensor* k, const pa_tensor* v, const pa_tensor* slot_mapping,
                   const pa_tensor* k_cache, const pa_tensor* v_cache,
                   float k_scale, float v_scale, void* stream);

/*
 * pa_copy_blocks -- duplicate physical blocks, the copy step of copy-on-write
 * (Tutorial §4.2, PagedKVCache supports copy-on-write for beam search;
 * Tutorial §4.3 "Prefix Caching" shares blocks between sequences): for each
 * pair (src, dst) of block_mapping, block dst of k_cache and of v_cache
 * becomes a byte-for-byte copy of block src (every row and KV head).
 *
 *   k_cache, v_cache  as in pa_cache_write (written); each block must fill
 *                     one contiguous range (the block dimension outermost
 *                     in memory order, the other three dense, in any order)
 *   block_mapping     [num_pairs, 2] int64 (src, dst), contiguous; a pair
 *                     with a negative or out-of-pool id is skipped
 * Preconditions (not checked): destinations distinct, and no block is both
 * a source and a destination in one call (pairs are copied concurrently).
 * num_pairs < 2^31; num_pairs == 0 returns PA_OK with no launch.
 */
int pa_copy_blocks(const pa_tensor* k_cache, const pa_tensor* v_cache, const pa_tensor* block_mapping,
                   void* stream);

/*
 * pa_decode -- one decode step of paged attention: every sequence's single
 * query token attends over its context_lens[i] cached tokens, reached
 * through its block-table row (Tutorial §4.2, PagedKVCache.get_kv;
 * nanoVLLM §4.2, attention through the logical-to-physical block map).
 * For query head h of sequence i, with g = num_q_heads / num_kv_heads and
 * KV head kh = h / g (Tutorial §4.4, GroupedQueryAttention: repeat_interleave
 * of the KV heads):
 *     s_j      = scale * sum_d q[i,h,d] * K_j[kh,d]      j < context_lens[i]
 *     out[i,h] = sum_j softmax(s)_j * V_j[kh,:]
 * with K_j, V_j row j mod block_size of block block_tables[i][j / block_size];
 * for fp8 caches K_j = code * k_scale and V_j = code * v_scale. Arithmetic is
 * float32 with bf16 inputs (ToPG §2: accumulate in FP32); out is rounded
 * to bf16 (nearest even). A sequence with context length 0 gets zeros.
 *
 *   q                [num_seqs, num_q_heads, head_dim] bf16
 *   k_cache, v_cache [num_blocks, block_size, num_kv_heads, head_dim]
 *   block_tables     [num_seqs, max_blocks_per_seq] int32; entries past
 *                    ceil(context_lens[i] / block_size) are never read
 *   context_lens     [num_seqs] int32, each in [0, max_blocks_per_seq * block_size]
 *   scale            the score scale (usually 1/sqrt(head_dim)), finite
 *   out              [num_seqs, num_q_heads, head_dim] bf16 (written)
 *   k_scale, v_scale fp8 caches: finite and > 0 (ignored for bf16)
 *   workspace        device, >= pa_decode_workspace_size(...) bytes, 256-byte
 *                    aligned (may be NULL when that size is 0): the work list
 *                    and the split-K partials; scratch, overwritten by each
 *                    call. Calls that share a workspace must be ordered on
 *                    one stream.
 *   opts             NULL or tuning options
 * Supported: head_dim in {64, 128}; g in [1, 1024] (above 16 the multi-row
 * kernel of pa_decode_multi runs); block_size a power of two in [16, 1024].
 */
int pa_decode(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
              const pa_tensor* block_tables, const pa_tensor* context_lens, float scale,
              const pa_tensor* out, float k_scale, float v_scale,
              void* workspace, size_t workspace_bytes, const pa_decode_opts* opts, void* stream);

/*
 * pa_decode_no_alloc -- pa_decode for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): the same operation, arguments and kernels, with the
 * work list and split-K partials in a static scratch array inside the
 * library instead of a caller workspace. The array is PA_NO_ALLOC_SCRATCH
 * bytes per device, allocated by the HIP runtime when the library's code is
 * loaded on that device and held until the process ends; its address is
 * looked up once per device, on the first call there. The call allocates
 * nothing. A plan that needs more (pa_decode_workspace_size above the limit)
 * returns PA_ERR_SCRATCH before launching. Every call on a device shares
 * that device's array: calls that may overlap on one device (different
 * streams without ordering, or concurrent host threads) race on it and give
 * unspecified results. Nothing in the array needs clearing between calls:
 * each launch writes every word it later reads.
 */
#define PA_NO_ALLOC_SCRATCH ((size_t)32 << 20)
int pa_decode_no_alloc(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                       const pa_tensor* block_tables, const pa_tensor* context_lens, float scale,
                       const pa_tensor* out, float k_scale, float v_scale, const pa_decode_opts* opts,
                       void* stream);

/*
 * pa_decode_get_plan -- the launch plan pa_decode would use for these
 * tensors on the current device (shapes, types and strides only; nothing is
 * read or launched). Returns PA_OK and fills *plan, or the error pa_decode
 * would return for them.
 * pa_decode_workspace_size -- bytes of workspace pa_decode needs (0 when it
 * needs none, or when the arguments are invalid).
 */
int pa_decode_get_plan(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* block_tables,
                       const pa_decode_opts* opts, pa_decode_plan* plan);
size_t pa_decode_workspace_size(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* block_tables,
                                const pa_decode_opts* opts);

/*
 * pa_decode_multi -- paged attention for several query tokens per sequence,
 * each attending causally over the paged context: the target model's pass
 * that verifies K draft tokens at once (Tutorial §5.1, speculative
 * decoding) and a prefill chunk over an already cached prefix (Tutorial
 * §6.2, chunked prefill). Sequence i has context_lens[i] = L cached tokens,
 * the last n_i = query_start[i+1] - query_start[i] of which are its query
 * tokens, already written with pa_cache_write. Query r of sequence i (row
 * query_start[i] + r of q and out) is the token at position L - n_i + r; for
 * query head h, with g = num_q_heads / num_kv_heads and kh = h / g,
 *     s_j = scale * sum_d q[row,h,d] * K_j[kh,d]      for j <= L - n_i + r
 *     out[row,h] = sum_j softmax(s)_j * V_j[kh,:]
 * (K_j, V_j and fp8 scaling as in pa_decode). n_i = 1 for every sequence is
 * exactly pa_decode's operation.
 *
 *   q, out          [num_query_tokens, num_q_heads, head_dim] bf16
 *   query_start     [num_seqs + 1] int32, non-decreasing, from 0 to
 *                   num_query_tokens (num_seqs = context_lens' length)
 *   max_query_len   host, >= every n_i (rows past it are not computed)
 *   partition_tokens 0 = chosen by the library, -1 = never split, > 0 =
 *                   split contexts into partitions of this many tokens
 *                   (multiple of 16) merged by log-sum-exp
 *   workspace       device, >= pa_decode_multi_workspace_size(...) bytes,
 *                   256-byte aligned (may be NULL when that size is 0)
 * Other arguments as in pa_decode. Preconditions (not checked, see
 * pa_check_multi_inputs): n_i <= context_lens[i]; a query with no visible
 * token gets a zero output row. g may be anything up to 1024.
 */
int pa_decode_multi(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                    const pa_tensor* block_tables, const pa_tensor* context_lens,
                    const pa_tensor* query_start, float scale, const pa_tensor* out, int32_t max_query_len,
                    float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                    int32_t partition_tokens, void* stream);

/* Bytes of workspace pa_decode_multi needs (0 when none, or for invalid arguments). */
size_t pa_decode_multi_workspace_size(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* block_tables,
                                      int32_t max_query_len, int32_t partition_tokens);

/*
 * pa_decode_cascade -- pa_decode for a batch in which groups of sequences
 * share a cached prefix, reading each shared prefix once per group instead
 * of once per sequence. Tutorial §4.3 (Prefix Caching): requests that share
 * a system prompt reuse the physical blocks cached for it; the prefix cache
 * keeps, per prefix, its list of blocks and its length -- here row k of
 * prefix_tables and prefix_lens[k].
 *
 * Group k is the run of sequences group_start[k] .. group_start[k+1] - 1 of
 * the batch (order the batch so that sharers are adjacent). Member i of
 * group k, with shared_i = min(context_lens[i], prefix_lens[k]), reads its
 * tokens 0 .. shared_i - 1 through prefix_tables[k] and its tokens shared_i
 * .. context_lens[i] - 1 through its own block_tables row; a sequence in no
 * group reads everything through its own row. Apart from that gather the
 * result is pa_decode's: for every query head, softmax(scale * q K^T) V over
 * the sequence's context_lens[i] tokens, bf16 output. When each member's
 * table already names the prefix blocks (as with prefix caching) it is the
 * same attention as pa_decode on the same arguments.
 *
 * How: one pass attends each group's prefix for all query heads of all its
 * members at once (the multi-row kernel of pa_decode_multi, so a prefix
 * tile is loaded once for the whole group), the decode kernels attend the
 * rest of every context, and a log-sum-exp merge combines the two.
 *
 *   prefix_tables    [num_groups, max_prefix_blocks] int32
 *   prefix_lens      [num_groups] int32 tokens, each a multiple of
 *                    block_size and <= max_prefix_blocks * block_size
 *   group_start      [num_groups + 1] int32, non-decreasing, from >= 0 to
 *                    <= num_seqs
 *   max_group_size   host, >= every group's size (sequences past it in a
 *                    group are treated as in no group)
 *   workspace        device, >= pa_decode_cascade_workspace_size(...) bytes,
 *                    256-byte aligned (always needed): the work list and
 *                    both passes' partial states
 * Other arguments as in pa_decode (opts apply to the decode kernels of the
 * second pass; the work list is always used). The three group tensors may
 * be NULL (or have num_groups = 0): a plain decode. Supported: as pa_decode
 * with at most 16 query heads per KV head (PA_ERR_UNSUPPORTED beyond).
 * Preconditions (pa_check_cascade_inputs verifies them): those of pa_decode
 * for block_tables and context_lens, the layout of the three group arrays
 * above, and prefix table entries covering prefix_lens[k] inside the pool.
 * A prefix length that is not whole blocks is rounded down, its last
 * tokens then being read through the member's own row.
 */
int pa_decode_cascade(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                      const pa_tensor* block_tables, const pa_tensor* context_lens,
                      const pa_tensor* prefix_tables, const pa_tensor* prefix_lens,
                      const pa_tensor* group_start, float scale, const pa_tensor* out,
                      int32_t max_group_size, float k_scale, float v_scale,
                      void* workspace, size_t workspace_bytes, const pa_decode_opts* opts, void* stream);

/* Bytes of workspace pa_decode_cascade needs (0 for invalid arguments). */
size_t pa_decode_cascade_workspace_size(const pa_tensor* q, const pa_tensor* k_cache,
                                        const pa_tensor* block_tables, const pa_tensor* prefix_tables,
                                        int32_t max_group_size, const pa_decode_opts* opts);

/*
 * Checks of the device-side preconditions the hot-path calls leave
 * unchecked. Each waits for `stream` and copies the index arrays to host
 * memory (no device allocation): debugging aids, not for the decode loop.
 * They return PA_OK, PA_ERR_PRECONDITION, an argument error, or
 * PA_ERR_LAUNCH if a copy fails. k_cache supplies the pool size and block
 * size only.
 *
 * pa_check_cache_write_inputs: every slot is negative (skipped) or in
 *   [0, num_blocks * block_size), and no slot appears twice (Tutorial §4.2,
 *   PagedKVCache: each appended token gets its own row).
 * pa_check_decode_inputs: every context length is in
 *   [0, max_blocks_per_seq * block_size] and the table entries covering it
 *   (the first ceil(ctx / block_size) of the row) are in [0, num_blocks).
 * pa_check_multi_inputs: those of pa_check_decode_inputs, and query_start
 *   non-decreasing from 0 with every n_i in [0, min(max_query_len,
 *   context_lens[i])] (a query token is one of the sequence's cached ones).
 * pa_check_cascade_inputs: group_start non-decreasing from >= 0 to
 *   <= num_seqs with no group larger than max_group_size; every prefix
 *   length a multiple of block_size in [0, max_prefix_blocks * block_size];
 *   the prefix table entries covering it in [0, num_blocks).
 */
int pa_check_cache_write_inputs(const pa_tensor* slot_mapping, const pa_tensor* k_cache, void* stream);
int pa_check_decode_inputs(const pa_tensor* block_tables, const pa_tensor* context_lens,
                           const pa_tensor* k_cache, void* stream);
int pa_check_multi_inputs(const pa_tensor* block_tables, const pa_tensor* context_lens,
                          const pa_tensor* query_start, int32_t max_query_len, const pa_tensor* k_cache,
                          void* stream);
int pa_check_cascade_inputs(const pa_tensor* prefix_tables, const pa_tensor* prefix_lens,
                            const pa_tensor* group_start, int32_t max_group_size, int32_t num_seqs,
                            const pa_tensor* k_cache, void* stream);

/*
 * pa_probe_stream_read -- read `bytes` bytes of device memory once with
 * 16-byte loads (default cache policy, or non-temporal like the decode
 * kernels' KV loads when `nontemporal` is nonzero). A measurement aid: the
 * read bandwidth a kernel of this library reaches on the current GPU, the
 * practical ceiling next to the published HBM peak. `sink` (device, >= 256
 * uint32) is written only in a case the data never produces in practice.
 * bytes must be a multiple of 16; buf 16-byte aligned.
 */
int pa_probe_stream_read(const void* buf, int64_t bytes, int32_t nontemporal, uint32_t* sink, void* stream);

/* Host-side reference of the kernels' fp8 encoder (same source as the
 * device code): n float32 inputs, already divided by the scale, to e4m3fn
 * codes. Host pointers. For testing the rounding rule without a GPU. */
void pa_fp8_e4m3fn_encode_host(const float* x, uint8_t* codes, int64_t n);

/* Static description of a status code. */
const char* pa_strerror(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
