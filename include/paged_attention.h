/*
 * Paged decode attention for AMD Instinct MI355X (gfx950): C ABI.
 *
 * One new query token per (sequence, query head) attends over the K/V vectors
 * of its context, which sit in fixed-size physical cache blocks reached
 * through a per-sequence block table.  This is the "single query cached KV
 * attention" operation of vLLM PR #420 ("[OPTIMIZATION] Optimizes the
 * single_query_cached_kv_attention kernel"), with the MQA/GQA head mapping of
 * vLLM PR #452 ("Optimize MQA Kernel": head_mapping = repeat_interleave(
 * arange(num_kv_heads), num_queries_per_kv), num_heads % num_kv_heads == 0),
 * the optional ALiBi bias switched by use_alibi in the kernel-latency
 * benchmark of vLLM PR #2744 ("[Performance] Support MQA/GQA in decode phase
 * by using FlashAttention"), and the split-context variant that the same
 * page's "Paged attention V2" column times.  gather_cached_kv is the copy of
 * cached K/V rows into contiguous tensors of vLLM PR #29 ("Memcpy kernel for
 * flash attention").
 *
 * For sequence s with context length L = context_lens[s] and query head h:
 *
 *   kvh        = h / (num_heads / num_kv_heads)
 *   z_t        = scale * dot(query[s,h,:], K_s[kvh, t, :])
 *                + (alibi_slopes ? alibi_slopes[h] * (t - (L - 1)) : 0)
 *   out[s,h,:] = sum_t softmax(z)_t * V_s[kvh, t, :],   t = 0 .. L - 1
 *
 * where token t of sequence s is row (t % block_size) of physical block
 * block_tables[s, t / block_size].
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are device memory owned by the caller.  The library
 *     allocates nothing and keeps no device memory.
 *   - Tensors are dense and row-major in the layouts stated below.
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call
 *     returns without synchronising; outputs are valid once the stream has
 *     reached that point.  The library never reads device memory on the host.
 *   - Return value: PA_OK (0) or one of the PA_ERR_* codes.  Every code but
 *     PA_ERR_LAUNCH means nothing was enqueued; PA_ERR_LAUNCH (the runtime
 *     rejected a kernel launch) can follow earlier kernels of the same call
 *     that were enqueued.  pa_last_error() then gives a message for the
 *     calling thread.  No entry point aborts, throws or exits.
 *   - Entry points are thread-safe and re-entrant.
 */
#ifndef PAGED_ATTENTION_H
#define PAGED_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Identical to hipStream_t. */
typedef struct ihipStream_t* pa_stream_t;

/* Storage types.  Query and output are PA_F16 or PA_BF16; caches are the
 * same type, or PA_FP8_E4M3 (OCP FP8 E4M3FN: bias 7, no infinities, NaN =
 * 0x7F/0xFF) with one fp32 scale per cache tensor (see pa_dims). */
typedef enum { PA_F16 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

/* Storage of the K/V caches relative to the query type. */
typedef enum {
  PA_KV_NATIVE = 0,  /* caches hold the query type (dtype)                      */
  PA_KV_FP8_E4M3 = 1 /* caches hold FP8 E4M3 codes; value = code * k/v_scale   */
} pa_kv_format;

/* Where K and V tiles sit relative to each other.  A tile is the block_size x
 * head_size slab of one (physical block, kv head); every layout keeps a tile
 * contiguous, rows of head_size elements.
 *   PA_KV_SEPARATE  two tensors, key_cache and value_cache, each
 *                   [num_blocks, num_kv_heads, block_size, head_size].
 *   PA_KV_JOINT     one tensor [num_blocks, num_kv_heads, 2, block_size,
 *                   head_size]: the K tile of (block, kv head) followed by its
 *                   V tile.  key_cache points at the first K tile and
 *                   value_cache at the first V tile, i.e. value_cache must be
 *                   key_cache + block_size * head_size elements.
 * Results do not depend on the layout.  The joint layout reads each
 * (block, kv head) as one contiguous run of K and V; on MI355X it measured
 * faster for decode than two tensors at whatever relative address the
 * allocator gives them. */
typedef enum { PA_KV_SEPARATE = 0, PA_KV_JOINT = 1 } pa_kv_layout;

/* Status codes. */
enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* null pointer, bad dimension, inconsistent arguments   */
  PA_ERR_UNSUPPORTED = 2, /* dtype / head_size / block_size / group size not built */
  PA_ERR_ALIGNMENT = 3,   /* pointer not aligned as required                        */
  PA_ERR_WORKSPACE = 4,   /* a forced split needs more workspace than given         */
  PA_ERR_LAUNCH = 5,      /* the HIP runtime rejected a launch                      */
  PA_ERR_DEVICE = 6       /* device query failed                                    */
};

/* Shapes of one decode call.
 *   query        [num_seqs, num_heads, head_size]                     dtype
 *   out          [num_seqs, num_heads, head_size]                     dtype
 *   key_cache    [num_blocks, num_kv_heads, block_size, head_size]    dtype   (strides
 *   value_cache  [num_blocks, num_kv_heads, block_size, head_size]    dtype    per kv_layout)
 *   block_tables [num_seqs, max_blocks_per_seq]                       int32
 *   context_lens [num_seqs]                                           int32
 *   alibi_slopes [num_heads]                                          float32, or NULL
 * Supported: head_size 64 or 128; block_size a power of two in [8, 256];
 * num_heads % num_kv_heads == 0 with num_heads / num_kv_heads <= 64; query
 * fp16 or bf16; caches of the query type or FP8 E4M3 (1 byte per element).
 * The fp8 cache format is this library's reading of the "fp8 kv cache" the
 * FlashAttention-decode page (vLLM PR #2744) names without defining. */
typedef struct {
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_size;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t dtype;     /* pa_dtype of query and out: PA_F16 or PA_BF16           */
  int32_t kv_format; /* pa_kv_format; 0 (native) for 16-bit caches             */
  float k_scale;     /* FP8 caches: real key = code * k_scale (finite, > 0)    */
  float v_scale;     /* FP8 caches: real value = code * v_scale; both ignored
                        for native caches                                      */
  int32_t kv_layout; /* pa_kv_layout; 0 (separate) when zero-initialised     */
} pa_dims;

/* Which inner engine computes q.K and p.V. */
typedef enum {
  PA_ENGINE_AUTO = 0, /* the planner's choice                                         */
  PA_ENGINE_VALU = 1, /* vector ALU: packed dot products, DPP cross-lane reductions     */
  PA_ENGINE_MFMA = 2  /* matrix cores: the query group as a 16-wide MFMA tile           */
} pa_engine;

/* How a decode call that splits the context on the matrix-core engine lays
 * its work out over workgroups.  GRID and LONGEST_FIRST cut each sequence into
 * fixed partitions, one workgroup each; with ragged context lengths these
 * units differ in size, and starting the longest first (a small ordering
 * kernel runs before the decode kernel) shortens the tail of the launch; on
 * the LDS-staged kernel at one workgroup per CU, the workgroups after the
 * first round take the remaining units in the order they start (a counter in
 * the workspace), so CUs that free first take the longer ones.
 * GRID and LONGEST_FIRST give identical results.  EQUAL_SHARES (groups of
 * more than 16 heads, at most 2048 sequences): as many workgroups as the
 * device holds at once each walk an equal share of the batch's cache tiles,
 * across sequence boundaries, and the pieces of a sequence are merged after;
 * its results differ from the partitioned schedules only by rounding. */
typedef enum {
  PA_SCHEDULE_AUTO = 0,          /* groups of more than 16 heads, when the plan
                                    splits: equal shares if the batch has fewer
                                    (kv head, sequence) items than the CUs hold
                                    decode workgroups, else longest first; other
                                    groups: the grid's order                      */
  PA_SCHEDULE_GRID = 1,          /* the grid's order (partition-major)              */
  PA_SCHEDULE_LONGEST_FIRST = 2, /* longest first whenever the plan splits (MFMA)   */
  PA_SCHEDULE_EQUAL_SHARES = 3   /* equal shares where they apply (see above), even
                                    when the auto plan would not split; otherwise
                                    as AUTO without equal shares                   */
} pa_schedule;

/* Optional overrides (pass NULL for the defaults). */
typedef struct {
  /* 0: the planner decides; -1: force one pass per (sequence, kv head);
   * > 0: force partitions of this many tokens (a multiple of block_size). */
  int32_t partition_size;
  int32_t engine;   /* pa_engine */
  int32_t num_cus;  /* 0: query the current device; > 0: plan for this many CUs */
  int32_t schedule; /* pa_schedule */
} pa_opts;

/* A launch plan (output of paged_attention_plan). */
typedef struct {
  int32_t num_partitions; /* partitions per sequence; 1 = single pass, no reduce.
                             EQUAL_SHARES: the most workgroups the call launches
                             (CUs times what the kernel's LDS lets one CU hold)  */
  int32_t partition_size; /* tokens per partition (multiple of block_size);
                             0 for EQUAL_SHARES                                   */
  int32_t engine;         /* resolved pa_engine                                     */
  int32_t schedule;       /* resolved: PA_SCHEDULE_GRID, _LONGEST_FIRST or
                             _EQUAL_SHARES                                          */
  size_t workspace_bytes; /* workspace this plan uses (0 for a single pass)         */
} pa_plan;

/*
 * paged_attention_decode -- decode attention over a paged KV cache.
 *
 * out, query, key_cache, value_cache, block_tables, context_lens: see pa_dims.
 *   out, query, key_cache and value_cache must be 16-byte aligned,
 *   block_tables and context_lens 4-byte aligned.
 * scale        multiplies q.k (callers normally pass 1/sqrt(head_size)).
 * block_size   must equal dims->block_size.
 * alibi_slopes one fp32 slope per query head, or NULL for no bias.
 * stream       HIP stream the kernels are enqueued on.
 * dims         shapes (host memory).
 * workspace    device scratch for the split-context partials, 256-byte
 *              aligned, or NULL when workspace_bytes is 0.  Size it with
 *              paged_attention_workspace_bytes().  Contents on entry are
 *              ignored; the call owns it until the stream passes the call.
 * opts         NULL, or overrides (host memory).
 *
 * Device-side preconditions (not checked, as that would need a host read):
 *   block ids in block_tables[s, 0 .. ceil(L/block_size) - 1] lie in
 *   [0, num_blocks); 0 <= L <= max_blocks_per_seq * block_size (larger values
 *   are clamped to that bound).  Table entries past a sequence's last block
 *   and cache slots past L in its last block are never used and may hold
 *   anything, NaN included.  A sequence with L = 0 gets a zero output row.
 *
 * With opts == NULL an undersized workspace makes the planner use fewer
 * partitions (down to a single pass); it never fails for lack of workspace.
 * An equal-share plan (pa_schedule) launches the CUs' count times as many
 * workgroups of the decode kernel as one CU holds on the current device; the
 * call looks that occupancy up once per device and configuration.
 */
int paged_attention_decode(void* out, const void* query, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables,
                           const int32_t* context_lens, float scale, int32_t block_size,
                           const float* alibi_slopes, pa_stream_t stream, const pa_dims* dims,
                           void* workspace, size_t workspace_bytes, const pa_opts* opts);

/*
 * paged_attention_decode_noalloc -- paged_attention_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the split-context partials live
 * in a scratch array the library itself holds on each GPU, so the caller
 * passes only inputs and outputs.  Same kernels, same results (bit for bit)
 * as paged_attention_decode given an equally large workspace.
 *
 * Arguments as paged_attention_decode, without the workspace.  The scratch
 * holds at most PA_NOALLOC_SCRATCH_BYTES bytes: with opts == NULL (or
 * opts->partition_size == 0) the planner uses fewer partitions when a split
 * would need more, down to a single pass; a forced partition_size whose
 * partials exceed it returns PA_ERR_WORKSPACE.  The array is a static part of
 * the library's device code: each GPU the library runs on holds one until the
 * process ends, and the first call on a device looks up its address (with
 * that device current).  The call allocates nothing and fills no memory.
 *
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents: calls that overlap on one GPU (on different streams, or
 * from several threads without ordering) race and may return wrong results.
 * Calls ordered on one stream are safe.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, float scale, int32_t block_size,
                                   const float* alibi_slopes, pa_stream_t stream,
                                   const pa_dims* dims, const pa_opts* opts);

/*
 * paged_attention_workspace_bytes -- workspace the planner's choice needs for
 * these shapes and overrides when given unlimited workspace (0 if it picks a
 * single pass).  Host only; returns 0 for invalid dims.
 */
size_t paged_attention_workspace_bytes(const pa_dims* dims, const pa_opts* opts);

/*
 * paged_attention_plan -- the launch plan paged_attention_decode would use
 * with this much workspace.  Host only: it touches no device unless
 * opts->num_cus is 0, in which case it queries the current device's compute
 * unit count once.  Returns a status code; *plan is written on PA_OK.
 */
int paged_attention_plan(const pa_dims* dims, size_t workspace_bytes, const pa_opts* opts,
                         pa_plan* plan);

/*
 * paged_attention_prefill -- causal multi-query attention over the paged
 * cache: a chunk of new tokens per sequence attends to the cached prefix and
 * to itself (the pages note the FlashAttention cache call serves prefill with
 * and without a cached prefix, vLLM PR #2744 discussion).
 *
 * Sequence s owns the packed query rows query_start_loc[s] ..
 * query_start_loc[s+1] - 1 (n_s rows, n_s <= context_lens[s]); these are its
 * last n_s context tokens, whose K/V are already in the cache (written with
 * paged_kv_cache_write).  New token i of s sits at position
 * p = context_lens[s] - n_s + i and attends to positions 0 .. p:
 *
 *   out[row, h, :] = sum_{t <= p} softmax_t(scale * q[row, h].K_s[kvh, t]
 *                                          + alibi_h * (t - p)) V_s[kvh, t, :]
 *
 * With n_s = 1 for every sequence this is paged_attention_decode.
 *
 * query, out        [num_query_tokens, num_heads, head_size]  dtype
 * query_start_loc   [num_seqs + 1] int32, non-decreasing, [0] = 0,
 *                   [num_seqs] = num_query_tokens (device memory)
 * max_query_len     host-side bound on n_s (sizes the grid); 1 .. 65535
 * Everything else as paged_attention_decode (dims->num_seqs sequences).  The
 * matrix-core engine computes it (PA_ENGINE_VALU is rejected).  Device-side
 * preconditions: n_s <= max_query_len and n_s <= context_lens[s].
 */
int paged_attention_prefill(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, const int32_t* query_start_loc,
                            int32_t num_query_tokens, int32_t max_query_len, float scale,
                            int32_t block_size, const float* alibi_slopes, pa_stream_t stream,
                            const pa_dims* dims, void* workspace, size_t workspace_bytes,
                            const pa_opts* opts);

/* Workspace and plan of a paged_attention_prefill call (host only; see the
 * decode versions). */
size_t paged_attention_prefill_workspace_bytes(const pa_dims* dims, int32_t num_query_tokens,
                                               int32_t max_query_len, const pa_opts* opts);
int paged_attention_prefill_plan(const pa_dims* dims, int32_t num_query_tokens,
                                 int32_t max_query_len, size_t workspace_bytes,
                                 const pa_opts* opts, pa_plan* plan);

/*
 * gather_cached_kv -- copy cached K/V rows into contiguous tensors, bit for
 * bit (the operation benchmarked on vLLM PR #29, whose parameters are
 * num_tokens, num_heads, head_size, block_size and num_blocks).
 *
 * key_out, value_out  [num_tokens, num_kv_heads, head_size]            dtype
 * key_cache, value_cache [num_blocks, num_kv_heads, block_size, head_size] dtype,
 *                     laid out as kv_layout says (pa_kv_layout)
 * slot_mapping        [num_tokens] int32; slot = block * block_size + offset.
 *                     A negative slot writes a zero row.  Slots must be
 *                     < num_blocks * block_size (device-side precondition).
 * dtype: PA_F16, PA_BF16 or PA_FP8_E4M3 (bytes are moved, never converted).
 * A row (head_size elements) must be a multiple of 16 bytes; data pointers
 * 16-byte aligned.  Any block_size >= 1 is accepted.  The rows moved
 * (num_tokens * num_kv_heads * head_size elements) must be fewer than 2^31
 * 16-byte pieces (32 GiB per tensor), else PA_ERR_INVALID_ARG.
 */
int gather_cached_kv(void* key_out, void* value_out, const void* key_cache,
                     const void* value_cache, const int32_t* slot_mapping, int32_t num_tokens,
                     int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                     int32_t num_blocks, int32_t dtype, int32_t kv_layout, pa_stream_t stream);

/*
 * paged_kv_cache_write -- store the K/V rows of new tokens into their cache
 * slots, bit for bit: the cache operation that runs before decode attention
 * (vLLM PR #2744 discusses its cost at large block sizes).  Inverse of
 * gather_cached_kv.
 *
 * key_cache, value_cache [num_blocks, num_kv_heads, block_size, head_size] dtype (written),
 *                        laid out as kv_layout says (pa_kv_layout)
 * key, value             [num_tokens, num_kv_heads, head_size]             dtype
 * slot_mapping           [num_tokens] int32; slot = block * block_size + offset.
 *                        A negative slot (a padding token) stores nothing.
 * Device-side preconditions: slots < num_blocks * block_size and no two tokens
 * share a slot (otherwise which row lands there is unspecified).
 * dtype: PA_F16, PA_BF16 or PA_FP8_E4M3 (bytes are moved, never converted).
 * A row (head_size elements) must be a multiple of 16 bytes; data pointers
 * 16-byte aligned; fewer than 2^31 16-byte pieces of rows, as for
 * gather_cached_kv.
 */
int paged_kv_cache_write(void* key_cache, void* value_cache, const void* key, const void* value,
                         const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                         int32_t head_size, int32_t block_size, int32_t num_blocks, int32_t dtype,
                         int32_t kv_layout, pa_stream_t stream);

/* Static description of a status code. */
const char* pa_status_string(int status);

/* Message for the calling thread's most recent non-zero status ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTENTION_H */
