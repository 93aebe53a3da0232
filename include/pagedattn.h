/*
 * pagedattn.h -- C ABI of the MI355X (gfx950) paged-attention library
 * (libpagedattn.so).
 *
 * The operations are those of the "ROCm attention backends" blog (vLLM on
 * AMD ROCm; English summary and the vllm.com.cn translation):
 *   - the cache write that keeps the KV cache in the preshuffled layout
 *     (ROCM_AITER_FA section, key innovation 4, and the decode-path
 *     paragraph: the custom cache-write operator always leaves the cache
 *     shuffled so decode reads it with no layout conversion);
 *   - memory-bound decode attention over that cache (phase taxonomy:
 *     decode loads the whole KV cache per step), for GQA/MHA and for
 *     absorbed MLA over the 576-wide latent (MLA section);
 *   - log-sum-exp merging of partial results (extend-path pseudocode:
 *     every chunk yields an output and an LSE and the merge is stable);
 *   - chunked extend: new-token attention, then a loop of
 *     gather -> attention -> merge over context chunks within a per-
 *     iteration token budget, then a final merge (extend-path pseudocode).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are device pointers (HBM) unless the name ends in _host.
 *    The caller owns every buffer; the library never allocates or frees
 *    device memory, keeps no mutable global state and is re-entrant, with
 *    one exception: pa_paged_decode_attn_write_noalloc works in a device
 *    array of the library's own, shared by all its calls on a device.
 *  - `stream` is a hipStream_t (NULL: the null stream).  Work is enqueued
 *    on it asynchronously; nothing synchronises.
 *  - Tensors are dense, row-major, no padding.  bf16 is the storage type
 *    of queries, keys, values, latents and attention outputs; arithmetic is
 *    fp32.  LSE values are natural-log log-sum-exp of the scaled scores,
 *    fp32, laid out [tokens, heads]; an empty set of keys gives out = 0 and
 *    lse = -inf.
 *  - Argument checks run on the host before anything is enqueued: a bad
 *    argument returns a status, enqueues nothing and leaves outputs
 *    untouched.  A failed launch returns PA_ERR_HIP.  Device data (block
 *    tables, lengths, slots) is range-checked in the kernels so that a bad
 *    entry never makes a kernel read or write outside the buffers whose
 *    sizes the arguments describe; the numerical result for such an entry
 *    is unspecified.
 *
 *  - Workspaces.  Every workspace the library sizes (the *_workspace_size
 *    queries) starts with the same region of PA_WORKSPACE_COUNTER_BYTES
 *    bytes of int32 completion counters, one per split (sequence, kv head)
 *    pair of a decode call; whatever else a call keeps in its workspace
 *    lies after that region.  A decode call that splits leaves every
 *    counter zero again and no call writes anything else into the region,
 *    so a workspace zero-filled once (e.g. one hipMemset at allocation)
 *    can serve any sequence of calls on one stream, of any shapes and any
 *    entry points, as long as it is at least as large as each call's size
 *    query.  Calls that may run concurrently must not share a workspace.
 *
 * Shuffled KV layout (x = 16 bytes / sizeof(bf16) = 8 elements):
 *   k_cache [num_blocks, num_kv_heads, head_dim / x, block_size, x]
 *   v_cache [num_blocks, num_kv_heads, block_size / x, head_dim, x]
 * A token's slot is physical_block * block_size + offset_in_block.
 * MLA latent layout: kv_cache [num_blocks, block_size, latent_dim].
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Size of the counter region at the start of every workspace; a split
 * decode call supports at most PA_WORKSPACE_COUNTER_BYTES / 4 (sequence,
 * kv head) pairs. */
#define PA_WORKSPACE_COUNTER_BYTES ((size_t)1 << 20)

typedef int32_t pa_status;
enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1,          /* null pointer, negative size, inconsistent shapes */
    PA_ERR_UNSUPPORTED = 2,          /* a valid shape outside the supported envelope */
    PA_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes < the size query's answer */
    PA_ERR_HIP = 4                   /* a HIP call or launch failed */
};

enum { PA_BF16 = 0, PA_F32 = 1 };                           /* element types for merge */
/* cache layouts; PA_LAYOUT_STANDARD_KV is the unshuffled
 * [num_blocks, block_size, num_kv_heads, head_dim] cache, kept only so that
 * the shuffled layout can be compared against it */
enum { PA_LAYOUT_SHUFFLED_KV = 0, PA_LAYOUT_MLA_LATENT = 1, PA_LAYOUT_STANDARD_KV = 2 };

/* Human-readable name of a status code (static storage). */
const char *pa_status_string(pa_status s);

/*
 * Cache write (reshape_and_cache).  Stage 1 of every forward on the pages:
 * the new tokens' K/V go into the paged cache before attention runs.
 *
 * PA_LAYOUT_SHUFFLED_KV: key, value [num_tokens, num_kv_heads, head_dim]
 *   bf16 are scattered into k_cache / v_cache in the shuffled layout.
 * PA_LAYOUT_STANDARD_KV: the same key and value rows are copied to
 *   k_cache / v_cache [num_blocks, block_size, num_kv_heads, head_dim].
 * PA_LAYOUT_MLA_LATENT: key is the latent [num_tokens, head_dim] bf16
 *   (head_dim = latent width, e.g. 576); value and v_cache must be NULL,
 *   num_kv_heads must be 1; k_cache is the latent cache.
 * slot_mapping [num_tokens] int64: destination slot of each token.  A
 *   negative slot, or one >= num_blocks * block_size, is skipped.
 * Supported: shuffled layout needs head_dim in {64, 128} and block_size in
 *   {16, 32}; the standard and latent layouts need head_dim % 8 == 0 and
 *   any block_size >= 1.  num_tokens == 0 is a no-op.
 */
pa_status pa_reshape_and_cache(int32_t layout, const void *key, const void *value,
                               void *k_cache, void *v_cache, const int64_t *slot_mapping,
                               int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int64_t num_blocks, void *stream);

/*
 * Split-KV partition length the decode entry points use for these
 * arguments when they use fixed partitions: partition_tokens > 0 is rounded
 * up to a multiple of 64; 0 picks one from the work size; -1 asks for as few
 * partitions as possible.  Partitions are capped at 4096 tokens.  (With 0
 * the entry points may use the balanced split instead, see
 * pa_decode_uses_balanced_split.)
 */
int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                   int32_t max_context_len, int32_t partition_tokens);

/*
 * 1 if pa_paged_decode_attn with these arguments uses the balanced split
 * (partition_tokens == -2, or 0 when fixed auto-sized partitions would
 * need more than one wave of workgroups on the current device), else 0.
 */
int32_t pa_decode_uses_balanced_split(int32_t num_seqs, int32_t num_kv_heads,
                                      int32_t max_context_len, int32_t partition_tokens);

/* Bytes of workspace pa_paged_decode_attn needs (0 if no split is needed;
 * otherwise the counter region plus the partials).  For partition_tokens 0
 * and -2 the size depends on the current device's compute-unit count. */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len,
                                int32_t partition_tokens);

/*
 * GQA / MHA paged decode attention (paged_decode_attn): one query token per
 * sequence attends to all context_lens[s] tokens of its sequence, found
 * through block_table (decode path: reads the shuffled cache directly).
 *
 * out [num_seqs, num_q_heads, head_dim] bf16; lse [num_seqs, num_q_heads]
 *   f32 (nullable).  query [num_seqs, num_q_heads, head_dim] bf16.
 * block_table [num_seqs, max_blocks_per_seq] int32 physical block ids;
 *   entries past ceil(context_lens[s] / block_size) are never read.
 * context_lens [num_seqs] int32, counting the token the step just wrote;
 *   values above max_context_len or max_blocks_per_seq * block_size are
 *   clamped.  max_context_len is a host-side bound used to size the grid.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * scale multiplies q . k before the softmax.
 * partition_tokens: > 0 or -1: fixed-length partitions, see
 *   pa_decode_partition_tokens; -2: balanced split: a grid of as many
 *   workgroups as the device holds at once shares all 16-token sub-blocks
 *   of all (sequence, kv head) pairs in near-equal pieces, whatever the
 *   length mix; 0: auto-sized partitions when they fit in one wave of
 *   workgroups, the balanced split otherwise.  A (sequence, kv head) pair
 *   whose tokens are split writes partial (out, lse) to the workspace;
 *   they are merged by log-sum-exp in token order.
 * workspace: device memory of at least pa_decode_workspace_size(...)
 *   bytes, 256-byte aligned, whose counter region is zero (see
 *   Workspaces above); the partials follow the counter region.
 *   Unsplit calls need none (null is accepted).
 * Supported: head_dim in {64, 128}, block_size in {16, 32}, group size
 *   num_q_heads / num_kv_heads in 1..16, max_context_len <= 1 << 20; a
 *   split call with num_seqs * num_kv_heads above the counter capacity
 *   returns PA_ERR_UNSUPPORTED (with partition_tokens 0 such a batch uses
 *   fixed partitions, which need no split up to 4096 tokens).
 */
pa_status pa_paged_decode_attn(void *out, float *lse, const void *query, const void *k_cache,
                               const void *v_cache, const int32_t *block_table,
                               int32_t max_blocks_per_seq, const int32_t *context_lens,
                               int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, float scale, int32_t partition_tokens,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * A decode step in one launch: the cache write of each sequence's new token
 * (reshape_and_cache; the blog's decode path writes the new token into the
 * preshuffled cache, then attention reads the whole cache) fused into
 * pa_paged_decode_attn.
 *
 * new_key, new_value [num_seqs, num_kv_heads, head_dim] bf16 (16-byte
 *   aligned); slot_mapping [num_seqs] int64: sequence s's token goes to
 *   slot slot_mapping[s] = block * block_size + offset, written exactly as
 *   pa_reshape_and_cache writes it (bit for bit); a negative or out-of-pool
 *   slot is skipped.  k_cache and v_cache are written.
 * Every other argument, the workspace and the result are those of
 *   pa_paged_decode_attn on the cache after the write, provided that
 *   slot_mapping[s] is the slot of token context_lens[s] - 1 through the
 *   block table (the usual decode step): the workgroup that reads that token
 *   writes it first.  Another slot is written too, but a concurrent read of
 *   it may see the old contents.
 */
pa_status pa_paged_decode_attn_write(void *out, float *lse, const void *query,
                                     const void *new_key, const void *new_value,
                                     const int64_t *slot_mapping, void *k_cache, void *v_cache,
                                     const int32_t *block_table, int32_t max_blocks_per_seq,
                                     const int32_t *context_lens, int32_t max_context_len,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                     float scale, int32_t partition_tokens, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* Bytes of the library's per-device scratch array used by
 * pa_paged_decode_attn_write_noalloc (counter region included). */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * pa_paged_decode_attn_write without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The call itself
 * allocates nothing.  Its workspace is a file-scope device array of
 * PA_NOALLOC_SCRATCH_BYTES bytes inside the library, one per device, held
 * from the library's load until the process ends; its device address is
 * taken once per device on the first call there, which also enqueues a
 * clear of the array's counter region on `stream` ahead of the call's own
 * work.  Every other argument, the result and the errors are those of
 * pa_paged_decode_attn_write; a call whose pa_decode_workspace_size
 * exceeds PA_NOALLOC_SCRATCH_BYTES returns PA_ERR_WORKSPACE_TOO_SMALL with
 * nothing enqueued.  All calls on one device share its array, which keeps
 * the last call's contents: calls that overlap in time on one device
 * (concurrent streams, threads or processes sharing the array's device
 * memory) race and must be serialised by the caller.
 */
pa_status pa_paged_decode_attn_write_noalloc(void *out, float *lse, const void *query,
                                             const void *new_key, const void *new_value,
                                             const int64_t *slot_mapping, void *k_cache,
                                             void *v_cache, const int32_t *block_table,
                                             int32_t max_blocks_per_seq,
                                             const int32_t *context_lens, int32_t max_context_len,
                                             int32_t num_seqs, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int64_t num_blocks, float scale,
                                             int32_t partition_tokens, void *stream);

/*
 * Paged GQA decode over a cache in either layout, with or without the fused
 * cache write: the blog credits the preshuffled layout with 15-20% more
 * decode throughput than the standard KV cache layout (ROCM_AITER_FA
 * section, hardware-optimised KV cache layout); this entry runs the same
 * kernel over both so the difference can be measured.
 * layout: PA_LAYOUT_SHUFFLED_KV (as pa_paged_decode_attn /
 *   pa_paged_decode_attn_write) or PA_LAYOUT_STANDARD_KV: k_cache and
 *   v_cache [num_blocks, block_size, num_kv_heads, head_dim] bf16.  In the
 *   standard layout K is read as in the shuffled one (a lane's 16-byte
 *   vectors are 8 dims of one token) and V is transposed through LDS into
 *   the registers the shuffled V vectors fill, so both layouts give
 *   bit-identical results.
 * new_key, new_value, slot_mapping: all NULL (no cache write, as
 *   pa_paged_decode_attn) or all given (as pa_paged_decode_attn_write, the
 *   rows written in `layout`).  Everything else as pa_paged_decode_attn;
 *   the workspace size is the same for both layouts.
 * Errors: PA_ERR_INVALID_ARG for another layout or a partial write triple,
 *   otherwise as pa_paged_decode_attn.
 */
pa_status pa_paged_decode_attn_layout(int32_t layout, void *out, float *lse, const void *query,
                                      const void *new_key, const void *new_value,
                                      const int64_t *slot_mapping, void *k_cache, void *v_cache,
                                      const int32_t *block_table, int32_t max_blocks_per_seq,
                                      const int32_t *context_lens, int32_t max_context_len,
                                      int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int64_t num_blocks, float scale, int32_t partition_tokens,
                                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * FP8 KV cache.  The pages' MLA extend path gathers the context and
 * dequantises it when the cache is quantised (the blog's AITER MLA section,
 * extend pseudocode); they fix no format.  This library reads it as OCP
 * 8-bit E4M3 ("fn": no infinities, largest finite 448) with one float32
 * scale per tensor:
 *   value(code) = E4M3(code) * scale,
 *   code(x)     = nearest E4M3 value to float32(x) * float32(1 / scale),
 *                 ties to the even code, saturating at +-448.
 * Caches hold codes (uint8) in the shuffled layout with x = 16 codes per
 * 16-byte vector:
 *   k_cache [num_blocks, num_kv_heads, head_dim / 16, block_size, 16]
 *   v_cache [num_blocks, num_kv_heads, block_size / 16, head_dim, 16].
 *
 * pa_reshape_and_cache_fp8: key, value [num_tokens, num_kv_heads, head_dim]
 *   bf16 quantised with k_scale / v_scale into the caches at slot_mapping
 *   (as pa_reshape_and_cache: negative or out-of-pool slots are skipped).
 * Supported: head_dim in {64, 128}, block_size in {16, 32}; scales finite and
 * positive (PA_ERR_INVALID_ARG otherwise).
 */
pa_status pa_reshape_and_cache_fp8(const void *key, const void *value, void *k_cache,
                                   void *v_cache, const int64_t *slot_mapping, int64_t num_tokens,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int64_t num_blocks, float k_scale, float v_scale, void *stream);

/*
 * GQA paged decode over FP8 caches: pa_paged_decode_attn (or, with new_key,
 * new_value and slot_mapping all given, pa_paged_decode_attn_write, the new
 * token quantised as pa_reshape_and_cache_fp8 does) with K and V the
 * dequantised values code * k_scale and code * v_scale.  The codes are
 * converted exactly (every E4M3 value is a bf16); k_scale folds into the
 * softmax scale and v_scale into the output.  Workspace as for
 * pa_paged_decode_attn.  Supported: head_dim in {64, 128}, block_size in
 * {16, 32}, group size 1..16.
 */
pa_status pa_paged_decode_attn_fp8(void *out, float *lse, const void *query, const void *new_key,
                                   const void *new_value, const int64_t *slot_mapping,
                                   void *k_cache, void *v_cache, const int32_t *block_table,
                                   int32_t max_blocks_per_seq, const int32_t *context_lens,
                                   int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int64_t num_blocks, float scale, float k_scale, float v_scale,
                                   int32_t partition_tokens, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * The gather with dequantisation: pa_gather_cache_chunk over FP8 caches,
 * writing bf16(float(E4M3(code)) * scale) (float32 product, rounded to
 * nearest even) into the standard [rows, num_kv_heads, head_dim] outputs.
 * Supported: head_dim 128, block_size a multiple of 16.
 */
pa_status pa_gather_cache_chunk_fp8(void *k_out, void *v_out, const void *k_cache,
                                    const void *v_cache, const int32_t *block_table,
                                    int32_t max_blocks_per_seq, const int32_t *context_lens,
                                    int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int64_t num_blocks, int32_t iteration,
                                    int32_t chunk_tokens, float k_scale, float v_scale,
                                    void *stream);

/* Bytes of workspace pa_mla_decode_attn needs (0 if no split is needed).
 * For partition_tokens 0 and -2 the size depends on the current device's
 * compute-unit count. */
size_t pa_mla_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t v_dim,
                             int32_t max_context_len, int32_t partition_tokens);

/*
 * Absorbed MLA paged decode attention (mla_decode_attn; MLA section: decode
 * runs directly on the compressed 576-wide latent).  Every query head reads
 * the same latent row: keys are whole rows, values their first v_dim
 * entries.
 *
 * out [num_seqs, num_q_heads, v_dim] bf16; lse [num_seqs, num_q_heads] f32
 *   (nullable).  query [num_seqs, num_q_heads, latent_dim] bf16.
 * kv_cache [num_blocks, block_size, latent_dim] bf16.
 * block_table, context_lens, max_context_len, partition_tokens, workspace:
 *   as for pa_paged_decode_attn (with one kv head: the balanced split cuts
 *   each sequence into 32-token-tile pieces; pa_decode_uses_balanced_split
 *   with num_kv_heads = 1 tells which split the call uses).
 * Supported: latent_dim == 576, v_dim == 512, num_q_heads in 1..16,
 *   any block_size >= 1.
 */
pa_status pa_mla_decode_attn(void *out, float *lse, const void *query, const void *kv_cache,
                             const int32_t *block_table, int32_t max_blocks_per_seq,
                             const int32_t *context_lens, int32_t max_context_len,
                             int32_t num_seqs, int32_t num_q_heads, int32_t latent_dim,
                             int32_t v_dim, int32_t block_size, int64_t num_blocks, float scale,
                             int32_t partition_tokens, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * An MLA decode step in one launch: the cache write of each sequence's new
 * latent (reshape_and_cache, MLA layout) fused into pa_mla_decode_attn.
 * new_latent [num_seqs, latent_dim] bf16 (16-byte aligned); slot_mapping
 * [num_seqs] int64: sequence s's latent goes to slot slot_mapping[s]
 * exactly as pa_reshape_and_cache writes it; a negative or out-of-pool slot
 * is skipped.  kv_cache is written.  Everything else is as for
 * pa_mla_decode_attn on the cache after the write, provided that
 * slot_mapping[s] is the slot of token context_lens[s] - 1 through the block
 * table (the workgroup that reads that token writes it first).
 */
pa_status pa_mla_decode_attn_write(void *out, float *lse, const void *query,
                                   const void *new_latent, const int64_t *slot_mapping,
                                   void *kv_cache, const int32_t *block_table,
                                   int32_t max_blocks_per_seq, const int32_t *context_lens,
                                   int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t latent_dim, int32_t v_dim, int32_t block_size,
                                   int64_t num_blocks, float scale, int32_t partition_tokens,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * Absorbed MLA paged decode on the matrix cores (MLA section of the "vLLM ROCm
 * attention backends" blog: the assembly decode kernel of the pages keeps
 * the latent read at memory speed).  The same operation as
 * pa_mla_decode_attn, optionally with the fused latent write of
 * pa_mla_decode_attn_write: new_latent and slot_mapping both NULL (no write)
 * or both given.  QK (num_q_heads x 576 by 576 x tokens) and P.V (by
 * tokens x 512) run as bf16 matrix products with fp32 accumulation, the
 * weights as bf16 hi + lo parts; the result agrees with pa_mla_decode_attn
 * to rounding.  Arguments, workspace (pa_mla_workspace_size), support and
 * errors as for pa_mla_decode_attn; bf16 latents (FP8 latents:
 * pa_mla_decode_attn_fp8_mfma).
 */
pa_status pa_mla_decode_attn_mfma(void *out, float *lse, const void *query,
                                  const void *new_latent, const int64_t *slot_mapping,
                                  void *kv_cache, const int32_t *block_table,
                                  int32_t max_blocks_per_seq, const int32_t *context_lens,
                                  int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t latent_dim, int32_t v_dim, int32_t block_size,
                                  int64_t num_blocks, float scale, int32_t partition_tokens,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * FP8 latent cache (the MLA extend pseudocode of the "vLLM ROCm attention
 * backends" blog gathers the latent cache and may dequantise it; the code
 * format is that of pa_reshape_and_cache_fp8, with one scale for the whole
 * cache): kv_cache [num_blocks, block_size, latent_dim] E4M3 codes, value =
 * E4M3(code) * kv_scale.
 *
 * pa_reshape_and_cache_mla_fp8: latent [num_tokens, latent_dim] bf16
 *   quantised (nearest-even code of float32(x) * float32(1 / kv_scale),
 *   saturating at +-448) into the row of slot slot_mapping[i]; negative or
 *   out-of-pool slots are skipped.  Supported: latent_dim % 16 == 0.
 *
 * pa_mla_decode_attn_fp8: pa_mla_decode_attn over such a cache, keys and
 *   values the dequantised rows (the codes are converted exactly; kv_scale
 *   folds into the softmax scale and the output).  new_latent and
 *   slot_mapping: both NULL (no write) or both given (the fused write of
 *   pa_mla_decode_attn_write, quantised as above).  Workspace, support and
 *   errors as for pa_mla_decode_attn; kv_scale finite and positive
 *   (PA_ERR_INVALID_ARG otherwise).
 */
pa_status pa_reshape_and_cache_mla_fp8(const void *latent, void *kv_cache,
                                       const int64_t *slot_mapping, int64_t num_tokens,
                                       int32_t latent_dim, int32_t block_size, int64_t num_blocks,
                                       float kv_scale, void *stream);

pa_status pa_mla_decode_attn_fp8(void *out, float *lse, const void *query, const void *new_latent,
                                 const int64_t *slot_mapping, void *kv_cache,
                                 const int32_t *block_table, int32_t max_blocks_per_seq,
                                 const int32_t *context_lens, int32_t max_context_len,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t latent_dim,
                                 int32_t v_dim, int32_t block_size, int64_t num_blocks,
                                 float scale, float kv_scale, int32_t partition_tokens,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_mla_decode_attn_fp8 on the matrix cores: the operation and arguments of
 * pa_mla_decode_attn_fp8 (FP8 latent cache, kv_scale, optional fused write),
 * computed as pa_mla_decode_attn_mfma computes it, the codes widened exactly
 * to bf16 on chip and kv_scale folded into the softmax scale and the output.
 * Workspace (pa_mla_workspace_size), support and errors as for
 * pa_mla_decode_attn_fp8.
 */
pa_status pa_mla_decode_attn_fp8_mfma(void *out, float *lse, const void *query,
                                      const void *new_latent, const int64_t *slot_mapping,
                                      void *kv_cache, const int32_t *block_table,
                                      int32_t max_blocks_per_seq, const int32_t *context_lens,
                                      int32_t max_context_len, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t latent_dim, int32_t v_dim,
                                      int32_t block_size, int64_t num_blocks, float scale,
                                      float kv_scale, int32_t partition_tokens, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * Log-sum-exp merge of two partial attention results (merge_attn_states;
 * extend-path pseudocode): with M = max(Lp, Ls), wp = exp(Lp - M),
 * ws = exp(Ls - M): out = (wp * Op + ws * Os) / (wp + ws),
 * out_lse = M + log(wp + ws).  A part with lse = -inf has weight 0; two
 * empty parts give out = 0, out_lse = -inf.
 *
 * prefix_out, suffix_out [num_tokens, num_heads, head_dim] of in_dtype;
 * prefix_lse, suffix_lse [num_tokens, num_heads] f32; out of out_dtype,
 * out_lse f32 (nullable).  out may be prefix_out or suffix_out itself (the
 * same address) when the dtypes match: each element is read before it is
 * written by the same thread.  Any other overlap between an output and an
 * input, and in particular out_lse overlapping prefix_lse or suffix_lse (a
 * row's LSEs are read by threads of several workgroups), returns
 * PA_ERR_INVALID_ARG.  Supported: head_dim % 8 == 0, head_dim <= 1024.
 */
pa_status pa_merge_attn_states(void *out, float *out_lse, int32_t out_dtype,
                               const void *prefix_out, const float *prefix_lse,
                               const void *suffix_out, const float *suffix_lse, int32_t in_dtype,
                               int64_t num_tokens, int32_t num_heads, int32_t head_dim,
                               void *stream);

/*
 * Per-request chunk length one extend iteration gathers: the budget spread
 * over the requests that still have context, rounded down to a multiple of
 * block_size (at least block_size).
 */
int32_t pa_extend_chunk_tokens(int32_t num_seqs, int32_t block_size,
                               int32_t chunk_budget_tokens);

/*
 * Context gather of one extend iteration (extend-path pseudocode: each
 * chunk of cached context is copied out of the shuffled cache into the
 * standard [tokens, kv_heads, head_dim] layout before attention).
 * Request r contributes its context tokens
 *   [iteration * chunk_tokens, min((iteration + 1) * chunk_tokens, context_lens[r]))
 * in order; requests follow each other, so request r's first row is the sum
 * of the earlier requests' lengths.  k_out, v_out [rows, num_kv_heads,
 * head_dim] bf16 with rows <= num_seqs * chunk_tokens.  The copy is exact
 * (bit for bit).  A block-table entry outside [0, num_blocks) gathers
 * zeros.  Supported: head_dim == 128, block_size and chunk_tokens multiples
 * of 8, chunk_tokens a multiple of block_size.
 */
pa_status pa_gather_cache_chunk(void *k_out, void *v_out, const void *k_cache,
                                const void *v_cache, const int32_t *block_table,
                                int32_t max_blocks_per_seq, const int32_t *context_lens,
                                int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int64_t num_blocks, int32_t iteration,
                                int32_t chunk_tokens, void *stream);

/* Bytes of workspace pa_chunked_extend_attn needs. */
size_t pa_extend_workspace_size(int32_t num_seqs, int32_t total_new_tokens, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t chunk_budget_tokens);

/*
 * Chunked extend attention (chunked_extend_attn; extend-path pseudocode).
 * Request r has context_lens[r] cached tokens (in the shuffled cache,
 * through block_table) and new query tokens at rows
 * query_start_loc[r] .. query_start_loc[r+1]; new token i attends to every
 * cached token and to new tokens 0..i.
 *
 * The pages' three stages (new-token causal attention; per context chunk of
 * pa_extend_chunk_tokens tokens, attention and a running LSE merge; a final
 * merge) are computed as follows: the context is cut into at most 4 pieces
 * of whole chunks; one pass per piece attends to the piece's chunks straight
 * from the shuffled cache (no gather copy) and, for the last piece, then to
 * the new tokens with the causal mask, all in one online softmax; a request
 * with several pieces gets its pieces merged by LSE (merge_attn_states over
 * n parts).  The result equals the three-stage recipe up to rounding order.
 *
 * out [total_new_tokens, num_q_heads, head_dim] bf16; lse
 *   [total_new_tokens, num_q_heads] f32 (nullable).
 * query [total_new_tokens, num_q_heads, head_dim] bf16; k_new, v_new
 *   [total_new_tokens, num_kv_heads, head_dim] bf16.
 * query_start_loc [num_seqs + 1] int32 on the device and the same values in
 *   query_start_loc_host; context_lens [num_seqs] int32 on the device and
 *   the same values in context_lens_host (the host copies size the launch
 *   without a device read-back; the kernels read the device copies and stay
 *   in bounds if the two disagree).
 * A block-table entry outside [0, num_blocks) reads as zero K and V.
 * The workspace (pa_extend_workspace_size bytes, 256-byte aligned) holds,
 *   after the counter region (which the call neither reads nor writes), the
 *   plan, the new tokens' V regrouped into 8-token groups and the pieces'
 *   fp32 partials; it needs no initialisation.
 * Supported: head_dim == 128, block_size in {16, 32}, group size 1..16,
 *   context lengths up to 2^20.
 */
pa_status pa_chunked_extend_attn(void *out, float *lse, const void *query, const void *k_new,
                                 const void *v_new, const int32_t *query_start_loc,
                                 const int32_t *query_start_loc_host, const void *k_cache,
                                 const void *v_cache, const int32_t *block_table,
                                 int32_t max_blocks_per_seq, const int32_t *context_lens,
                                 const int32_t *context_lens_host, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks, float scale,
                                 int32_t chunk_budget_tokens, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * Three-path routing of one mixed batch (the blog's ROCM_AITER_FA section:
 * decode, extend and prefill requests go to separate kernels, after the model
 * runner has reordered the batch as [decode : extend : prefill] with a
 * reorder threshold of one token).
 *
 * A request r has query_start_loc[r + 1] - query_start_loc[r] >= 1 new
 * tokens and context_lens[r] cached tokens before them.  It is decode when
 * it has one new token (it attends to its cached tokens and itself),
 * prefill when it has more and nothing is cached, extend otherwise.
 *
 * pa_mixed_batch_plan (host only): order_host[0 .. num_reqs) receives the
 *   request indices in [decode : extend : prefill] order, stable within each
 *   path; counts_host[0..3) the number of decode, extend and prefill
 *   requests.  PA_ERR_INVALID_ARG if a request has no new token, a negative
 *   context, or query_start_loc_host[0] != 0.
 */
pa_status pa_mixed_batch_plan(int32_t num_reqs, const int32_t *query_start_loc_host,
                              const int32_t *context_lens_host, int32_t *order_host,
                              int32_t *counts_host);

/* Bytes of workspace pa_mixed_batch_attn needs for this batch (0 on invalid
 * arguments). */
size_t pa_mixed_batch_workspace_size(int32_t num_reqs, const int32_t *query_start_loc_host,
                                     const int32_t *context_lens_host, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int32_t chunk_budget_tokens);

/*
 * Attention of one mixed batch already in [decode : extend : prefill] order
 * (PA_ERR_INVALID_ARG otherwise), on one stream: the cache write of every
 * new token (pa_reshape_and_cache, shuffled layout), then
 * pa_paged_decode_attn over the decode requests (context length cached + 1)
 * and one pa_chunked_extend_attn over the extend and prefill requests, which
 * the order leaves adjacent (the extend kernel takes a request with nothing
 * cached as a causal prefill).
 * out [T, num_q_heads, head_dim] bf16 and lse [T, num_q_heads] f32
 *   (nullable) for the T = query_start_loc_host[num_reqs] new tokens, in
 *   batch order; query [T, num_q_heads, head_dim], key / value
 *   [T, num_kv_heads, head_dim] bf16 of the new tokens; slot_mapping [T]
 *   int64 their cache slots (token i of request r at position
 *   context_lens[r] + i through block_table row r).
 * query_start_loc [num_reqs + 1], context_lens [num_reqs] int32 on the
 *   device, with the same values in the _host copies (read during the call).
 * k_cache, v_cache: the shuffled caches; block_table [num_reqs,
 *   max_blocks_per_seq].  The workspace (pa_mixed_batch_workspace_size
 *   bytes, 256-byte aligned) needs no initialisation: the call zeroes the
 *   counters its decode step uses, and like every call leaves the counter
 *   region zero.
 * Supported: what the three paths support (head_dim 128 when an extend or
 *   prefill request is present).  Errors of a path are returned as they are;
 *   paths launched before it have run.
 */
pa_status pa_mixed_batch_attn(void *out, float *lse, const void *query, const void *key,
                              const void *value, const int64_t *slot_mapping,
                              const int32_t *query_start_loc, const int32_t *query_start_loc_host,
                              const int32_t *context_lens, const int32_t *context_lens_host,
                              void *k_cache, void *v_cache, const int32_t *block_table,
                              int32_t max_blocks_per_seq, int32_t num_reqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, float scale, int32_t chunk_budget_tokens,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Streaming read (a measurement aid, not a step of the method): reads the
 * `bytes` bytes at src once, in 16-byte vectors, with `workgroups`
 * workgroups of 256 threads walking the buffer grid-stride, and stores one
 * xor word per workgroup in sink[0 .. workgroups) when verify is nonzero
 * (with verify 0 nothing is reduced and a lane stores its own word only if
 * it is all ones, so that a timed read adds no reduction or store drain; the
 * sink contents are then meaningless).  Its time at a given size
 * is the yardstick for the decode kernels' achieved bandwidth: the paged
 * decode's claim is to be memory-bound, and this is what plain reading of
 * the same number of bytes achieves on the same GPU.
 * src: device, 16-byte aligned, bytes a multiple of 16.  sink: device,
 * `workgroups` uint32 words.  workgroups in [1, 65536].
 * Errors: PA_ERR_INVALID_ARG (nothing launched), PA_ERR_HIP.
 */
pa_status pa_stream_read(const void *src, size_t bytes, uint32_t *sink, int32_t workgroups,
                         int32_t verify, void *stream);

/*
 * Block-table gather read (a measurement aid, not a step of the method):
 * for every sequence s < num_seqs and kv head g < num_kv_heads, reads the
 * K and V units of the blocks that hold the sequence's first
 * context_lens[s] tokens -- unit_bytes each from k_cache and from v_cache
 * at byte (block_table[s * max_blocks_per_seq + b] * num_kv_heads + g) *
 * unit_bytes, b < ceil(context_lens[s] / block_size), the bytes a decode
 * over the preshuffled cache reads (unit_bytes = head_dim * block_size *
 * element size) -- one wave per block, four blocks per workgroup of 256
 * threads, grid ordered block-major like the decode's partition-major grid,
 * in 16-byte vectors folded into xor words.  Its time is the yardstick for
 * the decode's bandwidth on its own access pattern: the same blocks, no
 * arithmetic.  Context lengths are clamped to [0, max_blocks_per_seq *
 * block_size]; block ids outside [0, num_blocks) are skipped.  sink: device,
 * one uint32 per workgroup (num_seqs * num_kv_heads *
 * ceil(max_blocks_per_seq / 4) words): with verify nonzero workgroup
 * (b4 * num_seqs * num_kv_heads + s * num_kv_heads + g) stores the xor of
 * every 32-bit word it read (the K and V units of blocks 4 b4 .. 4 b4 + 3
 * of (s, g)); with verify 0 the contents are meaningless, as in
 * pa_stream_read.  Caches 16-byte aligned; unit_bytes a multiple of 1024 in
 * [1024, 65536].
 * Errors: PA_ERR_INVALID_ARG (nothing launched), PA_ERR_HIP.
 */
pa_status pa_gather_read(const void *k_cache, const void *v_cache, const int32_t *block_table,
                         const int32_t *context_lens, int32_t num_seqs, int32_t num_kv_heads,
                         int32_t max_blocks_per_seq, int32_t block_size, int64_t num_blocks,
                         int32_t unit_bytes, uint32_t *sink, int32_t verify, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
