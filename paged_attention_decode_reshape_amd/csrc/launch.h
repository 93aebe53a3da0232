// Host-side launchers of the gfx950 kernels (internal; the public ABI is
// include/pagedattn.h).  Each launcher enqueues on `stream` and returns
// hipGetLastError() after the launch.  Arguments are assumed validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

hipError_t launch_cache_write_shuffled(const void *key, const void *value, void *k_cache,
                                       void *v_cache, const int64_t *slot_mapping,
                                       int64_t num_tokens, int Hkv, int D, int B,
                                       int64_t num_blocks, hipStream_t stream);

hipError_t launch_cache_write_standard(const void *key, const void *value, void *k_cache,
                                       void *v_cache, const int64_t *slot_mapping,
                                       int64_t num_tokens, int Hkv, int D, int B,
                                       int64_t num_blocks, hipStream_t stream);
hipError_t launch_cache_write_fp8(const void *key, const void *value, void *k_cache, void *v_cache,
                                  const int64_t *slot_mapping, int64_t num_tokens, int Hkv, int D,
                                  int B, int64_t num_blocks, float k_inv, float v_inv,
                                  hipStream_t stream);
hipError_t launch_cache_write_latent(const void *latent, void *kv_cache,
                                     const int64_t *slot_mapping, int64_t num_tokens, int Dl,
                                     int B, int64_t num_blocks, hipStream_t stream);
hipError_t launch_cache_write_latent_fp8(const void *latent, void *kv_cache,
                                         const int64_t *slot_mapping, int64_t num_tokens, int Dl,
                                         int B, int64_t num_blocks, float inv, hipStream_t stream);

struct DecodeParams {
    void *out;                 // bf16 [S, Hq, D]
    float *lse;                // f32 [S, Hq] or null
    const void *query;         // bf16 [S, Hq, D]
    const void *k_cache;       // shuffled (or standard: std_layout)
    const void *v_cache;       // shuffled (or standard: std_layout)
    const int32_t *block_table;
    int32_t max_blocks;
    const int32_t *context_lens;
    int32_t max_ctx;           // context lengths are clamped to this and max_blocks * B
    int32_t S, Hq, Hkv, D, B;
    int64_t num_blocks;
    float scale;
    int32_t partition;         // tokens per partition (multiple of 64)
    int32_t max_parts;         // partitions per sequence in the grid
    float *part_out;           // f32 [S, Hq, max_parts, D] (when max_parts > 1),
                               //   [balanced_workgroups, Hq / Hkv, D] (balanced)
    float *part_lse;           // f32 [S, Hq, max_parts] / [balanced_workgroups, Hq / Hkv]
    int *counters;             // [S, Hkv] pieces finished; zero between calls
    int32_t balanced_workgroups;  // > 0: balanced split over at most this many workgroups
    int32_t num_cus;              // compute units of the device (balanced split)
    // Fused cache write (null slot_mapping: none): new_key / new_value
    // [S, Hkv, D] bf16, sequence s's token goes to slot slot_mapping[s]
    // (< 0: skipped) of the caches, written by the workgroup that
    // reads the sequence's last token before it reads it.
    const void *new_key, *new_value;
    const int64_t *slot_mapping;
    // cache layout: 0 shuffled bf16; 1 standard bf16 [num_blocks, block_size,
    // kv_heads, head_dim]; 2 shuffled FP8 E4M3 codes (x = 16) with per-tensor
    // scales (value = code * scale; the fused write quantises with the
    // float32 reciprocals k_inv, v_inv)
    int32_t layout;
    float k_scale, v_scale, k_inv, v_inv;
};

hipError_t launch_paged_decode(const DecodeParams &p, hipStream_t stream);

// The checks, split planning and launch behind every GQA decode entry point
// (api.hip): returns a pa_status.  layout: 0 shuffled bf16, 1 standard
// bf16, 2 shuffled FP8.  The workspace starts with the counter region.
// dry_run: every check (the workspace may be null, its size still counts),
// nothing enqueued.
int32_t decode_impl(int layout, float k_scale, float v_scale, void *out, float *lse,
                    const void *query, const void *new_key, const void *new_value,
                    const int64_t *slot_mapping, const void *k_cache, const void *v_cache,
                    const int32_t *block_table, int32_t max_blocks_per_seq,
                    const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int64_t num_blocks, float scale,
                    int32_t partition_tokens, void *workspace, size_t workspace_bytes,
                    void *stream, bool dry_run = false);

struct MLAParams {
    void *out;                 // bf16 [S, Hq, Dv]
    float *lse;                // f32 [S, Hq] or null
    const void *query;         // bf16 [S, Hq, Dl]
    const void *kv_cache;      // bf16 [NB, B, Dl]
    const int32_t *block_table;
    int32_t max_blocks;
    const int32_t *context_lens;
    int32_t S, Hq, Dl, Dv, B;
    int64_t num_blocks;
    float scale;
    int32_t max_ctx;           // context lengths are clamped to this and max_blocks * B
    int32_t partition;
    int32_t max_parts;
    float *part_out;           // f32 [S, Hq, max_parts, Dv] / [balanced_workgroups, Hq, Dv]
    float *part_lse;           // f32 [S, Hq, max_parts] / [balanced_workgroups, Hq]
    int *counters;             // [S] pieces finished; zero between calls
    int32_t balanced_workgroups;  // > 0: balanced split over at most this many workgroups
    int32_t num_cus;              // compute units of the device (balanced split)
    // Fused cache write (null slot_mapping: none): sequence s's new latent
    // new_latent[s] ([S, Dl] bf16) goes to slot slot_mapping[s] (< 0:
    // skipped), written by the workgroup that reads the sequence's last
    // token before it reads it.
    const void *new_latent;
    const int64_t *slot_mapping;
    // nonzero: kv_cache holds FP8 E4M3 codes [NB, B, Dl] with one scale
    // (value = code * kv_scale; the fused write quantises with kv_inv)
    int32_t fp8;
    float kv_scale, kv_inv;
    // nonzero: the matrix-core engine (bf16 latents only)
    int32_t mfma;
};

hipError_t launch_mla_decode(const MLAParams &p, hipStream_t stream);

// Chunked extend (extend.hip).
struct GatherParams {
    const void *k_cache;       // shuffled [NB, Hkv, D/8, B, 8]
    const void *v_cache;       // shuffled [NB, Hkv, B/8, D, 8]
    const int32_t *block_table;
    int32_t max_blocks;
    const int32_t *context_lens;  // [S] cached tokens per request
    int32_t S, Hkv, B;         // head_dim 128
    int64_t num_blocks;
    int32_t iteration, chunk;  // gathers context tokens [iteration * chunk, +chunk)
    void *k_out, *v_out;       // standard [rows, Hkv, D] bf16, request-major
    // nonzero: the caches hold FP8 codes (x = 16 layout) and the gather
    // writes bf16(code value * scale)
    int32_t fp8;
    float k_scale, v_scale;
};

hipError_t launch_gather_chunk(const GatherParams &p, int max_chunk_len, hipStream_t stream);

// Context pieces of one extend request: the context is cut into runs of
// whole chunks, at most max_pieces runs of about `target` tokens each;
// *piece_len receives the run length.  A request without context has one
// empty piece, which carries its new tokens.  Host and device both call
// this, so the grid and the kernels agree on the plan.  32-bit arithmetic:
// callers keep ctx, target and chunk within [0, 2^20].
__host__ __device__ inline int32_t extend_pieces(int32_t ctx, int32_t target, int32_t chunk,
                                                 int32_t max_pieces, int32_t *piece_len) {
    if (ctx <= 0) {
        *piece_len = 0;
        return 1;
    }
    int32_t n = (ctx + target - 1) / target;
    n = n < 1 ? 1 : (n > max_pieces ? max_pieces : n);
    int32_t len = (ctx + n - 1) / n;
    len = (len + chunk - 1) / chunk * chunk;
    *piece_len = len;
    return (ctx + len - 1) / len;
}

constexpr int32_t kExtendMaxPieces = 4;

struct ExtendParams {
    const void *q;             // bf16 [Tn, Hq, 128]
    const void *k_new;         // bf16 [Tn, Hkv, 128]
    const void *v_new;         // bf16 [Tn, Hkv, 128]
    void *v_new_sh;            // bf16 [Hkv, new_groups, 128, 8]: new V in 8-token groups
    int32_t new_groups;        // (Tn + 7) / 8 + S + 1; request r starts at group q_start[r] / 8 + r
    const void *k_cache;       // shuffled [NB, Hkv, 16, B, 8]
    const void *v_cache;       // shuffled [NB, Hkv, B / 8, 128, 8]
    const int32_t *block_table;
    int32_t max_blocks;
    int64_t num_blocks;
    const int32_t *q_start;    // [S + 1]
    const int32_t *context_lens;  // [S]
    int32_t *group_prefix;     // [S + 1]: workgroup groups before request r
    int32_t S, Hq, Hkv, B, Tn;
    int32_t chunk, piece_target, max_pieces;
    int32_t max_ctx;           // context lengths are clamped to [0, max_ctx] (<= 2^20)
    int32_t q_blocks;          // 128-row query blocks of the longest request
    int32_t num_groups;        // sum over requests of pieces * Hkv
    float scale;
    float *part_out;           // f32 [Tn * Hq, max_pieces, 128] (split requests)
    float *part_lse;           // f32 [Tn * Hq, max_pieces]
    void *out;                 // bf16 [Tn, Hq, 128]
    float *lse;                // f32 [Tn, Hq] or null
};

hipError_t launch_extend(const ExtendParams &p, int max_new, hipStream_t stream);

hipError_t launch_merge_pair(void *out, float *out_lse, int out_f32, const void *a,
                             const float *a_lse, const void *b, const float *b_lse, int in_f32,
                             int64_t rows, int D, hipStream_t stream);

}  // namespace pa
