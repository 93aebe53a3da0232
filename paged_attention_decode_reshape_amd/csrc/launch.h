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

hipError_t launch_cache_write_latent(const void *latent, void *kv_cache,
                                     const int64_t *slot_mapping, int64_t num_tokens, int Dl,
                                     int B, int64_t num_blocks, hipStream_t stream);

struct DecodeParams {
    void *out;                 // bf16 [S, Hq, D]
    float *lse;                // f32 [S, Hq] or null
    const void *query;         // bf16 [S, Hq, D]
    const void *k_cache;       // shuffled
    const void *v_cache;       // shuffled
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
};

hipError_t launch_paged_decode(const DecodeParams &p, hipStream_t stream);

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
};

hipError_t launch_gather_chunk(const GatherParams &p, int max_chunk_len, hipStream_t stream);

struct FAParams {
    const void *q;             // bf16 [Tn, Hq, 128]
    const void *k, *v;         // bf16 standard [rows, Hkv, 128]
    const int32_t *q_start;    // [S + 1] query rows of request r
    const int32_t *context_lens;  // chunk > 0: keys are the gathered chunk rows of request r
    int32_t iteration, chunk;  // chunk == 0: keys are the request's new tokens (rows of q)
    int32_t S, Hq, Hkv;
    float scale;
    float *run_out;            // fp32 [Tn, Hq, 128] running output
    float *run_lse;            // fp32 [Tn, Hq]
    void *out;                 // bf16 [Tn, Hq, 128] (final step)
    float *lse;                // fp32 [Tn, Hq] or null (final step)
};

// mode 0: result -> running state; mode 1: merged into it.  final_: write
// out / lse instead of the running state.
hipError_t launch_fa(const FAParams &p, int max_q_len, bool causal, int mode, bool final_,
                     hipStream_t stream);

hipError_t launch_merge_pair(void *out, float *out_lse, int out_f32, const void *a,
                             const float *a_lse, const void *b, const float *b_lse, int in_f32,
                             int64_t rows, int D, hipStream_t stream);

}  // namespace pa
