// C ABI of libpagedattn (declared in include/pagedattn.h): host-side
// argument checks, partition / chunk planning and kernel launches.
// Nothing here allocates device memory or keeps state between calls (the
// one entry point with device state of its own is in noalloc.hip).
#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "pagedattn.h"

using namespace pa;

namespace {

constexpr int32_t kMaxContext = 1 << 20;
constexpr int kAutoTargetWorkgroups = 1024;  // ~4 per CU on 256 CUs

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline pa_status from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }
// [a, a + an) and [b, b + bn) share a byte
inline bool overlaps(const void *a, size_t an, const void *b, size_t bn) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return an > 0 && bn > 0 && x < y + bn && y < x + an;
}

// A workgroup's 4 waves take 16-token sub-blocks round-robin and a wave
// tracks at most 64 of them, so a partition holds at most 4096 tokens.
constexpr int32_t kMaxPartition = 4096;

int32_t partition_tokens_for(int32_t S, int32_t H, int32_t max_ctx, int32_t requested) {
    const int32_t ctx = max_ctx > 0 ? max_ctx : 1;
    int32_t P;
    if (requested == -1)
        P = (int32_t)cdiv(ctx, 64) * 64;
    else if (requested > 0)
        P = (int32_t)cdiv(requested, 64) * 64;
    else {
        // auto: 256-token partitions, doubled while the grid would still hold
        // >= kAutoTargetWorkgroups workgroups
        P = 256;
        while (P < kMaxPartition &&
               (int64_t)S * H * cdiv(ctx, 2 * (int64_t)P) >= kAutoTargetWorkgroups)
            P *= 2;
    }
    return P < kMaxPartition ? P : kMaxPartition;
}

// Every workspace the library sizes starts with the same fixed region of
// completion counters (one int32 per split (sequence, kv head) pair);
// call-specific data follows it.  The split kernels leave their counters
// zero again, and no call writes anything else into the region, so one
// workspace zero-filled once serves any sequence of calls, whatever their
// shapes, and also when decode and extend calls share it.
constexpr size_t kCounterBytes = PA_WORKSPACE_COUNTER_BYTES;
constexpr int64_t kCounterCapacity = (int64_t)(kCounterBytes / sizeof(int32_t));
static_assert(kCounterBytes % 256 == 0, "counter region keeps the data 256-byte aligned");

struct Split {
    int32_t P;
    int32_t parts;
    size_t counter_bytes, out_bytes, lse_bytes;
    size_t total() const { return counter_bytes + out_bytes + lse_bytes; }
};

Split plan_split(int32_t S, int32_t Hq, int32_t H_units, int32_t Dv, int32_t max_ctx,
                 int32_t requested) {
    Split sp;
    sp.P = partition_tokens_for(S, H_units, max_ctx, requested);
    sp.parts = max_ctx > 0 ? (int32_t)cdiv(max_ctx, sp.P) : 1;
    if (sp.parts <= 1) {
        sp.parts = 1;
        sp.counter_bytes = sp.out_bytes = sp.lse_bytes = 0;
    } else {
        sp.counter_bytes = kCounterBytes;
        sp.out_bytes = align256((size_t)S * Hq * sp.parts * Dv * sizeof(float));
        sp.lse_bytes = align256((size_t)S * Hq * sp.parts * sizeof(float));
    }
    return sp;
}

// Balanced split (GQA decode): a grid of as many workgroups as fit on the
// device at once (at most kBalancedMaxPerCU per compute unit) shares all
// sub-blocks evenly; each workgroup leaves at most one partial result, so
// the workspace is sized for the maximum.  partition_tokens == -2 asks for
// it; 0 takes it when fixed auto-sized partitions would need more than
// one wave of workgroups (kAutoPartitionedPerCU per compute unit), where
// unequal sequence lengths leave a tail of lone workgroups.
constexpr int kBalancedMaxPerCU = 4;
constexpr int kAutoPartitionedPerCU = 2;
constexpr int32_t kRequestBalanced = -2;

int32_t device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    return cus;
}
int32_t balanced_workgroups() { return kBalancedMaxPerCU * device_cus(); }

// A split call needs one counter per (sequence, kv head) pair.
inline bool counters_fit(int32_t S, int32_t H_units) {
    return (int64_t)S * H_units <= kCounterCapacity;
}

bool decode_uses_balanced(int32_t S, int32_t Hkv, int32_t max_ctx, int32_t requested) {
    if (requested == kRequestBalanced) return true;
    if (requested != 0) return false;
    // auto with more pairs than counters: fixed partitions, which at this
    // many pairs are whole sequences whenever the context allows it
    if (!counters_fit(S, Hkv)) return false;
    const int32_t P = partition_tokens_for(S, Hkv, max_ctx, 0);
    const int64_t grid = (int64_t)S * Hkv * (max_ctx > 0 ? cdiv(max_ctx, P) : 1);
    return grid > (int64_t)kAutoPartitionedPerCU * device_cus();
}

Split plan_balanced(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t NW) {
    Split sp;
    sp.P = 0;
    sp.parts = 0;
    const size_t Ga = (size_t)(Hq / Hkv);
    sp.counter_bytes = kCounterBytes;
    sp.out_bytes = align256((size_t)NW * Ga * D * sizeof(float));
    sp.lse_bytes = align256((size_t)NW * Ga * sizeof(float));
    return sp;
}

}  // namespace

extern "C" {

const char *pa_status_string(pa_status s) {
    switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PA_ERR_HIP: return "HIP error";
    default: return "unknown status";
    }
}

pa_status pa_reshape_and_cache(int32_t layout, const void *key, const void *value, void *k_cache,
                               void *v_cache, const int64_t *slot_mapping, int64_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, void *stream) {
    if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1)
        return PA_ERR_INVALID_ARG;
    if (!key || !k_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
    if (!aligned(key, 16) || !aligned(k_cache, 16)) return PA_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    if (layout == PA_LAYOUT_SHUFFLED_KV) {
        if (!value || !v_cache || !aligned(value, 16) || !aligned(v_cache, 16))
            return PA_ERR_INVALID_ARG;
        if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
        if (block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
        if (num_tokens == 0) return PA_OK;
        return from_hip(launch_cache_write_shuffled(key, value, k_cache, v_cache, slot_mapping,
                                                    num_tokens, num_kv_heads, head_dim, block_size,
                                                    num_blocks, st));
    }
    if (layout == PA_LAYOUT_STANDARD_KV) {
        if (!value || !v_cache || !aligned(value, 16) || !aligned(v_cache, 16))
            return PA_ERR_INVALID_ARG;
        if (head_dim % 8 != 0) return PA_ERR_UNSUPPORTED;
        if (num_tokens == 0) return PA_OK;
        return from_hip(launch_cache_write_standard(key, value, k_cache, v_cache, slot_mapping,
                                                    num_tokens, num_kv_heads, head_dim,
                                                    block_size, num_blocks, st));
    }
    if (layout == PA_LAYOUT_MLA_LATENT) {
        if (value || v_cache || num_kv_heads != 1) return PA_ERR_INVALID_ARG;
        if (head_dim % 8 != 0) return PA_ERR_UNSUPPORTED;
        if (num_tokens == 0) return PA_OK;
        return from_hip(launch_cache_write_latent(key, k_cache, slot_mapping, num_tokens, head_dim,
                                                  block_size, num_blocks, st));
    }
    return PA_ERR_INVALID_ARG;
}

int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                                   int32_t partition_tokens) {
    return partition_tokens_for(num_seqs, num_kv_heads, max_context_len, partition_tokens);
}

int32_t pa_decode_uses_balanced_split(int32_t num_seqs, int32_t num_kv_heads,
                                      int32_t max_context_len, int32_t partition_tokens) {
    return decode_uses_balanced(num_seqs, num_kv_heads, max_context_len, partition_tokens) ? 1 : 0;
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len,
                                int32_t partition_tokens) {
    if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
        max_context_len < 0 || partition_tokens < kRequestBalanced)
        return 0;
    if (decode_uses_balanced(num_seqs, num_kv_heads, max_context_len, partition_tokens))
        return plan_balanced(num_seqs, num_q_heads, num_kv_heads, head_dim, balanced_workgroups())
            .total();
    Split sp = plan_split(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                          partition_tokens);
    return sp.total();
}

}  // extern "C"

// GQA decode, optionally with the fused cache write of each sequence's new
// token (new_key / new_value / slot_mapping all null: no write); shared by
// the GQA decode entry points, including the one in noalloc.hip.
// layout: 0 shuffled bf16, 1 standard bf16, 2 shuffled FP8 (k_scale,
// v_scale used only there)
int32_t pa::decode_impl(int layout, float k_scale, float v_scale, void *out, float *lse,
                        const void *query, const void *new_key, const void *new_value,
                        const int64_t *slot_mapping, const void *k_cache, const void *v_cache,
                        const int32_t *block_table, int32_t max_blocks_per_seq,
                        const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int64_t num_blocks, float scale,
                        int32_t partition_tokens, void *workspace, size_t workspace_bytes,
                        void *stream, bool dry_run) {
    if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || max_blocks_per_seq < 1 ||
        num_blocks < 1 || max_context_len < 0 || partition_tokens < kRequestBalanced ||
        !isfinite(scale))
        return PA_ERR_INVALID_ARG;
    if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    if (!out || !query || !k_cache || !v_cache || !block_table || !context_lens)
        return PA_ERR_INVALID_ARG;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(query, 4) ||
        !aligned(out, 4) || !aligned(lse, 4))
        return PA_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
    if (num_q_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
    if (max_context_len > kMaxContext || num_seqs > 65535 || num_kv_heads > 65535)
        return PA_ERR_UNSUPPORTED;
    const bool balanced =
        decode_uses_balanced(num_seqs, num_kv_heads, max_context_len, partition_tokens);
    const int32_t cus = balanced ? device_cus() : 0;
    const int32_t NW = kBalancedMaxPerCU * cus;
    Split sp = balanced ? plan_balanced(num_seqs, num_q_heads, num_kv_heads, head_dim, NW)
                        : plan_split(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                     max_context_len, partition_tokens);
    if ((balanced || sp.parts > 1) && !counters_fit(num_seqs, num_kv_heads))
        return PA_ERR_UNSUPPORTED;
    if (sp.total() > 0) {
        if ((!workspace && !dry_run) || workspace_bytes < sp.total())
            return PA_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned(workspace, 256)) return PA_ERR_INVALID_ARG;
    }
    if (num_seqs == 0 || dry_run) return PA_OK;
    DecodeParams p;
    p.out = out;
    p.lse = lse;
    p.query = query;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_table = block_table;
    p.max_blocks = max_blocks_per_seq;
    p.context_lens = context_lens;
    p.max_ctx = max_context_len;
    p.S = num_seqs;
    p.Hq = num_q_heads;
    p.Hkv = num_kv_heads;
    p.D = head_dim;
    p.B = block_size;
    p.num_blocks = num_blocks;
    p.scale = scale;
    p.partition = sp.P;
    p.max_parts = sp.parts;
    p.balanced_workgroups = NW;
    p.num_cus = cus;
    char *ws = (char *)workspace;
    const bool split = balanced || sp.parts > 1;
    p.counters = split ? (int *)ws : nullptr;
    p.part_out = split ? (float *)(ws + sp.counter_bytes) : nullptr;
    p.part_lse = split ? (float *)(ws + sp.counter_bytes + sp.out_bytes) : nullptr;
    p.new_key = new_key;
    p.new_value = new_value;
    p.slot_mapping = slot_mapping;
    p.layout = layout;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.k_inv = 1.0f / k_scale;
    p.v_inv = 1.0f / v_scale;
    return from_hip(launch_paged_decode(p, (hipStream_t)stream));
}

extern "C" {

pa_status pa_paged_decode_attn(void *out, float *lse, const void *query, const void *k_cache,
                               const void *v_cache, const int32_t *block_table,
                               int32_t max_blocks_per_seq, const int32_t *context_lens,
                               int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, float scale, int32_t partition_tokens,
                               void *workspace, size_t workspace_bytes, void *stream) {
    return decode_impl(0, 1.f, 1.f, out, lse, query, nullptr, nullptr, nullptr, k_cache, v_cache,
                       block_table,
                       max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, scale, partition_tokens,
                       workspace, workspace_bytes, stream);
}

pa_status pa_paged_decode_attn_write(void *out, float *lse, const void *query,
                                     const void *new_key, const void *new_value,
                                     const int64_t *slot_mapping, void *k_cache, void *v_cache,
                                     const int32_t *block_table, int32_t max_blocks_per_seq,
                                     const int32_t *context_lens, int32_t max_context_len,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                     float scale, int32_t partition_tokens, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    if (!new_key || !new_value || !slot_mapping) return PA_ERR_INVALID_ARG;
    if (!aligned(new_key, 16) || !aligned(new_value, 16) || !aligned(slot_mapping, 8))
        return PA_ERR_INVALID_ARG;
    return decode_impl(0, 1.f, 1.f, out, lse, query, new_key, new_value, slot_mapping, k_cache,
                       v_cache, block_table, max_blocks_per_seq, context_lens, max_context_len,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       scale, partition_tokens, workspace, workspace_bytes, stream);
}

pa_status pa_paged_decode_attn_layout(int32_t layout, void *out, float *lse, const void *query,
                                      const void *new_key, const void *new_value,
                                      const int64_t *slot_mapping, void *k_cache, void *v_cache,
                                      const int32_t *block_table, int32_t max_blocks_per_seq,
                                      const int32_t *context_lens, int32_t max_context_len,
                                      int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int64_t num_blocks, float scale, int32_t partition_tokens,
                                      void *workspace, size_t workspace_bytes, void *stream) {
    if (layout != PA_LAYOUT_SHUFFLED_KV && layout != PA_LAYOUT_STANDARD_KV)
        return PA_ERR_INVALID_ARG;
    const int given = (new_key != nullptr) + (new_value != nullptr) + (slot_mapping != nullptr);
    if (given != 0 && given != 3) return PA_ERR_INVALID_ARG;
    if (given == 3 && (!aligned(new_key, 16) || !aligned(new_value, 16) ||
                       !aligned(slot_mapping, 8)))
        return PA_ERR_INVALID_ARG;
    return decode_impl(layout == PA_LAYOUT_STANDARD_KV ? 1 : 0, 1.f, 1.f, out, lse, query,
                       new_key, new_value,
                       slot_mapping, k_cache, v_cache, block_table, max_blocks_per_seq,
                       context_lens, max_context_len, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, num_blocks, scale, partition_tokens, workspace,
                       workspace_bytes, stream);
}

static bool valid_scale(float s) { return isfinite(s) && s > 0.f && isfinite(1.0f / s); }

pa_status pa_paged_decode_attn_fp8(void *out, float *lse, const void *query, const void *new_key,
                                   const void *new_value, const int64_t *slot_mapping,
                                   void *k_cache, void *v_cache, const int32_t *block_table,
                                   int32_t max_blocks_per_seq, const int32_t *context_lens,
                                   int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int64_t num_blocks, float scale, float k_scale, float v_scale,
                                   int32_t partition_tokens, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    if (!valid_scale(k_scale) || !valid_scale(v_scale)) return PA_ERR_INVALID_ARG;
    const int given = (new_key != nullptr) + (new_value != nullptr) + (slot_mapping != nullptr);
    if (given != 0 && given != 3) return PA_ERR_INVALID_ARG;
    if (given == 3 && (!aligned(new_key, 16) || !aligned(new_value, 16) ||
                       !aligned(slot_mapping, 8)))
        return PA_ERR_INVALID_ARG;
    return decode_impl(2, k_scale, v_scale, out, lse, query, new_key, new_value, slot_mapping,
                       k_cache, v_cache, block_table, max_blocks_per_seq, context_lens,
                       max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, scale, partition_tokens, workspace, workspace_bytes, stream);
}

pa_status pa_reshape_and_cache_fp8(const void *key, const void *value, void *k_cache,
                                   void *v_cache, const int64_t *slot_mapping, int64_t num_tokens,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int64_t num_blocks, float k_scale, float v_scale,
                                   void *stream) {
    if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1)
        return PA_ERR_INVALID_ARG;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
    if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
        return PA_ERR_INVALID_ARG;
    if (!valid_scale(k_scale) || !valid_scale(v_scale)) return PA_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PA_OK;
    return from_hip(launch_cache_write_fp8(key, value, k_cache, v_cache, slot_mapping, num_tokens,
                                           num_kv_heads, head_dim, block_size, num_blocks,
                                           1.0f / k_scale, 1.0f / v_scale, (hipStream_t)stream));
}

size_t pa_mla_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t v_dim,
                             int32_t max_context_len, int32_t partition_tokens) {
    if (num_seqs < 0 || num_q_heads < 1 || v_dim < 1 || max_context_len < 0 ||
        partition_tokens < kRequestBalanced)
        return 0;
    if (decode_uses_balanced(num_seqs, 1, max_context_len, partition_tokens))
        return plan_balanced(num_seqs, num_q_heads, 1, v_dim, balanced_workgroups()).total();
    Split sp = plan_split(num_seqs, num_q_heads, 1, v_dim, max_context_len, partition_tokens);
    return sp.total();
}

// MLA decode, optionally with the fused cache write of each sequence's new
// latent (new_latent / slot_mapping null: no write).
static pa_status mla_impl(bool fp8, bool mfma, float kv_scale, void *out, float *lse,
                          const void *query,
                          const void *new_latent,
                          const int64_t *slot_mapping, const void *kv_cache,
                          const int32_t *block_table, int32_t max_blocks_per_seq,
                          const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                          int32_t num_q_heads, int32_t latent_dim, int32_t v_dim,
                          int32_t block_size, int64_t num_blocks, float scale,
                          int32_t partition_tokens, void *workspace, size_t workspace_bytes,
                          void *stream) {
    if (num_seqs < 0 || num_q_heads < 1 || block_size < 1 || num_blocks < 1 ||
        max_blocks_per_seq < 1 || max_context_len < 0 || partition_tokens < kRequestBalanced ||
        !isfinite(scale))
        return PA_ERR_INVALID_ARG;
    if (!out || !query || !kv_cache || !block_table || !context_lens) return PA_ERR_INVALID_ARG;
    if (!aligned(out, 16) || !aligned(query, 4) || !aligned(kv_cache, 16) || !aligned(lse, 4) ||
        !aligned(block_table, 4) || !aligned(context_lens, 4))
        return PA_ERR_INVALID_ARG;
    if (latent_dim != 576 || v_dim != 512 || num_q_heads > 16 || max_context_len > kMaxContext ||
        num_seqs > 65535 || num_blocks * (int64_t)block_size > 0x7fffffff)
        return PA_ERR_UNSUPPORTED;
    const bool balanced = decode_uses_balanced(num_seqs, 1, max_context_len, partition_tokens);
    const int32_t cus = balanced ? device_cus() : 0;
    const int32_t NW = kBalancedMaxPerCU * cus;
    Split sp = balanced ? plan_balanced(num_seqs, num_q_heads, 1, v_dim, NW)
                        : plan_split(num_seqs, num_q_heads, 1, v_dim, max_context_len,
                                     partition_tokens);
    if ((balanced || sp.parts > 1) && !counters_fit(num_seqs, 1)) return PA_ERR_UNSUPPORTED;
    if (sp.total() > 0) {
        if (!workspace || workspace_bytes < sp.total()) return PA_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned(workspace, 256)) return PA_ERR_INVALID_ARG;
    }
    if (num_seqs == 0) return PA_OK;
    MLAParams p;
    p.out = out;
    p.lse = lse;
    p.query = query;
    p.kv_cache = kv_cache;
    p.block_table = block_table;
    p.max_blocks = max_blocks_per_seq;
    p.context_lens = context_lens;
    p.S = num_seqs;
    p.Hq = num_q_heads;
    p.Dl = latent_dim;
    p.Dv = v_dim;
    p.B = block_size;
    p.num_blocks = num_blocks;
    p.scale = scale;
    p.max_ctx = max_context_len;
    p.partition = sp.P;
    p.max_parts = sp.parts;
    p.balanced_workgroups = NW;
    p.num_cus = cus;
    char *ws = (char *)workspace;
    const bool split = balanced || sp.parts > 1;
    p.counters = split ? (int *)ws : nullptr;
    p.part_out = split ? (float *)(ws + sp.counter_bytes) : nullptr;
    p.part_lse = split ? (float *)(ws + sp.counter_bytes + sp.out_bytes) : nullptr;
    p.new_latent = new_latent;
    p.slot_mapping = slot_mapping;
    p.fp8 = fp8 ? 1 : 0;
    p.kv_scale = kv_scale;
    p.kv_inv = 1.0f / kv_scale;
    p.mfma = mfma ? 1 : 0;
    return from_hip(launch_mla_decode(p, (hipStream_t)stream));
}

pa_status pa_mla_decode_attn(void *out, float *lse, const void *query, const void *kv_cache,
                             const int32_t *block_table, int32_t max_blocks_per_seq,
                             const int32_t *context_lens, int32_t max_context_len,
                             int32_t num_seqs, int32_t num_q_heads, int32_t latent_dim,
                             int32_t v_dim, int32_t block_size, int64_t num_blocks, float scale,
                             int32_t partition_tokens, void *workspace, size_t workspace_bytes,
                             void *stream) {
    return mla_impl(false, false, 1.f, out, lse, query, nullptr, nullptr, kv_cache, block_table,
                    max_blocks_per_seq,
                    context_lens, max_context_len, num_seqs, num_q_heads, latent_dim, v_dim,
                    block_size, num_blocks, scale, partition_tokens, workspace, workspace_bytes,
                    stream);
}

pa_status pa_mla_decode_attn_write(void *out, float *lse, const void *query,
                                   const void *new_latent, const int64_t *slot_mapping,
                                   void *kv_cache, const int32_t *block_table,
                                   int32_t max_blocks_per_seq, const int32_t *context_lens,
                                   int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t latent_dim, int32_t v_dim, int32_t block_size,
                                   int64_t num_blocks, float scale, int32_t partition_tokens,
                                   void *workspace, size_t workspace_bytes, void *stream) {
    if (!new_latent || !slot_mapping) return PA_ERR_INVALID_ARG;
    if (!aligned(new_latent, 16) || !aligned(slot_mapping, 8)) return PA_ERR_INVALID_ARG;
    return mla_impl(false, false, 1.f, out, lse, query, new_latent, slot_mapping, kv_cache, block_table,
                    max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                    latent_dim, v_dim, block_size, num_blocks, scale, partition_tokens, workspace,
                    workspace_bytes, stream);
}

pa_status pa_mla_decode_attn_mfma(void *out, float *lse, const void *query,
                                  const void *new_latent, const int64_t *slot_mapping,
                                  void *kv_cache, const int32_t *block_table,
                                  int32_t max_blocks_per_seq, const int32_t *context_lens,
                                  int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t latent_dim, int32_t v_dim, int32_t block_size,
                                  int64_t num_blocks, float scale, int32_t partition_tokens,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    const int given = (new_latent != nullptr) + (slot_mapping != nullptr);
    if (given == 1) return PA_ERR_INVALID_ARG;
    if (given == 2 && (!aligned(new_latent, 16) || !aligned(slot_mapping, 8)))
        return PA_ERR_INVALID_ARG;
    return mla_impl(false, true, 1.f, out, lse, query, new_latent, slot_mapping, kv_cache,
                    block_table, max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                    num_q_heads, latent_dim, v_dim, block_size, num_blocks, scale,
                    partition_tokens, workspace, workspace_bytes, stream);
}

pa_status pa_mla_decode_attn_fp8(void *out, float *lse, const void *query, const void *new_latent,
                                 const int64_t *slot_mapping, void *kv_cache,
                                 const int32_t *block_table, int32_t max_blocks_per_seq,
                                 const int32_t *context_lens, int32_t max_context_len,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t latent_dim,
                                 int32_t v_dim, int32_t block_size, int64_t num_blocks,
                                 float scale, float kv_scale, int32_t partition_tokens,
                                 void *workspace, size_t workspace_bytes, void *stream) {
    if (!valid_scale(kv_scale)) return PA_ERR_INVALID_ARG;
    const int given = (new_latent != nullptr) + (slot_mapping != nullptr);
    if (given == 1) return PA_ERR_INVALID_ARG;
    if (given == 2 && (!aligned(new_latent, 16) || !aligned(slot_mapping, 8)))
        return PA_ERR_INVALID_ARG;
    return mla_impl(true, false, kv_scale, out, lse, query, new_latent, slot_mapping, kv_cache,
                    block_table, max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                    num_q_heads, latent_dim, v_dim, block_size, num_blocks, scale,
                    partition_tokens, workspace, workspace_bytes, stream);
}

pa_status pa_mla_decode_attn_fp8_mfma(void *out, float *lse, const void *query,
                                      const void *new_latent, const int64_t *slot_mapping,
                                      void *kv_cache, const int32_t *block_table,
                                      int32_t max_blocks_per_seq, const int32_t *context_lens,
                                      int32_t max_context_len, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t latent_dim, int32_t v_dim,
                                      int32_t block_size, int64_t num_blocks, float scale,
                                      float kv_scale, int32_t partition_tokens, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    if (!valid_scale(kv_scale)) return PA_ERR_INVALID_ARG;
    const int given = (new_latent != nullptr) + (slot_mapping != nullptr);
    if (given == 1) return PA_ERR_INVALID_ARG;
    if (given == 2 && (!aligned(new_latent, 16) || !aligned(slot_mapping, 8)))
        return PA_ERR_INVALID_ARG;
    return mla_impl(true, true, kv_scale, out, lse, query, new_latent, slot_mapping, kv_cache,
                    block_table, max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                    num_q_heads, latent_dim, v_dim, block_size, num_blocks, scale,
                    partition_tokens, workspace, workspace_bytes, stream);
}

pa_status pa_reshape_and_cache_mla_fp8(const void *latent, void *kv_cache,
                                       const int64_t *slot_mapping, int64_t num_tokens,
                                       int32_t latent_dim, int32_t block_size, int64_t num_blocks,
                                       float kv_scale, void *stream) {
    if (num_tokens < 0 || latent_dim < 1 || block_size < 1 || num_blocks < 1)
        return PA_ERR_INVALID_ARG;
    if (!latent || !kv_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
    if (!aligned(latent, 16) || !aligned(kv_cache, 16) || !aligned(slot_mapping, 8))
        return PA_ERR_INVALID_ARG;
    if (!valid_scale(kv_scale)) return PA_ERR_INVALID_ARG;
    if (latent_dim % 16 != 0) return PA_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PA_OK;
    return from_hip(launch_cache_write_latent_fp8(latent, kv_cache, slot_mapping, num_tokens,
                                                  latent_dim, block_size, num_blocks,
                                                  1.0f / kv_scale, (hipStream_t)stream));
}

pa_status pa_merge_attn_states(void *out, float *out_lse, int32_t out_dtype,
                               const void *prefix_out, const float *prefix_lse,
                               const void *suffix_out, const float *suffix_lse, int32_t in_dtype,
                               int64_t num_tokens, int32_t num_heads, int32_t head_dim,
                               void *stream) {
    if (num_tokens < 0 || num_heads < 1 || head_dim < 1) return PA_ERR_INVALID_ARG;
    if ((in_dtype != PA_BF16 && in_dtype != PA_F32) || (out_dtype != PA_BF16 && out_dtype != PA_F32))
        return PA_ERR_INVALID_ARG;
    if (!out || !prefix_out || !prefix_lse || !suffix_out || !suffix_lse) return PA_ERR_INVALID_ARG;
    if (!aligned(out, 16) || !aligned(prefix_out, 16) || !aligned(suffix_out, 16) ||
        !aligned(prefix_lse, 4) || !aligned(suffix_lse, 4) || !aligned(out_lse, 4))
        return PA_ERR_INVALID_ARG;
    if (head_dim % 8 != 0 || head_dim > 1024) return PA_ERR_UNSUPPORTED;
    // A row's LSEs are read by all of its threads, which may sit in several
    // workgroups, while one of them writes out_lse: out_lse must not overlap
    // an input LSE.  out may be an input itself (same address and dtype:
    // each thread reads its vector before writing it), but no other overlap.
    const size_t rows = (size_t)num_tokens * num_heads;
    const size_t in_bytes = rows * head_dim * (in_dtype == PA_F32 ? 4 : 2);
    const size_t out_bytes = rows * head_dim * (out_dtype == PA_F32 ? 4 : 2);
    if (out_lse && (overlaps(out_lse, rows * 4, prefix_lse, rows * 4) ||
                    overlaps(out_lse, rows * 4, suffix_lse, rows * 4) ||
                    overlaps(out_lse, rows * 4, prefix_out, in_bytes) ||
                    overlaps(out_lse, rows * 4, suffix_out, in_bytes) ||
                    overlaps(out_lse, rows * 4, out, out_bytes)))
        return PA_ERR_INVALID_ARG;
    for (const void *in : {prefix_out, suffix_out}) {
        const bool same = in == out && in_dtype == out_dtype;
        if (!same && overlaps(out, out_bytes, in, in_bytes)) return PA_ERR_INVALID_ARG;
    }
    if (overlaps(out, out_bytes, prefix_lse, rows * 4) ||
        overlaps(out, out_bytes, suffix_lse, rows * 4))
        return PA_ERR_INVALID_ARG;
    if (num_tokens == 0) return PA_OK;
    return from_hip(launch_merge_pair(out, out_lse, out_dtype == PA_F32, prefix_out, prefix_lse,
                                      suffix_out, suffix_lse, in_dtype == PA_F32,
                                      num_tokens * num_heads, head_dim, (hipStream_t)stream));
}

int32_t pa_extend_chunk_tokens(int32_t num_seqs, int32_t block_size, int32_t chunk_budget_tokens) {
    if (num_seqs < 1 || block_size < 1 || chunk_budget_tokens < 1) return block_size > 0 ? block_size : 1;
    int32_t c = chunk_budget_tokens / num_seqs / block_size * block_size;
    return c < block_size ? block_size : c;
}

static pa_status gather_impl(bool fp8, float k_scale, float v_scale, void *k_out, void *v_out,
                             const void *k_cache, const void *v_cache,
                             const int32_t *block_table, int32_t max_blocks_per_seq,
                             const int32_t *context_lens, int32_t num_seqs, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks,
                             int32_t iteration, int32_t chunk_tokens, void *stream) {
    if (num_seqs < 0 || num_kv_heads < 1 || block_size < 1 || num_blocks < 1 ||
        max_blocks_per_seq < 1 || iteration < 0 || chunk_tokens < 1)
        return PA_ERR_INVALID_ARG;
    if (!k_out || !v_out || !k_cache || !v_cache || !block_table || !context_lens)
        return PA_ERR_INVALID_ARG;
    if (!aligned(k_out, 16) || !aligned(v_out, 16) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 16))
        return PA_ERR_INVALID_ARG;
    if (head_dim != 128 || block_size % (fp8 ? 16 : 8) != 0 || chunk_tokens % block_size != 0 ||
        num_seqs > 65535 || (int64_t)iteration * chunk_tokens > kMaxContext)
        return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    GatherParams gp;
    gp.k_cache = k_cache;
    gp.v_cache = v_cache;
    gp.block_table = block_table;
    gp.max_blocks = max_blocks_per_seq;
    gp.context_lens = context_lens;
    gp.S = num_seqs;
    gp.Hkv = num_kv_heads;
    gp.B = block_size;
    gp.num_blocks = num_blocks;
    gp.iteration = iteration;
    gp.chunk = chunk_tokens;
    gp.k_out = k_out;
    gp.v_out = v_out;
    gp.fp8 = fp8 ? 1 : 0;
    gp.k_scale = k_scale;
    gp.v_scale = v_scale;
    return from_hip(launch_gather_chunk(gp, chunk_tokens, (hipStream_t)stream));
}

pa_status pa_gather_cache_chunk(void *k_out, void *v_out, const void *k_cache,
                                const void *v_cache, const int32_t *block_table,
                                int32_t max_blocks_per_seq, const int32_t *context_lens,
                                int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int64_t num_blocks, int32_t iteration,
                                int32_t chunk_tokens, void *stream) {
    return gather_impl(false, 1.f, 1.f, k_out, v_out, k_cache, v_cache, block_table,
                       max_blocks_per_seq, context_lens, num_seqs, num_kv_heads, head_dim,
                       block_size, num_blocks, iteration, chunk_tokens, stream);
}

pa_status pa_gather_cache_chunk_fp8(void *k_out, void *v_out, const void *k_cache,
                                    const void *v_cache, const int32_t *block_table,
                                    int32_t max_blocks_per_seq, const int32_t *context_lens,
                                    int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int64_t num_blocks, int32_t iteration,
                                    int32_t chunk_tokens, float k_scale, float v_scale,
                                    void *stream) {
    if (!isfinite(k_scale) || !isfinite(v_scale)) return PA_ERR_INVALID_ARG;
    return gather_impl(true, k_scale, v_scale, k_out, v_out, k_cache, v_cache, block_table,
                       max_blocks_per_seq, context_lens, num_seqs, num_kv_heads, head_dim,
                       block_size, num_blocks, iteration, chunk_tokens, stream);
}

// Extend workspace: the counter region (left untouched: extend keeps no
// counters, but a workspace shared with decode calls keeps its counters
// there), the group prefix [S + 1], the new tokens' V in 8-token groups, and
// fp32 partials (output, LSE) for up to kExtendMaxPieces context pieces of
// every (new token, q head).
struct ExtendWorkspace {
    size_t prefix, vsh, part_out, part_lse;
    int32_t new_groups;
    size_t total() const { return kCounterBytes + prefix + vsh + part_out + part_lse; }
};

static ExtendWorkspace extend_workspace(int32_t S, int32_t Tn, int32_t Hq, int32_t Hkv) {
    ExtendWorkspace w;
    w.new_groups = (Tn + 7) / 8 + S + 1;
    w.prefix = align256((size_t)(S + 1) * sizeof(int32_t));
    w.vsh = align256((size_t)Hkv * w.new_groups * 128 * 8 * 2);
    w.part_out = align256((size_t)Tn * Hq * kExtendMaxPieces * 128 * sizeof(float));
    w.part_lse = align256((size_t)Tn * Hq * kExtendMaxPieces * sizeof(float));
    return w;
}

size_t pa_extend_workspace_size(int32_t num_seqs, int32_t total_new_tokens, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t chunk_budget_tokens) {
    if (num_seqs < 1 || total_new_tokens < 0 || num_q_heads < 1 || num_kv_heads < 1 ||
        head_dim < 1 || block_size < 1 || chunk_budget_tokens < 1)
        return 0;
    return extend_workspace(num_seqs, total_new_tokens, num_q_heads, num_kv_heads).total();
}

// Pieces are sized so that the longest unit of work is about an eighth of
// one workgroup slot's share of the whole call (2 workgroups per CU).
constexpr int64_t kExtendPieceFraction = 8;

pa_status pa_chunked_extend_attn(void *out, float *lse, const void *query, const void *k_new,
                                 const void *v_new, const int32_t *query_start_loc,
                                 const int32_t *query_start_loc_host, const void *k_cache,
                                 const void *v_cache, const int32_t *block_table,
                                 int32_t max_blocks_per_seq, const int32_t *context_lens,
                                 const int32_t *context_lens_host, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks, float scale,
                                 int32_t chunk_budget_tokens, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    if (num_seqs < 1 || num_q_heads < 1 || num_kv_heads < 1 || block_size < 1 ||
        num_blocks < 1 || max_blocks_per_seq < 1 || chunk_budget_tokens < 1 || !isfinite(scale))
        return PA_ERR_INVALID_ARG;
    if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    if (num_q_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
    if (!out || !query || !k_new || !v_new || !query_start_loc || !query_start_loc_host ||
        !k_cache || !v_cache || !block_table || !context_lens || !context_lens_host)
        return PA_ERR_INVALID_ARG;
    if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) ||
        !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(lse, 4))
        return PA_ERR_INVALID_ARG;
    if (head_dim != 128 || (block_size != 16 && block_size != 32) || num_seqs > 65535 ||
        num_q_heads > 65535)
        return PA_ERR_UNSUPPORTED;
    // plan on the host copies: lengths, the work per workgroup slot, pieces
    if (query_start_loc_host[0] != 0) return PA_ERR_INVALID_ARG;
    int32_t max_new = 0;
    int64_t work = 0;  // 64-key tiles over all (request, q head, 128-row block)
    for (int32_t r = 0; r < num_seqs; r++) {
        const int32_t n = query_start_loc_host[r + 1] - query_start_loc_host[r];
        const int32_t c = context_lens_host[r];
        if (n < 0 || c < 0 || (int64_t)c > (int64_t)max_blocks_per_seq * block_size)
            return PA_ERR_INVALID_ARG;
        if (c > kMaxContext) return PA_ERR_UNSUPPORTED;
        max_new = n > max_new ? n : max_new;
        work += cdiv(n, 128) * num_q_heads * cdiv((int64_t)c + n, 64);
    }
    const int32_t total_new = query_start_loc_host[num_seqs];
    const ExtendWorkspace w = extend_workspace(num_seqs, total_new, num_q_heads, num_kv_heads);
    if (!workspace || workspace_bytes < w.total()) return PA_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(workspace, 256)) return PA_ERR_INVALID_ARG;
    if (total_new == 0) return PA_OK;

    int32_t c = pa_extend_chunk_tokens(num_seqs, block_size, chunk_budget_tokens);
    if (c > kMaxContext) c = kMaxContext / block_size * block_size;
    const int64_t slots = 2 * (int64_t)device_cus();
    int64_t target = cdiv(cdiv(work, slots) * 64, kExtendPieceFraction);
    target = cdiv(target < c ? c : target, c) * c;
    if (target > kMaxContext) target = kMaxContext;
    ExtendParams p;
    p.chunk = c;
    p.piece_target = (int32_t)target;
    p.max_pieces = kExtendMaxPieces;
    const int64_t table_tokens = (int64_t)max_blocks_per_seq * block_size;
    p.max_ctx = table_tokens < kMaxContext ? (int32_t)table_tokens : kMaxContext;
    int64_t groups = 0;
    for (int32_t r = 0; r < num_seqs; r++) {
        int32_t len;
        groups += (int64_t)extend_pieces(context_lens_host[r], p.piece_target, c, p.max_pieces,
                                         &len) * num_kv_heads;
    }
    char *ws = (char *)workspace + kCounterBytes;
    p.q = query;
    p.k_new = k_new;
    p.v_new = v_new;
    p.group_prefix = (int32_t *)ws;
    p.v_new_sh = ws + w.prefix;
    p.new_groups = w.new_groups;
    p.part_out = (float *)(ws + w.prefix + w.vsh);
    p.part_lse = (float *)(ws + w.prefix + w.vsh + w.part_out);
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_table = block_table;
    p.max_blocks = max_blocks_per_seq;
    p.num_blocks = num_blocks;
    p.q_start = query_start_loc;
    p.context_lens = context_lens;
    p.S = num_seqs;
    p.Hq = num_q_heads;
    p.Hkv = num_kv_heads;
    p.B = block_size;
    p.Tn = total_new;
    p.q_blocks = (int32_t)cdiv(max_new, 128);
    p.num_groups = (int32_t)groups;
    p.scale = scale;
    p.out = out;
    p.lse = lse;
    return from_hip(launch_extend(p, max_new, (hipStream_t)stream));
}

}  // extern "C"
