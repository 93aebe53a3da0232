// Three-path routing of one mixed batch ("ROCm attention backends" blog,
// ROCM_AITER_FA section: requests are sorted into decode, extend and prefill
// paths, each served by its own kernel, after the model runner has reordered
// the batch as [decode : extend : prefill]).
//
// pa_mixed_batch_plan classifies requests on the host and returns the stable
// [decode : extend : prefill] order; pa_mixed_batch_attn takes a batch in that
// order and runs, on one stream: the cache write of every new token, the
// paged decode over the decode slice, and one chunked-extend launch over the
// extend and prefill slices together.  The library's extend kernel is a
// matrix-core tile attention that takes a request with nothing cached as a
// plain causal prefill, and the reorder leaves the two slices adjacent, so
// one launch (one plan, one merge) serves both paths.  A small kernel derives
// the per-slice device arrays (decode lengths including the new token,
// slice-relative query offsets) into the workspace.
#include <stdint.h>

#include <algorithm>
#include <vector>

#include <hip/hip_runtime.h>

#include "pagedattn.h"

namespace {

constexpr int kDecode = 0, kExtend = 1, kPrefill = 2;

// A request with at most one new token is decode (the reorder threshold of
// one); otherwise prefill when nothing is cached yet, else extend.
inline int path_of(int32_t new_tokens, int32_t cached) {
    if (new_tokens <= 1) return kDecode;
    return cached == 0 ? kPrefill : kExtend;
}

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Per-slice device arrays: decode lengths (cached + 1) of requests
// 0 .. nd - 1, and the query offsets of the extend + prefill slice (requests
// nd .. nd + nx) relative to its first request.  Also clears the decode
// call's completion counters (the first n_counters words of its workspace),
// so the routed call asks nothing of the workspace's previous contents.
__global__ void route_prepare_kernel(const int32_t *__restrict__ qsl,
                                     const int32_t *__restrict__ ctx, int nd, int nx,
                                     int32_t *__restrict__ dec_lens, int32_t *__restrict__ qsl_x,
                                     int32_t *__restrict__ counters, int n_counters) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nd) dec_lens[i] = ctx[i] + 1;
    if (i <= nx) qsl_x[i] = qsl[nd + i] - qsl[nd];
    if (i < n_counters) counters[i] = 0;
}

struct Slices {
    int32_t nd = 0, ne = 0, np = 0;  // requests per path
    int32_t td = 0, te = 0, tp = 0;  // new tokens per path
    int32_t max_dec_len = 0;
    bool ordered = true;
};

bool scan(int32_t R, const int32_t *qsl, const int32_t *ctx, Slices &sl) {
    if (qsl[0] != 0) return false;
    int last = kDecode;
    for (int32_t r = 0; r < R; r++) {
        const int32_t n = qsl[r + 1] - qsl[r], c = ctx[r];
        if (n < 1 || c < 0) return false;
        const int k = path_of(n, c);
        if (k < last) sl.ordered = false;
        last = k > last ? k : last;
        if (k == kDecode) {
            sl.nd++;
            sl.td += n;
            if (c + 1 > sl.max_dec_len) sl.max_dec_len = c + 1;
        } else if (k == kExtend) {
            sl.ne++;
            sl.te += n;
        } else {
            sl.np++;
            sl.tp += n;
        }
    }
    return true;
}

// Layout: the decode call's workspace first, so that its counters sit in the
// counter region every library workspace starts with (the region is
// reserved even without decode requests), then the per-slice arrays, then
// the extend call's workspace.
struct RouteWorkspace {
    size_t decode, arrays, extend;
    size_t total() const { return decode + arrays + extend; }
};

RouteWorkspace route_workspace(int32_t R, const Slices &sl, int32_t Hq, int32_t Hkv, int32_t D,
                               int32_t B, int32_t budget) {
    RouteWorkspace w;
    w.arrays = align256((size_t)(2 * R + 1) * sizeof(int32_t));
    w.decode = sl.nd ? align256(pa_decode_workspace_size(sl.nd, Hq, Hkv, D, sl.max_dec_len, 0))
                     : 0;
    if (w.decode < PA_WORKSPACE_COUNTER_BYTES) w.decode = PA_WORKSPACE_COUNTER_BYTES;
    const int32_t nx = sl.ne + sl.np;
    w.extend = nx ? align256(pa_extend_workspace_size(nx, sl.te + sl.tp, Hq, Hkv, D, B, budget))
                  : 0;
    return w;
}

}  // namespace

extern "C" {

pa_status pa_mixed_batch_plan(int32_t num_reqs, const int32_t *query_start_loc_host,
                              const int32_t *context_lens_host, int32_t *order_host,
                              int32_t *counts_host) {
    if (num_reqs < 0 || !query_start_loc_host || !context_lens_host || !order_host ||
        !counts_host)
        return PA_ERR_INVALID_ARG;
    Slices sl;
    if (!scan(num_reqs, query_start_loc_host, context_lens_host, sl)) return PA_ERR_INVALID_ARG;
    int32_t next[3] = {0, sl.nd, sl.nd + sl.ne};
    for (int32_t r = 0; r < num_reqs; r++) {
        const int k = path_of(query_start_loc_host[r + 1] - query_start_loc_host[r],
                              context_lens_host[r]);
        order_host[next[k]++] = r;
    }
    counts_host[0] = sl.nd;
    counts_host[1] = sl.ne;
    counts_host[2] = sl.np;
    return PA_OK;
}

size_t pa_mixed_batch_workspace_size(int32_t num_reqs, const int32_t *query_start_loc_host,
                                     const int32_t *context_lens_host, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int32_t chunk_budget_tokens) {
    if (num_reqs < 1 || !query_start_loc_host || !context_lens_host || num_q_heads < 1 ||
        num_kv_heads < 1 || head_dim < 1 || block_size < 1 || chunk_budget_tokens < 1)
        return 0;
    Slices sl;
    if (!scan(num_reqs, query_start_loc_host, context_lens_host, sl)) return 0;
    return route_workspace(num_reqs, sl, num_q_heads, num_kv_heads, head_dim, block_size,
                           chunk_budget_tokens)
        .total();
}

pa_status pa_mixed_batch_attn(void *out, float *lse, const void *query, const void *key,
                              const void *value, const int64_t *slot_mapping,
                              const int32_t *query_start_loc, const int32_t *query_start_loc_host,
                              const int32_t *context_lens, const int32_t *context_lens_host,
                              void *k_cache, void *v_cache, const int32_t *block_table,
                              int32_t max_blocks_per_seq, int32_t num_reqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, float scale, int32_t chunk_budget_tokens,
                              void *workspace, size_t workspace_bytes, void *stream) {
    if (num_reqs < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
        block_size < 1 || num_blocks < 1 || max_blocks_per_seq < 1 || chunk_budget_tokens < 1)
        return PA_ERR_INVALID_ARG;
    if (!out || !query || !key || !value || !slot_mapping || !query_start_loc ||
        !query_start_loc_host || !context_lens || !context_lens_host || !k_cache || !v_cache ||
        !block_table)
        return PA_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255) != 0) return PA_ERR_INVALID_ARG;
    Slices sl;
    if (!scan(num_reqs, query_start_loc_host, context_lens_host, sl) || !sl.ordered)
        return PA_ERR_INVALID_ARG;  // not in [decode : extend : prefill] order
    if (sl.nd > 0 && head_dim != 128 && head_dim != 64) return PA_ERR_UNSUPPORTED;
    if ((sl.ne > 0 || sl.np > 0) && head_dim != 128) return PA_ERR_UNSUPPORTED;
    const RouteWorkspace w = route_workspace(num_reqs, sl, num_q_heads, num_kv_heads, head_dim,
                                             block_size, chunk_budget_tokens);
    if (!workspace || workspace_bytes < w.total()) return PA_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t st = (hipStream_t)stream;
    const int64_t T = query_start_loc_host[num_reqs];

    // 1. every new token into the cache (the decode and extend paths read it there)
    pa_status s = pa_reshape_and_cache(PA_LAYOUT_SHUFFLED_KV, key, value, k_cache, v_cache,
                                       slot_mapping, T, num_kv_heads, head_dim, block_size,
                                       num_blocks, stream);
    if (s != PA_OK) return s;

    char *ws = (char *)workspace;
    int32_t *dec_lens = (int32_t *)(ws + w.decode);
    int32_t *qsl_x = dec_lens + num_reqs;
    const int32_t nx = sl.ne + sl.np;
    // the decode workspace starts with one completion counter per (sequence, kv head)
    int32_t *dec_ws = (int32_t *)ws;
    const int n_counters = sl.nd * num_kv_heads < (int)(PA_WORKSPACE_COUNTER_BYTES / 4)
                               ? sl.nd * num_kv_heads
                               : (int)(PA_WORKSPACE_COUNTER_BYTES / 4);
    const int n = std::max({sl.nd, nx + 1, n_counters});
    hipLaunchKernelGGL(route_prepare_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       query_start_loc, context_lens, sl.nd, nx, dec_lens, qsl_x, dec_ws,
                       n_counters);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;

    const size_t row_q = (size_t)num_q_heads * head_dim * 2;   // bytes per query / out row
    const size_t row_kv = (size_t)num_kv_heads * head_dim * 2;  // bytes per new K / V row
    char *o = (char *)out;
    const char *q = (const char *)query, *k = (const char *)key, *v = (const char *)value;

    // 2. decode path: requests 0 .. nd - 1, one query row each
    if (sl.nd > 0) {
        s = pa_paged_decode_attn(out, lse, query, k_cache, v_cache, block_table,
                                 max_blocks_per_seq, dec_lens, sl.max_dec_len, sl.nd, num_q_heads,
                                 num_kv_heads, head_dim, block_size, num_blocks, scale, 0,
                                 dec_ws, w.decode, stream);
        if (s != PA_OK) return s;
    }
    // 3. extend and prefill paths: requests nd .. num_reqs - 1 in one launch
    if (nx > 0) {
        const int32_t r0 = sl.nd, row0 = query_start_loc_host[r0];
        std::vector<int32_t> qh(nx + 1);
        for (int32_t i = 0; i <= nx; i++) qh[i] = query_start_loc_host[r0 + i] - row0;
        s = pa_chunked_extend_attn(o + row0 * row_q, lse ? lse + (size_t)row0 * num_q_heads : nullptr,
                                   q + row0 * row_q, k + row0 * row_kv, v + row0 * row_kv, qsl_x,
                                   qh.data(), k_cache, v_cache,
                                   block_table + (size_t)r0 * max_blocks_per_seq,
                                   max_blocks_per_seq, context_lens + r0, context_lens_host + r0,
                                   nx, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                   scale, chunk_budget_tokens, ws + w.decode + w.arrays, w.extend,
                                   stream);
        if (s != PA_OK) return s;
    }
    return PA_OK;
}

}  // extern "C"
