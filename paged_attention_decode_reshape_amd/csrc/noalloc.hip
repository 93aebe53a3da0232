// pa_paged_decode_attn_write_noalloc: the fused decode step of
// pa_paged_decode_attn_write for callers that cannot allocate device memory,
// with the workspace in a fixed per-device array of this library.
//
// `scratch` is a file-scope device array; in host code its name is only a
// stand-in, so the host takes the array's device address once per device
// with hipGetSymbolAddress and passes that pointer to the kernels, like a
// workspace.  The array starts with the same counter region every
// workspace starts with (split calls leave it zero); the first call on a
// device clears that region on the caller's stream before its own work.
// Every call on a device shares the array: calls that overlap in time on
// one device race.
#include <mutex>

#include <hip/hip_runtime.h>

#include "launch.h"
#include "pagedattn.h"

namespace {

constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0 && kScratchBytes > PA_WORKSPACE_COUNTER_BYTES,
              "the scratch array holds the counter region and partials");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    void *ptr = nullptr;    // device address of `scratch` on this device
    bool cleared = false;   // counter region cleared by a completed (not captured) enqueue
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

__global__ __launch_bounds__(256) void clear_counters_kernel(uint4 *p, int n16) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The scratch address on the current device; on the first call there, also
// enqueues the counter-region clear on `stream`.  A clear recorded into a
// captured graph runs only when the graph does, so it does not count as done.
pa_status device_scratch(hipStream_t stream, void **ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceScratch &d = g_dev[dev];
    if (!d.ptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PA_ERR_HIP;
        d.ptr = p;
    }
    if (!d.cleared) {
        const int n16 = (int)(PA_WORKSPACE_COUNTER_BYTES / 16);
        hipLaunchKernelGGL(clear_counters_kernel, dim3(256), dim3(256), 0, stream,
                           (uint4 *)d.ptr, n16);
        if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return PA_ERR_HIP;
        d.cleared = cs == hipStreamCaptureStatusNone;
    }
    *ptr = d.ptr;
    return PA_OK;
}

}  // namespace

extern "C" pa_status pa_paged_decode_attn_write_noalloc(
    void *out, float *lse, const void *query, const void *new_key, const void *new_value,
    const int64_t *slot_mapping, void *k_cache, void *v_cache, const int32_t *block_table,
    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, float scale, int32_t partition_tokens,
    void *stream) {
    if (!new_key || !new_value || !slot_mapping) return PA_ERR_INVALID_ARG;
    if (((uintptr_t)new_key & 15) || ((uintptr_t)new_value & 15) || ((uintptr_t)slot_mapping & 7))
        return PA_ERR_INVALID_ARG;
    // every check first, the array's size included (a call that needs more
    // than it holds gets PA_ERR_WORKSPACE_TOO_SMALL), with nothing enqueued
    pa_status s = pa::decode_impl(0, 1.f, 1.f, out, lse, query, new_key, new_value, slot_mapping,
                                  k_cache, v_cache, block_table, max_blocks_per_seq, context_lens,
                                  max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                  block_size, num_blocks, scale, partition_tokens, nullptr,
                                  kScratchBytes, stream, /*dry_run=*/true);
    if (s != PA_OK || num_seqs == 0) return s;
    void *ws = nullptr;
    s = device_scratch((hipStream_t)stream, &ws);
    if (s != PA_OK) return s;
    return pa::decode_impl(0, 1.f, 1.f, out, lse, query, new_key, new_value, slot_mapping,
                           k_cache, v_cache, block_table, max_blocks_per_seq, context_lens,
                           max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                           block_size, num_blocks, scale, partition_tokens, ws, kScratchBytes,
                           stream);
}
