// Measurement aids, not steps of the attention method.  Plain streaming read
// of a device buffer: the yardstick for what the memory system delivers at a
// given transfer size, against which the decode kernels' achieved bandwidth
// is read; and a read of the blocks a decode reads, through the block table,
// with no arithmetic.  The streaming read's workgroups walk the buffer
// grid-stride in 16-byte vectors (4 in flight per lane per iteration); both
// fold what they read into one xor word.  With `verify` set every workgroup
// stores its word; otherwise there is no reduction and a lane stores its
// own word only if it is all ones, which keeps every load live without
// adding a reduction or a store drain to the timed read.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "pagedattn.h"

namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ src,
                                                          size_t n16, uint32_t *__restrict__ sink,
                                                          int verify) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
               d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (!verify) {  // timing: no reduction, no stores (unless a lane's word is all ones)
        if (acc == ~0u) sink[blockIdx.x] = acc;
        return;
    }
    // xor over the wave (lane shuffles), then over the 4 waves through LDS
    for (int w = 32; w > 0; w >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, w, 64);
    __shared__ uint32_t part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Block-table gather read: wave w of workgroup (b4, unit) reads the K and V
// units of block 4 b4 + w of unit = (sequence, kv head), if the sequence's
// context reaches it: 16-byte vectors, 4 per lane in flight, folded into
// one xor word as above.  The grid is block-major (b4 outer), like the
// decode's partition-major grid.
__global__ __launch_bounds__(256) void gather_read_kernel(const uint4 *__restrict__ kc,
                                                          const uint4 *__restrict__ vc,
                                                          const int32_t *__restrict__ block_table,
                                                          const int32_t *__restrict__ context_lens,
                                                          int32_t units, int32_t num_kv_heads,
                                                          int32_t max_blocks, int32_t block_size,
                                                          int64_t num_blocks, int32_t unit16,
                                                          uint32_t *__restrict__ sink, int verify) {
    const int unit = blockIdx.x % units, b4 = blockIdx.x / units;
    const int s = unit / num_kv_heads, g = unit - s * num_kv_heads;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int b = 4 * b4 + wave;
    int ctx = context_lens[s];
    ctx = ctx < 0 ? 0 : (ctx > max_blocks * block_size ? max_blocks * block_size : ctx);
    uint32_t acc = 0;
    if (b * block_size < ctx) {
        const int blk = block_table[(size_t)s * max_blocks + b];
        if (blk >= 0 && blk < num_blocks) {
            const size_t base = ((size_t)blk * num_kv_heads + g) * unit16;
            const uint4 *k = kc + base, *v = vc + base;
            for (int i = lane; i < unit16; i += 256) {
                uint4 x[8];
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const int j = i + 64 * u < unit16 ? i + 64 * u : i;  // in range
                    x[u] = k[j];
                    x[4 + u] = v[j];
                }
#pragma unroll
                for (int u = 0; u < 4; u++)
                    if (i + 64 * u < unit16)
                        acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w ^ x[4 + u].x ^ x[4 + u].y ^
                               x[4 + u].z ^ x[4 + u].w;
            }
        }
    }
    if (!verify) {
        if (acc == ~0u) sink[blockIdx.x] = acc;
        return;
    }
    for (int w = 32; w > 0; w >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, w, 64);
    __shared__ uint32_t part[4];
    if (lane == 0) part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

extern "C" pa_status pa_gather_read(const void *k_cache, const void *v_cache,
                                    const int32_t *block_table, const int32_t *context_lens,
                                    int32_t num_seqs, int32_t num_kv_heads,
                                    int32_t max_blocks_per_seq, int32_t block_size,
                                    int64_t num_blocks, int32_t unit_bytes, uint32_t *sink,
                                    int32_t verify, void *stream) {
    if (!k_cache || !v_cache || !block_table || !context_lens || !sink || num_seqs < 0 ||
        num_kv_heads < 1 || max_blocks_per_seq < 1 || block_size < 1 || num_blocks < 1 ||
        unit_bytes < 1024 || unit_bytes > 65536 || unit_bytes % 1024 != 0 ||
        ((uintptr_t)k_cache & 15) != 0 || ((uintptr_t)v_cache & 15) != 0 ||
        (int64_t)max_blocks_per_seq * block_size > 0x7fffffff)
        return PA_ERR_INVALID_ARG;
    const int64_t units = (int64_t)num_seqs * num_kv_heads;
    const int64_t grid = units * ((max_blocks_per_seq + 3) / 4);
    if (grid > 0x7fffffff) return PA_ERR_INVALID_ARG;
    if (grid == 0) return PA_OK;
    hipLaunchKernelGGL(gather_read_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint4 *)k_cache, (const uint4 *)v_cache, block_table, context_lens,
                       (int32_t)units, num_kv_heads, max_blocks_per_seq, block_size, num_blocks,
                       unit_bytes / 16, sink, verify);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" pa_status pa_stream_read(const void *src, size_t bytes, uint32_t *sink,
                                    int32_t workgroups, int32_t verify, void *stream) {
    if (!src || !sink || bytes % 16 != 0 || ((uintptr_t)src & 15) != 0 || workgroups < 1 ||
        workgroups > 65536)
        return PA_ERR_INVALID_ARG;
    if (bytes == 0) return PA_OK;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                       (hipStream_t)stream, (const uint4 *)src, bytes / 16, sink, verify);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
