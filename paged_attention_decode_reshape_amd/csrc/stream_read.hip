// Plain streaming read of a device buffer: the yardstick for what the memory
// system delivers at a given transfer size, against which the decode kernels'
// achieved bandwidth is read.  It is a measurement aid, not a step of the
// attention method.  Every workgroup walks the buffer grid-stride in 16-byte
// vectors (4 in flight per lane per iteration) and folds them into one xor
// word.  With `verify` set every workgroup stores its word; otherwise there
// is no reduction and a lane stores its own word only if it is all ones,
// which keeps every load live without adding a reduction or a store drain
// to the timed read.
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

}  // namespace

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
