// Cache write into the preshuffled KV layout and into the MLA latent cache.
//
// "ROCm attention backends" blog, ROCM_AITER_FA section (key innovation 4)
// and the decode-path paragraph: the custom cache-write operator always
// leaves the cache in the shuffled layout
//   k_cache [num_blocks, kv_heads, head_dim / x, block_size, x]
//   v_cache [num_blocks, kv_heads, block_size / x, head_dim, x]
// so decode never converts it.  x = 8 bf16 = one 16-byte vector.
//
// K: one 16-byte source vector (8 consecutive dims of one token) maps to one
// 16-byte destination vector, so each thread moves one vector with a single
// dwordx4 load and store.
// V: a destination vector holds 8 consecutive *tokens* of one dim, so a lone
// token contributes 2 bytes to each of head_dim vectors.  Each thread loads
// 8 dims of one token and issues 8 two-byte stores; neighbouring threads hit
// neighbouring 16-byte vectors, which L2 write-combines.
#include "common.h"
#include "fp8.h"
#include "launch.h"

namespace pa {

// Four dwords as one 16-byte vector value, the type the non-temporal access
// builtins take.
typedef unsigned int dw4_t __attribute__((ext_vector_type(4)));

// Lanes are laid out so that 8 neighbouring lanes take 8 consecutive tokens
// of the same 8 dims (lane = 8 * (chunk % 8) + token % 8): when those tokens
// go to consecutive slots (a prefill or a bulk fill), the 2-byte V values of
// one store instruction sit next to each other in memory and are written
// together, and K's vectors are contiguous too.  (Transposing whole 8-token
// groups through LDS to store full V vectors gained nothing on a bulk fill
// whose sequences start at arbitrary token offsets.)
template <int D>
__global__ __launch_bounds__(256) void cache_write_shuffled_kernel(
    const uint4 *__restrict__ key, const uint4 *__restrict__ value, uint16_t *__restrict__ k_cache,
    uint16_t *__restrict__ v_cache, const int64_t *__restrict__ slot_mapping, int64_t num_tokens,
    int Hkv, int B, int64_t num_blocks) {
    constexpr int C = D / 8;  // 16-byte vectors per head row (a multiple of 8)
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // t = ((group of 8 tokens * Hkv + g) * C / 8 + chunk block) * 64 + 8 * (chunk % 8) + token % 8
    const int lane = (int)(t & 63);
    const int64_t wv = t >> 6;
    const int cq = (int)(wv % (C / 8));
    const int g = (int)((wv / (C / 8)) % Hkv);
    const int64_t i8 = wv / ((int64_t)(C / 8) * Hkv);
    const int64_t i = i8 * 8 + (lane & 7);
    const int c = cq * 8 + (lane >> 3);
    if (i >= num_tokens) return;
    const int64_t idx = (i * Hkv + g) * C + c;  // source vector
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= num_blocks * B) return;
    const int64_t p = slot / B;
    const int o = (int)(slot % B);
    // The source is read once and the K vectors are written whole, so both
    // are non-temporal accesses; V's 2-byte stores keep the default policy,
    // under which L2 combines them into whole vectors (measured on a 93k-token
    // bulk fill: 6.5% faster than the default policy throughout; non-temporal
    // V stores made it 55% slower).
    const dw4_t kv = __builtin_nontemporal_load(reinterpret_cast<const dw4_t *>(key) + idx);
    const dw4_t vv = __builtin_nontemporal_load(reinterpret_cast<const dw4_t *>(value) + idx);
    // K vector (dims c*8 .. c*8+7 of token o) -> k_cache[p][g][c][o][0..8)
    dw4_t *kdst = reinterpret_cast<dw4_t *>(k_cache) + ((p * Hkv + g) * C + c) * B + o;
    __builtin_nontemporal_store(kv, kdst);
    // V: dim d = c*8 + e of token o -> v_cache[p][g][o / 8][d][o % 8]
    uint16_t *vdst = v_cache + (((p * Hkv + g) * (B / 8) + o / 8) * D + c * 8) * 8 + (o % 8);
    const uint32_t w[4] = {vv[0], vv[1], vv[2], vv[3]};
#pragma unroll
    for (int e = 0; e < 8; e++) {
        const uint32_t word = w[e / 2];
        vdst[e * 8] = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
    }
}

// Standard layout [num_blocks, block_size, kv_heads, head_dim] (the layout the
// shuffled one replaces; kept so the two can be compared): a token's head row
// is contiguous in source and cache, one 16-byte K and V vector per thread.
__global__ __launch_bounds__(256) void cache_write_standard_kernel(
    const uint4 *__restrict__ key, const uint4 *__restrict__ value, uint4 *__restrict__ k_cache,
    uint4 *__restrict__ v_cache, const int64_t *__restrict__ slot_mapping, int64_t num_tokens,
    int row_vecs, int B, int64_t num_blocks) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= num_tokens * row_vecs) return;
    const int64_t i = idx / row_vecs;
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= num_blocks * B) return;
    const int64_t dst = slot * row_vecs + (idx - i * row_vecs);  // (slot, head g, vector c)
    k_cache[dst] = key[idx];
    v_cache[dst] = value[idx];
}

// FP8 shuffled layout (x = 16 codes): thread (token, kv head, 16-dim group
// c) quantises 16 dims of K into one 16-byte vector,
// k_cache[p][g][c][o][0..16), and 16 dims of V into 16 single bytes,
// v_cache[p][g][o / 16][16 c + j][o % 16].  As for bf16, 16 neighbouring
// lanes take 16 consecutive tokens of the same dims (lane = 16 * (c % 4) +
// token % 16), so V's byte stores of consecutive slots sit side by side.
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(
    const uint4 *__restrict__ key, const uint4 *__restrict__ value, uint4 *__restrict__ k_cache,
    uint8_t *__restrict__ v_cache, const int64_t *__restrict__ slot_mapping, int64_t num_tokens,
    int Hkv, int D, int B, int64_t num_blocks, float k_inv, float v_inv) {
    const int C16 = D / kFp8X;  // a multiple of 4
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // t = ((group of 16 tokens * Hkv + g) * C16 / 4 + chunk block) * 64 + 16 * (c % 4) + token % 16
    const int lane = (int)(t & 63);
    const int64_t wv = t >> 6;
    const int cq = (int)(wv % (C16 / 4));
    const int g = (int)((wv / (C16 / 4)) % Hkv);
    const int64_t i16 = wv / ((int64_t)(C16 / 4) * Hkv);
    const int64_t i = i16 * 16 + (lane & 15);
    const int c = cq * 4 + (lane >> 4);
    if (i >= num_tokens) return;
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= num_blocks * B) return;
    const int64_t p = slot / B;
    const int o = (int)(slot % B);
    const size_t src = ((size_t)(i * Hkv + g) * C16 + c) * 2;  // two bf16 vectors per 16 dims
    k_cache[((p * Hkv + g) * C16 + c) * B + o] = quantize16(key[src], key[src + 1], k_inv);
    const uint4 vq = quantize16(value[src], value[src + 1], v_inv);
    const uint32_t w[4] = {vq.x, vq.y, vq.z, vq.w};
    uint8_t *vdst = v_cache + (((p * Hkv + g) * (B / kFp8X) + o / kFp8X) * D + c * kFp8X) * kFp8X +
                    o % kFp8X;
#pragma unroll
    for (int j = 0; j < 16; j++) vdst[j * kFp8X] = (uint8_t)(w[j / 4] >> ((j % 4) * 8));
}

// Latent rows are contiguous in both source and cache: one 16-byte vector per thread.
__global__ __launch_bounds__(256) void cache_write_latent_kernel(
    const uint4 *__restrict__ latent, uint4 *__restrict__ kv_cache,
    const int64_t *__restrict__ slot_mapping, int64_t num_tokens, int C, int B,
    int64_t num_blocks) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= num_tokens * C) return;
    const int64_t i = idx / C;
    const int c = (int)(idx % C);
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= num_blocks * B) return;
    kv_cache[slot * C + c] = latent[idx];
}

// FP8 latent rows: thread per 16-value vector, two bf16 vectors in, one code vector out.
__global__ __launch_bounds__(256) void cache_write_latent_fp8_kernel(
    const uint4 *__restrict__ latent, uint4 *__restrict__ kv_cache,
    const int64_t *__restrict__ slot_mapping, int64_t num_tokens, int C16, int B,
    int64_t num_blocks, float inv) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= num_tokens * C16) return;
    const int64_t i = idx / C16;
    const int c = (int)(idx % C16);
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= num_blocks * B) return;
    kv_cache[slot * C16 + c] = quantize16(latent[2 * idx], latent[2 * idx + 1], inv);
}

hipError_t launch_cache_write_shuffled(const void *key, const void *value, void *k_cache,
                                       void *v_cache, const int64_t *slot_mapping,
                                       int64_t num_tokens, int Hkv, int D, int B,
                                       int64_t num_blocks, hipStream_t stream) {
    const int64_t total = (num_tokens + 7) / 8 * 8 * Hkv * (D / 8);  // whole groups of 8 tokens
    const int64_t grid = (total + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (D == 128)
        hipLaunchKernelGGL(cache_write_shuffled_kernel<128>, dim3((unsigned)grid), dim3(256), 0,
                           stream, (const uint4 *)key, (const uint4 *)value, (uint16_t *)k_cache,
                           (uint16_t *)v_cache, slot_mapping, num_tokens, Hkv, B, num_blocks);
    else
        hipLaunchKernelGGL(cache_write_shuffled_kernel<64>, dim3((unsigned)grid), dim3(256), 0,
                           stream, (const uint4 *)key, (const uint4 *)value, (uint16_t *)k_cache,
                           (uint16_t *)v_cache, slot_mapping, num_tokens, Hkv, B, num_blocks);
    return hipGetLastError();
}

hipError_t launch_cache_write_standard(const void *key, const void *value, void *k_cache,
                                       void *v_cache, const int64_t *slot_mapping,
                                       int64_t num_tokens, int Hkv, int D, int B,
                                       int64_t num_blocks, hipStream_t stream) {
    const int row_vecs = Hkv * (D / 8);
    const int64_t grid = (num_tokens * row_vecs + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(cache_write_standard_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint4 *)key, (const uint4 *)value, (uint4 *)k_cache,
                       (uint4 *)v_cache, slot_mapping, num_tokens, row_vecs, B, num_blocks);
    return hipGetLastError();
}

hipError_t launch_cache_write_fp8(const void *key, const void *value, void *k_cache, void *v_cache,
                                  const int64_t *slot_mapping, int64_t num_tokens, int Hkv, int D,
                                  int B, int64_t num_blocks, float k_inv, float v_inv,
                                  hipStream_t stream) {
    const int64_t threads = (num_tokens + 15) / 16 * 16 * Hkv * (D / kFp8X);  // groups of 16
    const int64_t grid = (threads + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(cache_write_fp8_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint4 *)key, (const uint4 *)value, (uint4 *)k_cache,
                       (uint8_t *)v_cache, slot_mapping, num_tokens, Hkv, D, B, num_blocks, k_inv,
                       v_inv);
    return hipGetLastError();
}

hipError_t launch_cache_write_latent(const void *latent, void *kv_cache,
                                     const int64_t *slot_mapping, int64_t num_tokens, int Dl,
                                     int B, int64_t num_blocks, hipStream_t stream) {
    const int C = Dl / 8;
    const int64_t grid = (num_tokens * C + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(cache_write_latent_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint4 *)latent, (uint4 *)kv_cache, slot_mapping, num_tokens, C, B,
                       num_blocks);
    return hipGetLastError();
}

hipError_t launch_cache_write_latent_fp8(const void *latent, void *kv_cache,
                                         const int64_t *slot_mapping, int64_t num_tokens, int Dl,
                                         int B, int64_t num_blocks, float inv,
                                         hipStream_t stream) {
    const int C16 = Dl / kFp8X;
    const int64_t grid = (num_tokens * C16 + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(cache_write_latent_fp8_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint4 *)latent, (uint4 *)kv_cache, slot_mapping, num_tokens, C16, B,
                       num_blocks, inv);
    return hipGetLastError();
}

}  // namespace pa
