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
// together, and K's vectors are contiguous too.  One thread per 16-byte
// source vector: the fastest form for small writes (a decode step, a mixed
// batch), where the chunked kernel below has too few workgroups to hide its
// barriers.
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
    // under which L2 combines them into whole vectors (non-temporal V stores
    // were 55% slower on a bulk fill).
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

// Chunks of kRun consecutive tokens of one kv head per workgroup.  K vectors
// go straight to the cache as above.  V is staged in LDS: an 8-slot group of
// a V vector (8 consecutive tokens of one dim) whose 8 slots are filled by 8
// consecutive tokens with consecutive slots is written whole, as 16-byte
// vectors, by the workgroup whose chunk holds the group's first token (it
// stages kExt tokens past its chunk to complete such groups); every other
// token's V is written 2 bytes per dim.  Token t's group is full when its
// would-be first token t0 = t - slot(t) % 8 has slot(t0) % 8 == 0 and tokens
// t0 .. t0 + 7 have slots slot(t0) .. slot(t0) + 7, all inside the cache;
// every workgroup that sees a group decides the same way, so each V value
// is written exactly once.  A prefill or bulk fill (sequences starting
// at slot 0 of their blocks, consecutive slots) writes all but each
// sequence's last partial group whole.  Access policies as above.  Measured
// against the per-vector kernel (one kv head, head_dim 128): 25.9 vs 32.9 us
// for 93.5k tokens, 6.4 vs 7.4 us for 16k, 5.4 vs 5.2 us for 8k, 4.6 vs
// 2.9 us for 256; the launcher picks it from kRunsMinRows token-heads up.
constexpr int kRun = 32, kExt = 8;
constexpr int64_t kRunsMinRows = 12288;  // tokens x kv heads
template <int D>
__global__ __launch_bounds__(256) void cache_write_runs_kernel(
    const uint4 *__restrict__ key, const uint4 *__restrict__ value, uint16_t *__restrict__ k_cache,
    uint16_t *__restrict__ v_cache, const int64_t *__restrict__ slot_mapping, int64_t num_tokens,
    int Hkv, int B, int64_t num_blocks) {
    constexpr int C = D / 8;                  // 16-byte vectors per head row
    constexpr int kWin = kExt + kRun + kExt;  // slots of tokens t_begin - kExt .. t_begin + kRun + kExt
    __shared__ int64_t sl[kWin];
    __shared__ uint8_t full[kExt + kRun];      // full group starting at token t_begin + r - kExt
    __shared__ int64_t kb[kRun], vb[kRun];     // cache offsets of chunk token r for dim 0
    __shared__ int64_t vs[kRun];               // vb[r] if token r's V is stored 2 bytes a dim, else -1
    __shared__ __align__(16) uint16_t vl[kRun + kExt][D];
    // workgroups go round-robin over the 8 XCDs: give each XCD a contiguous
    // range of chunks, so that the 8 tokens a chunk stages past its end are
    // read by the L2 that also holds the next chunk
    const uint32_t n = gridDim.x, per = n / 8, rem = n % 8, x = blockIdx.x % 8;
    const uint32_t wg = x * per + min(x, rem) + blockIdx.x / 8;
    const int g = (int)(wg % Hkv);
    const int64_t t_begin = (int64_t)(wg / Hkv) * kRun;
    const int tid = threadIdx.x;
    const int64_t cap = num_blocks * B;
    // Every global load is issued before the first wait: the slots, V of
    // tokens t_begin .. t_begin + kRun + kExt - 1 and K of the chunk's tokens.
    // The loads are unconditional, from indexes clamped into the inputs, so
    // that none waits for another; what a clamped load brings (tokens past
    // the end) is never stored, as those tokens have no slot.
    constexpr int NV = ((kRun + kExt) * C + 255) / 256, NK = (kRun * C + 255) / 256;
    const int64_t last = num_tokens - 1;
    const int64_t ts = t_begin - kExt + min(tid, kWin - 1);
    const int64_t sv = slot_mapping[ts < 0 ? 0 : (ts > last ? last : ts)];
    dw4_t vr[NV], kr[NK];
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int idx = min(tid + 256 * i, (kRun + kExt) * C - 1), r = idx / C, c = idx % C;
        const int64_t t = min(t_begin + r, last);
        vr[i] = __builtin_nontemporal_load(reinterpret_cast<const dw4_t *>(value) +
                                           ((size_t)t * Hkv + g) * C + c);
    }
#pragma unroll
    for (int i = 0; i < NK; i++) {
        const int idx = min(tid + 256 * i, kRun * C - 1), r = idx / C, c = idx % C;
        const int64_t t = min(t_begin + r, last);
        kr[i] = __builtin_nontemporal_load(reinterpret_cast<const dw4_t *>(key) +
                                           ((size_t)t * Hkv + g) * C + c);
    }
    if (tid < kWin) sl[tid] = (ts < 0 || ts > last || sv < 0 || sv >= cap) ? -1 : sv;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int idx = tid + 256 * i, r = idx / C, c = idx % C;
        if (idx < (kRun + kExt) * C) *reinterpret_cast<dw4_t *>(&vl[r][8 * c]) = vr[i];
    }
    __syncthreads();
    // Which tokens start a full group (wave 0), and each chunk token's cache
    // offsets for dim 0 and whether its V goes 2 bytes a dim (wave 1), one
    // 64-bit division per token.
    if (tid < kExt + kRun) {
        const int64_t s0 = sl[tid];
        bool f = s0 >= 0 && (s0 & 7) == 0;
#pragma unroll
        for (int j = 1; j < 8; j++) f = f && sl[tid + j] == s0 + j;
        full[tid] = f;
    } else if (tid >= 64 && tid < 64 + kRun) {
        const int r = tid - 64;
        const int64_t slot = sl[kExt + r];
        int64_t single = -1;
        if (slot >= 0) {
            const int64_t p = slot / B;
            const int o = (int)(slot - p * B);
            kb[r] = ((p * Hkv + g) * C) * B + o;                          // 16-byte vectors
            vb[r] = (((p * Hkv + g) * (B / 8) + o / 8) * D) * 8 + (o & 7);  // 2-byte elements
            // the same test as above, for the group this token would belong to
            const int j0 = kExt + r - (int)(slot & 7);
            const int64_t s0 = sl[j0];
            bool f = s0 >= 0 && (s0 & 7) == 0;
#pragma unroll
            for (int j = 1; j < 8; j++) f = f && sl[j0 + j] == s0 + j;
            if (!f) single = vb[r];
        }
        vs[r] = single;
    }
    __syncthreads();
    // K vector (dims 8c .. 8c+7 of slot o) -> k_cache[p][g][c][o][0..8)
#pragma unroll
    for (int i = 0; i < NK; i++) {
        const int idx = tid + 256 * i, r = idx / C, c = idx % C;
        if (idx < kRun * C && sl[kExt + r] >= 0)
            __builtin_nontemporal_store(kr[i], reinterpret_cast<dw4_t *>(k_cache) + kb[r] + c * B);
    }
    // every wave takes the mask of full groups starting in the chunk itself
    const int lane = tid & 63;
    const uint32_t fm = (uint32_t)__ballot(lane < kRun && full[kExt + lane]);
    const int nfull = __popc(fm);
    // whole V vectors of those groups: v_cache[p][g][o / 8][d][0..8), o % 8 == 0
    for (int q = tid / D; q < nfull; q += 256 / D) {
        uint32_t mm = fm;
        for (int k = 0; k < q; k++) mm &= mm - 1;
        const int r = __builtin_ctz(mm);
        const int d = tid % D;
        dw4_t v;
#pragma unroll
        for (int j = 0; j < 4; j++)
            v[j] = (uint32_t)vl[r + 2 * j][d] | ((uint32_t)vl[r + 2 * j + 1][d] << 16);
        reinterpret_cast<uint4 *>(v_cache)[vb[r] / 8 + d] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    // the other tokens of the chunk, 2 bytes per dim: v_cache[p][g][o / 8][d][o % 8]
#pragma unroll
    for (int i = 0; i < kRun * D / 256; i++) {
        const int idx = tid + 256 * i, r = idx / D, d = idx % D;
        const int64_t dst = vs[r];
        if (dst >= 0) v_cache[dst + d * 8] = vl[r][d];
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
    if (num_tokens * Hkv < kRunsMinRows) {
        const int64_t total = (num_tokens + 7) / 8 * 8 * Hkv * (D / 8);  // whole groups of 8 tokens
        const int64_t vgrid = (total + 255) / 256;
        if (vgrid == 0) return hipSuccess;
        if (D == 128)
            hipLaunchKernelGGL(cache_write_shuffled_kernel<128>, dim3((unsigned)vgrid), dim3(256), 0,
                               stream, (const uint4 *)key, (const uint4 *)value, (uint16_t *)k_cache,
                               (uint16_t *)v_cache, slot_mapping, num_tokens, Hkv, B, num_blocks);
        else
            hipLaunchKernelGGL(cache_write_shuffled_kernel<64>, dim3((unsigned)vgrid), dim3(256), 0,
                               stream, (const uint4 *)key, (const uint4 *)value, (uint16_t *)k_cache,
                               (uint16_t *)v_cache, slot_mapping, num_tokens, Hkv, B, num_blocks);
        return hipGetLastError();
    }
    const int64_t grid = (num_tokens + kRun - 1) / kRun * Hkv;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (D == 128)
        hipLaunchKernelGGL(cache_write_runs_kernel<128>, dim3((unsigned)grid), dim3(256), 0,
                           stream, (const uint4 *)key, (const uint4 *)value, (uint16_t *)k_cache,
                           (uint16_t *)v_cache, slot_mapping, num_tokens, Hkv, B, num_blocks);
    else
        hipLaunchKernelGGL(cache_write_runs_kernel<64>, dim3((unsigned)grid), dim3(256), 0,
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
