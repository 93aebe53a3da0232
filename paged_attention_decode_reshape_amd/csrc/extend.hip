// Chunked extend: new query tokens attend to their request's cached context
// (in the shuffled cache) and, causally, to themselves.
//
// The extend-path recipe of the "ROCm attention backends" blog processes
// the context in chunks: each chunk's attention yields a partial output and
// LSE, and merge_attn_states combines the partials and the new-token result.
// The blog gathers each chunk out of the shuffled cache into the standard
// [tokens, kv_heads, head_dim] layout first, because its attention kernel
// cannot read the shuffled one.  On gfx950 the shuffled layout is already
// the matrix-core operand layout (a K x-vector is 8 consecutive dims of one
// token, a V x-vector 8 consecutive tokens of one dim), so here the
// attention kernel reads the cache directly through the block table and the
// gather (gather_chunk_kernel) remains a separate exported operation.
//
// extend_attn_kernel  flash attention on gfx950 MFMA
//   (v_mfma_f32_32x32x16_bf16), head_dim 128, bf16 inputs, fp32
//   accumulation.  A workgroup takes 128 query rows of one (request, q head)
//   -- 32 per wave -- and one piece of the request's context: a run of whole
//   chunks (pieces exist only to balance long contexts over the GPU).  The
//   last piece also takes the request's new tokens with the causal mask.
//   Keys go 64 at a time through double-buffered LDS tiles: the next tile is
//   loaded straight into the other buffer (buffer_load_dwordx4 ... lds, in
//   the cache's own order) while the current one is used; one barrier per
//   tile.  Per tile:
//     S^T = K Q^T    (keys x queries): lane l owns query l % 32, so a
//                    query's softmax state sits in one lane pair (l, l + 32);
//                    the K rows are fed in a permuted order so that each
//                    lane's scores are already in the P^T operand layout;
//     O^T += V^T P^T (dims x queries): P is split into bf16 hi + lo parts
//                    (two MFMAs, ~2^-16 relative accuracy of the weights).
//   The online softmax keeps a reference maximum that moves only when a
//   score exceeds it by more than 8 (log2 units), so most tiles skip the
//   rescale of the running sum and output.  A request with one piece writes
//   its output and LSE directly; otherwise each piece writes an fp32 partial
//   (output, LSE) and extend_merge_kernel combines them.
// Workgroups are numbered so that the units sharing one (request, kv head,
// piece) -- and so the same K/V tiles -- run together on one XCD (blocks
// are dealt to the 8 XCDs round-robin) and share its L2.
#include "common.h"
#include "decode_common.h"
#include "fp8.h"
#include "launch.h"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kD = 128;
constexpr int kBM = 128;       // query rows per workgroup
constexpr int kBN = 64;        // keys per tile
constexpr int kXCDs = 8;
constexpr float kLazyLog2 = 8.f;

// Length of request r's context chunk in iteration `it` and its first row in
// the gathered chunk (prefix over earlier requests); recomputed on the
// device from the context lengths, so no host-built table is needed.
__device__ __forceinline__ int chunk_len(const int32_t *ctx, int r, int it, int chunk) {
    const int64_t rest = (int64_t)ctx[r] - (int64_t)it * chunk;
    return rest <= 0 ? 0 : (rest < chunk ? (int)rest : chunk);
}
__device__ __forceinline__ int chunk_start(const int32_t *ctx, int r, int it, int chunk) {
    int st = 0;
    for (int i = 0; i < r; i++) st += chunk_len(ctx, i, it, chunk);
    return st;
}

// One workgroup per (8-token group, request): K vectors are copied as they
// are; V goes through an 8 x 8 transpose per (kv head, 8 dims).
__global__ __launch_bounds__(256) void gather_chunk_kernel(GatherParams p) {
    const int r = blockIdx.y;
    const int it = p.iteration;
    const int len = chunk_len(p.context_lens, r, it, p.chunk);
    const int t8 = blockIdx.x * 8;  // first token of the group, chunk-relative
    if (t8 >= len) return;
    const int row0 = chunk_start(p.context_lens, r, it, p.chunk) + t8;
    const int ctx_t0 = it * p.chunk + t8;  // context position of the group's first token
    const int nt = min(8, len - t8);
    const int C = kD / 8;
    const uint4 *kc = reinterpret_cast<const uint4 *>(p.k_cache);
    const uint4 *vc = reinterpret_cast<const uint4 *>(p.v_cache);
    uint4 *ko = reinterpret_cast<uint4 *>(p.k_out);
    uint4 *vo = reinterpret_cast<uint4 *>(p.v_out);
    // the group lies inside one block (block_size is a multiple of 8)
    const int bi = ctx_t0 / p.B;
    const int b = bi < p.max_blocks ? p.block_table[(size_t)r * p.max_blocks + bi] : -1;
    const bool ok = b >= 0 && (int64_t)b < p.num_blocks;
    const int o0 = ctx_t0 % p.B;
    // K: Hkv * 8 tokens * 16 vectors
    for (int i = threadIdx.x; i < p.Hkv * 8 * C; i += blockDim.x) {
        const int g = i / (8 * C), t = (i / C) % 8, c = i % C;
        if (t >= nt) continue;
        const uint4 v = ok ? kc[(((size_t)b * p.Hkv + g) * C + c) * p.B + o0 + t] : make_uint4(0, 0, 0, 0);
        ko[((size_t)(row0 + t) * p.Hkv + g) * C + c] = v;
    }
    // V: Hkv * 16 dim groups, each an 8 x 8 transpose
    for (int i = threadIdx.x; i < p.Hkv * C; i += blockDim.x) {
        const int g = i / C, d8 = (i % C) * 8;
        uint32_t w[8][4];  // w[e] = 8 tokens of dim d8 + e, as 4 bf16 pairs
        const uint4 *src = vc + (((size_t)b * p.Hkv + g) * (p.B / 8) + o0 / 8) * kD + d8;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const uint4 v = ok ? src[e] : make_uint4(0, 0, 0, 0);
            w[e][0] = v.x; w[e][1] = v.y; w[e][2] = v.z; w[e][3] = v.w;
        }
#pragma unroll
        for (int t = 0; t < 8; t++) {
            if (t >= nt) break;
            uint32_t d[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; e2++) {
                // dims d8 + 2 e2 (lo) and d8 + 2 e2 + 1 (hi) of token t
                const uint32_t lo = (w[2 * e2][t >> 1] >> ((t & 1) * 16)) & 0xffffu;
                const uint32_t hi = (w[2 * e2 + 1][t >> 1] >> ((t & 1) * 16)) & 0xffffu;
                d[e2] = lo | (hi << 16);
            }
            vo[((size_t)(row0 + t) * p.Hkv + g) * C + d8 / 8] = make_uint4(d[0], d[1], d[2], d[3]);
        }
    }
}

// FP8 cache: thread (token, kv head, 8-dim group) writes 8 dequantised bf16
// values of K and of V: bf16(float(code) * scale), round to nearest even.
// K's 8 codes are half of one 16-byte vector; V's are one byte of each of 8
// dims' token vectors.
__global__ __launch_bounds__(256) void gather_chunk_fp8_kernel(GatherParams p) {
    const int r = blockIdx.y;
    const int it = p.iteration;
    const int len = chunk_len(p.context_lens, r, it, p.chunk);
    const int C8 = kD / 8, C16 = kD / kFp8X;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int t = (int)(idx / (p.Hkv * C8));
    if (t >= len) return;
    const int g = (int)(idx / C8 % p.Hkv), c8 = (int)(idx % C8);
    const int row = chunk_start(p.context_lens, r, it, p.chunk) + t;
    const int pos = it * p.chunk + t;
    const int bi = pos / p.B, o = pos % p.B;
    const int b = bi < p.max_blocks ? p.block_table[(size_t)r * p.max_blocks + bi] : -1;
    const bool ok = b >= 0 && (int64_t)b < p.num_blocks;
    const uint8_t *kc = reinterpret_cast<const uint8_t *>(p.k_cache);
    const uint8_t *vc = reinterpret_cast<const uint8_t *>(p.v_cache);
    uint32_t kw[2] = {0, 0}, vw[2] = {0, 0};
    if (ok) {
        const uint2 k2 = *reinterpret_cast<const uint2 *>(
            kc + ((((size_t)b * p.Hkv + g) * C16 + c8 / 2) * p.B + o) * kFp8X + (c8 % 2) * 8);
        kw[0] = k2.x;
        kw[1] = k2.y;
        const uint8_t *vs =
            vc + ((((size_t)b * p.Hkv + g) * (p.B / kFp8X) + o / kFp8X) * kD + c8 * 8) * kFp8X +
            o % kFp8X;
#pragma unroll
        for (int e = 0; e < 8; e++) vw[e / 4] |= (uint32_t)vs[e * kFp8X] << ((e % 4) * 8);
    }
    float kf[8], vf[8];
    fp8x4_to_f32(kw[0], kf);
    fp8x4_to_f32(kw[1], kf + 4);
    fp8x4_to_f32(vw[0], vf);
    fp8x4_to_f32(vw[1], vf + 4);
    uint32_t ko[4], vo[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        ko[e] = f32_to_bf16_rne(kf[2 * e] * p.k_scale) |
                (f32_to_bf16_rne(kf[2 * e + 1] * p.k_scale) << 16);
        vo[e] = f32_to_bf16_rne(vf[2 * e] * p.v_scale) |
                (f32_to_bf16_rne(vf[2 * e + 1] * p.v_scale) << 16);
    }
    const size_t dst = ((size_t)row * p.Hkv + g) * C8 + c8;
    reinterpret_cast<uint4 *>(p.k_out)[dst] = make_uint4(ko[0], ko[1], ko[2], ko[3]);
    reinterpret_cast<uint4 *>(p.v_out)[dst] = make_uint4(vo[0], vo[1], vo[2], vo[3]);
}

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t &a, const bf16x8_t &b, const f32x16_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4 &v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

// Raw buffer access: a descriptor of `bytes` bytes from `base`; a load past
// the end returns zeros without touching memory (a 0-byte descriptor turns
// every load into zeros).  0x00020000: gfx9 descriptor word 3, raw access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ext_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// The new tokens' V rearranged into the cache's 8-token groups:
// v_new_sh[g][grp][d][0..8) holds dim d of request r's new tokens
// 8 i .. 8 i + 7 at grp = q_start[r] / 8 + r + i (tokens past the request's
// end are zero).  The groups of consecutive requests never overlap:
// q_start[r + 1] / 8 + r + 1 >= q_start[r] / 8 + r + ceil(n_r / 8).
// One workgroup per (8-token group, request); a thread transposes 8 tokens x
// 8 dims of one kv head in registers.
__global__ __launch_bounds__(256) void shuffle_new_v_kernel(ExtendParams p) {
    const int r = blockIdx.y;
    const int q0 = p.q_start[r], q1 = p.q_start[r + 1];
    const int i8 = blockIdx.x * 8;
    if (q0 < 0 || q1 > p.Tn || i8 >= q1 - q0) return;
    const int nt = min(8, q1 - q0 - i8);
    const int grp = q0 / 8 + r + (int)blockIdx.x;
    const uint4 *src = reinterpret_cast<const uint4 *>(p.v_new);
    uint4 *dst = reinterpret_cast<uint4 *>(p.v_new_sh);
    for (int it = threadIdx.x; it < p.Hkv * 16; it += blockDim.x) {
        const int g = it >> 4, c = it & 15;
        uint32_t w[8][4];  // w[t] = dims 8 c .. 8 c + 7 of token t, as bf16 pairs
#pragma unroll
        for (int t = 0; t < 8; t++) {
            const uint4 v = t < nt ? src[((size_t)(q0 + i8 + t) * p.Hkv + g) * 16 + c]
                                   : make_uint4(0, 0, 0, 0);
            w[t][0] = v.x; w[t][1] = v.y; w[t][2] = v.z; w[t][3] = v.w;
        }
        uint4 *o = dst + ((size_t)g * p.new_groups + grp) * kD + 8 * c;
#pragma unroll
        for (int e = 0; e < 8; e++) {  // dim 8 c + e: tokens 0..7 as 4 bf16 pairs
            uint32_t d[4];
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint32_t lo = (w[2 * k][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                const uint32_t hi = (w[2 * k + 1][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                d[k] = lo | (hi << 16);
            }
            o[e] = make_uint4(d[0], d[1], d[2], d[3]);
        }
    }
}

// Exclusive prefix over requests of pieces * Hkv (the workgroup groups of
// each request), one workgroup, 256 requests per step.
__global__ __launch_bounds__(256) void extend_plan_kernel(ExtendParams p) {
    __shared__ int sc[256];
    int carry = 0;
    for (int base = 0; base < p.S; base += 256) {
        const int r = base + threadIdx.x;
        int v = 0;
        if (r < p.S) {
            int32_t len;
            v = extend_pieces(min(p.context_lens[r], p.max_ctx), p.piece_target, p.chunk, p.max_pieces, &len) * p.Hkv;
        }
        sc[threadIdx.x] = v;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int add = threadIdx.x >= off ? sc[threadIdx.x - off] : 0;
            __syncthreads();
            sc[threadIdx.x] += add;
            __syncthreads();
        }
        if (r < p.S) p.group_prefix[r + 1] = carry + sc[threadIdx.x];
        carry += sc[255];
        __syncthreads();
    }
    if (threadIdx.x == 0) p.group_prefix[0] = 0;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4
// ... lds): lane l's bytes land at lds + 16 l.  An instruction offset would
// move the LDS address as well, so none is used.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint4 *lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds, 16, (int)voff, 0, 0, 0);
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt not waited for)
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// LDS tiles of 64 keys, one per buffer (two buffers, distinct variables so
// that the compiler can tell the tile being read from the one being loaded):
//   K: [16-key run w][x-vector c][key w * 16 + o] (the cache block's own
//      order), 16 bytes each; wave w loads run w.
//   V: [8-token group][dim], 16 bytes (8 tokens of one dim) each; wave w
//      loads groups 2 w, 2 w + 1.
__shared__ __align__(16) uint4 ext_k0[kBN * 16];
__shared__ __align__(16) uint4 ext_k1[kBN * 16];
__shared__ __align__(16) uint4 ext_v0[8 * kD];
__shared__ __align__(16) uint4 ext_v1[8 * kD];

template <bool HILO>
__global__ __launch_bounds__(256, 2) void extend_attn_kernel(ExtendParams p) {
    // workgroup -> (group j, unit u): the units of a group are consecutive
    // blocks of one XCD
    const int G = p.Hq / p.Hkv;
    const int gs = G * p.q_blocks;
    const int t = (int)(blockIdx.x / kXCDs);
    const int j = (t / gs) * kXCDs + (int)(blockIdx.x % kXCDs);
    if (j >= p.num_groups) return;
    const int u = t % gs;
    // request of group j: the last r with group_prefix[r] <= j
    int lo = 0, hi = p.S - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (__builtin_amdgcn_readfirstlane(p.group_prefix[mid]) <= j) lo = mid;
        else hi = mid - 1;
    }
    const int r = lo;
    const int local = j - __builtin_amdgcn_readfirstlane(p.group_prefix[r]);
    const int piece = local / p.Hkv, g = local % p.Hkv;
    const int qb = u / G, h = g * G + u % G;
    const int q0 = __builtin_amdgcn_readfirstlane(p.q_start[r]);
    const int q1 = __builtin_amdgcn_readfirstlane(p.q_start[r + 1]);
    const int nq = q1 - q0;
    if (q0 < 0 || q1 > p.Tn || qb * kBM >= nq) return;
    const int ctx = min(__builtin_amdgcn_readfirstlane(p.context_lens[r]), p.max_ctx);
    int32_t plen;
    const int npieces = extend_pieces(ctx, p.piece_target, p.chunk, p.max_pieces, &plen);
    if (piece >= npieces) return;
    // keys: context tokens [c0, c1), then (last piece) new tokens [0, nk_new)
    const int c0 = piece * plen;
    const int c1 = max(c0, min(ctx, c0 + plen));
    const int n_ctx_tiles = (c1 - c0 + kBN - 1) / kBN;
    const int nk_new = piece == npieces - 1 ? min(nq, (qb + 1) * kBM) : 0;
    const int ntiles = n_ctx_tiles + (nk_new + kBN - 1) / kBN;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31, hl = lane >> 5, l16 = lane & 15, l4 = lane >> 4;
    const int qi = qb * kBM + wave * 32 + l32;  // this lane's query, request-relative
    const bool q_ok = qi < nq;
    const size_t qrow = (size_t)q0 + (q_ok ? qi : 0);


    // Q^T operand for the 8 k-steps of head_dim: dims 16 ks + 8 hl .. + 7
    bf16x8_t qf[8];
    {
        const uint4 *qp = reinterpret_cast<const uint4 *>(
            reinterpret_cast<const uint16_t *>(p.q) + (qrow * p.Hq + h) * kD) + hl;
        // a negative scale is applied as -q with |scale| (exact), so that
        // the softmax can take its maximum over raw scores
        const uint32_t sign = p.scale < 0.f ? 0x80008000u : 0u;
#pragma unroll
        for (int ks = 0; ks < 8; ks++) {
            uint4 v = q_ok ? qp[2 * ks] : make_uint4(0, 0, 0, 0);
            v.x ^= sign; v.y ^= sign; v.z ^= sign; v.w ^= sign;
            qf[ks] = as_bf16x8(v);
        }
    }

    f32x16_t o[4];
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
        for (int i = 0; i < 16; i++) o[db][i] = 0.f;
    float m = kNegInf, lsum = 0.f;
    // log2-domain scale, kept positive (a zero scale acts as 1e-30: the
    // weights are then 1 to within 1e-25, the uniform average)
    const float sl2 = fmaxf(fabsf(p.scale) * kLog2e, 1e-30f);

    const int B = p.B;
    const uint32_t k_ctx_off = (uint32_t)((l4 * B + l16) * 16);
    const uint32_t k_new_off = (uint32_t)((l16 * p.Hkv * 16 + l4) * 16);
    const uint32_t v_off = (uint32_t)(lane * 16);
    const int gbase = q0 / 8 + r;        // first group of the request's new V
    const int ngrp_r = (nq + 7) / 8;

    // Block-table entries of the wave's context tokens, 64 tiles at a time:
    // lane j of `win` holds the entry of tile win_base + j (-1: none).  The
    // window is read only when no tile load is in flight, so waiting for it
    // never waits for a tile, and the tile loop itself reads no table.
    const int32_t *bt_row = p.block_table + (size_t)r * p.max_blocks;
    int win = -1, win_base = 0;
    auto fetch_window = [&](int base) {
        const int ti = base + lane;
        const int tw = c0 + kBN * ti + 16 * wave;
        win = ti < n_ctx_tiles && tw < c1 ? bt_row[tw / B] : -1;
        win_base = base;
    };
    auto tile_block = [&](int i) {
        if (i - win_base >= 64) fetch_window(i);
        return __builtin_amdgcn_readlane(win, i - win_base);
    };
    // tile i's K and V into LDS (kbuf, vbuf): lane l of load u fills vector
    // slot 256 wave + 64 u + l of both
    auto load_tile = [&](int i, int blk, uint4 *kbuf, uint4 *vbuf) {
        uint4 *dk = kbuf + 256 * wave, *dv = vbuf + 256 * wave;
        if (i < n_ctx_tiles) {
            // context tokens tw .. tw + 15 lie in one cache block (B % 16 == 0)
            const int tw = c0 + kBN * i + 16 * wave;
            const int o0 = tw % B;
            const bool live = blk >= 0 && (int64_t)blk < p.num_blocks;
            const size_t region = (size_t)(live ? blk : 0) * p.Hkv + g;  // (block, kv head)
            const auto rk = ext_rsrc(reinterpret_cast<const char *>(p.k_cache) +
                                         (region * 16 * B + o0) * 16,
                                     live ? (uint32_t)((16 * B - o0) * 16) : 0u);
            const auto rv = ext_rsrc(reinterpret_cast<const char *>(p.v_cache) +
                                         (region * (B / 8) + o0 / 8) * (kD * 16),
                                     live ? (uint32_t)(2 * kD * 16) : 0u);
#pragma unroll
            for (int u4 = 0; u4 < 4; u4++) dma16(rk, dk + 64 * u4, k_ctx_off + u4 * 4 * B * 16);
#pragma unroll
            for (int u4 = 0; u4 < 4; u4++) dma16(rv, dv + 64 * u4, v_off + u4 * 64 * 16);
        } else {
            // new tokens tw .. tw + 15 (rows of k_new; groups of v_new_sh)
            const int tw = kBN * (i - n_ctx_tiles) + 16 * wave;
            const bool live = tw < nk_new;
            const auto rk = ext_rsrc(reinterpret_cast<const char *>(p.k_new) +
                                         ((size_t)(q0 + (live ? tw : 0)) * p.Hkv + g) * (kD * 2),
                                     live ? (uint32_t)(((nq - tw - 1) * p.Hkv + 1) * kD * 2) : 0u);
            const int gi = tw / 8;
            const auto rv = ext_rsrc(reinterpret_cast<const char *>(p.v_new_sh) +
                                         ((size_t)g * p.new_groups + gbase + (live ? gi : 0)) * (kD * 16),
                                     live ? (uint32_t)(min(2, ngrp_r - gi) * kD * 16) : 0u);
#pragma unroll
            for (int u4 = 0; u4 < 4; u4++) dma16(rk, dk + 64 * u4, k_new_off + u4 * 64);
#pragma unroll
            for (int u4 = 0; u4 < 4; u4++) dma16(rv, dv + 64 * u4, v_off + u4 * 64 * 16);
        }
    };
    // once the wave's loads of tile i have landed: context V past c1
    // (possibly uninitialised cache memory) is zeroed in the wave's own
    // slots, so that a zero weight never meets a NaN
    auto fix_tile = [&](int i, uint4 *vbuf) {
        if (i >= n_ctx_tiles) return;
        const int tw = c0 + kBN * i + 16 * wave;
        if (tw >= c1 || tw + 16 <= c1) return;
#pragma unroll
        for (int u4 = 0; u4 < 4; u4++) {
            const int nv = c1 - (tw + 8 * (u4 >> 1));  // valid tokens of the group
            uint4 &slot = vbuf[256 * wave + 64 * u4 + lane];
            uint4 v = slot;
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k2 = 0; k2 < 4; k2++)
                w[k2] &= (2 * k2 < nv ? 0xffffu : 0u) | (2 * k2 + 1 < nv ? 0xffff0000u : 0u);
            slot = make_uint4(w[0], w[1], w[2], w[3]);
        }
    };

    if (ntiles > 0) {
        fetch_window(0);
        load_tile(0, tile_block(0), ext_k0, ext_v0);
        wait_dma();
        fix_tile(0, ext_v0);
    }
    __syncthreads();
    // one tile: start loading tile i + 1 into the other buffers, attend to
    // tile i, wait for tile i + 1 and meet at the barrier
    auto step = [&](int i, const uint4 *sk, const uint4 *sv, uint4 *nk, uint4 *nv) {
        if (i + 1 < ntiles) load_tile(i + 1, tile_block(i + 1), nk, nv);
        // S^T = K Q^T for the two 32-key blocks of the tile
        f32x16_t s[2];
        // A-operand row l32 holds tile key 32 kb + pi(l32), pi swapping bits
        // 2 and 3 (run 2 kb + l32 / 16 of the LDS tile); then the result rows
        // a lane holds are 8 consecutive keys per 16-key step, the layout of
        // the P^T operand, and no regrouping of P across lanes is needed.
        // The two key blocks' accumulations alternate, so that consecutive
        // matrix instructions are independent.
        const int pr = (l32 & 3) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
        const uint4 *kr = sk + (l32 >> 4) * 256 + 16 * hl + pr;
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int e = 0; e < 16; e++) s[kb][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ks++)
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
                s[kb] = mfma32(as_bf16x8(kr[2 * kb * 256 + 32 * ks]), qf[ks], s[kb]);
        // s[kb][e]: tile key 32 kb + 16 (e / 8) + 8 hl + e % 8 of query qi.
        // Visible keys: tile keys below `lim` (context end; new tokens: the
        // causal bound and the request's end).
        int lim, wave_lim;
        if (i < n_ctx_tiles) {
            lim = wave_lim = c1 - (c0 + kBN * i);
        } else {
            const int kt0 = kBN * (i - n_ctx_tiles);
            lim = min(qi + 1, nk_new) - kt0;
            wave_lim = min(qb * kBM + wave * 32 + 1, nk_new) - kt0;  // the wave's first query
        }
        // the maximum is taken over raw scores (sl2 > 0); hidden keys get -inf
        float mx = kNegInf;
        if (wave_lim >= kBN) {
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int e = 0; e < 16; e++) mx = fmax_nc(mx, s[kb][e]);
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const int kl = 32 * kb + 16 * (e >> 3) + 8 * hl + (e & 7);
                    s[kb][e] = kl < lim ? s[kb][e] : kNegInf;
                    mx = fmax_nc(mx, s[kb][e]);
                }
        }
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                             false, false);
            mx = fmax_nc(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            mx = mx == kNegInf ? kNegInf : mx * sl2;
        }
        // lazy reference maximum: moves only when a score passes it by more
        // than 2^8, so weights stay <= 256
        const bool grow = mx > m + kLazyLog2;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float mn = grow ? mx : m;
            const float alpha = grow ? fast_exp2(m - mn) : 1.f;
            m = mn;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < 4; db++)
#pragma unroll
                for (int e = 0; e < 16; e++) o[db][e] *= alpha;
        }
        const float mref = m == kNegInf ? 0.f : m;
        // P^T as the B operand of O^T += V^T P^T: bf16 pairs (e, e + 1); lane
        // half hl holds keys 8 hl .. 8 hl + 7 of each 16-key step
        uint32_t pk[2][8], pl[2][8];
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
#pragma unroll
            for (int jj = 0; jj < 8; jj++) {
                const float a = fast_exp2(__builtin_fmaf(s[kb][2 * jj], sl2, -mref));
                const float c = fast_exp2(__builtin_fmaf(s[kb][2 * jj + 1], sl2, -mref));
                pk[kb][jj] = pack_bf16x2(a, c);
                if constexpr (HILO) {
                    pl[kb][jj] = pack_bf16x2(a - bf16_lo(pk[kb][jj]), c - bf16_hi(pk[kb][jj]));
                    lsum += a + c;
                } else {
                    lsum += bf16_lo(pk[kb][jj]) + bf16_hi(pk[kb][jj]);
                }
            }
        }
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int sp = 0; sp < 2; sp++) {
                const bf16x8_t pb = as_bf16x8(make_uint4(pk[kb][4 * sp], pk[kb][4 * sp + 1],
                                                         pk[kb][4 * sp + 2], pk[kb][4 * sp + 3]));
                bf16x8_t pbl;
                if constexpr (HILO)
                    pbl = as_bf16x8(make_uint4(pl[kb][4 * sp], pl[kb][4 * sp + 1],
                                               pl[kb][4 * sp + 2], pl[kb][4 * sp + 3]));
                // V^T operand: dims 32 db + l32, tokens of group 4 kb + 2 sp + hl;
                // the hi products of the 4 dim blocks go first, then the lo
                // ones, so that consecutive matrix instructions are independent
                const uint4 *vr = sv + (4 * kb + 2 * sp + hl) * kD + l32;
                bf16x8_t va[4];
#pragma unroll
                for (int db = 0; db < 4; db++) {
                    va[db] = as_bf16x8(vr[32 * db]);
                    o[db] = mfma32(va[db], pb, o[db]);
                }
                if constexpr (HILO)
#pragma unroll
                    for (int db = 0; db < 4; db++) o[db] = mfma32(va[db], pbl, o[db]);
            }
        if (i + 1 < ntiles) {
            wait_dma();
            fix_tile(i + 1, nv);
        }
        __syncthreads();
    };
    for (int i = 0; i < ntiles; i += 2) {
        step(i, ext_k0, ext_v0, ext_k1, ext_v1);
        if (i + 1 < ntiles) step(i + 1, ext_k1, ext_v1, ext_k0, ext_v0);
    }

    // the lane pair (l, l + 32) holds the same query over different keys
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum),
                                                         false, false);
        lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const float L = lsum > 0.f ? (m + fast_log2(lsum)) * kLn2 : kNegInf;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    if (!q_ok) return;
    // o[db][e]: dim 32 db + 8 (e / 4) + 4 hl + e % 4 of query qi
    const size_t row = qrow * p.Hq + h;
    if (npieces == 1) {
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
            for (int e = 0; e < 16; e += 4) {
                const int d = 32 * db + 8 * (e >> 2) + 4 * hl;
                uint2 w;
                w.x = pack_bf16x2(o[db][e] * inv, o[db][e + 1] * inv);
                w.y = pack_bf16x2(o[db][e + 2] * inv, o[db][e + 3] * inv);
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.out) + row * kD + d) = w;
            }
        if (hl == 0 && p.lse) p.lse[row] = L;
    } else {
        float *po = p.part_out + (row * p.max_pieces + piece) * kD;
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
            for (int e = 0; e < 16; e += 4) {
                const int d = 32 * db + 8 * (e >> 2) + 4 * hl;
                *reinterpret_cast<float4 *>(po + d) =
                    make_float4(o[db][e] * inv, o[db][e + 1] * inv, o[db][e + 2] * inv, o[db][e + 3] * inv);
            }
        if (hl == 0) p.part_lse[row * p.max_pieces + piece] = L;
    }
}

// LSE merge of the pieces of split requests (merge_attn_states over n
// parts): 8 (token, head) rows per workgroup, 4 dims per thread.
__global__ __launch_bounds__(256) void extend_merge_kernel(ExtendParams p) {
    const int r = blockIdx.y;
    const int q0 = p.q_start[r], q1 = p.q_start[r + 1];
    if (q0 < 0 || q1 > p.Tn || q1 <= q0) return;
    int32_t plen;
    const int npieces =
        extend_pieces(min(p.context_lens[r], p.max_ctx), p.piece_target, p.chunk, p.max_pieces, &plen);
    if (npieces < 2) return;
    const int64_t rows = (int64_t)(q1 - q0) * p.Hq;
    const int64_t first = (int64_t)blockIdx.x * 8;
    if (first >= rows) return;
    merge_partition_rows<kD, 4, kExtendMaxPieces, 256>(
        p.part_out, p.part_lse, p.max_pieces, reinterpret_cast<uint16_t *>(p.out), p.lse,
        (size_t)q0 * p.Hq + first, (int)min<int64_t>(8, rows - first), npieces);
}

}  // namespace

hipError_t launch_gather_chunk(const GatherParams &p, int max_chunk_len, hipStream_t stream) {
    if (max_chunk_len <= 0 || p.S <= 0) return hipSuccess;
    if (p.fp8) {
        const int64_t threads = (int64_t)max_chunk_len * p.Hkv * (kD / 8);
        hipLaunchKernelGGL(gather_chunk_fp8_kernel, dim3((unsigned)((threads + 255) / 256), (unsigned)p.S),
                           dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    const unsigned gx = (unsigned)((max_chunk_len + 7) / 8);
    hipLaunchKernelGGL(gather_chunk_kernel, dim3(gx, (unsigned)p.S), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_extend(const ExtendParams &p, int max_new, hipStream_t stream) {
    if (max_new <= 0 || p.S <= 0 || p.num_groups <= 0) return hipSuccess;
    hipLaunchKernelGGL(extend_plan_kernel, dim3(1), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(shuffle_new_v_kernel, dim3((unsigned)((max_new + 7) / 8), (unsigned)p.S),
                       dim3(256), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t gs = (int64_t)(p.Hq / p.Hkv) * p.q_blocks;
    const int64_t blocks = (int64_t)(p.num_groups + kXCDs - 1) / kXCDs * kXCDs * gs;
    // hi / lo weights: a single bf16 rounding of the weights misses the
    // output tolerance when a few keys dominate
    hipLaunchKernelGGL(extend_attn_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t rows = (int64_t)max_new * p.Hq;
    hipLaunchKernelGGL(extend_merge_kernel, dim3((unsigned)((rows + 7) / 8), (unsigned)p.S),
                       dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa
