// Chunked extend: context gather and MFMA tile attention with LSE merges.
//
// The extend-path recipe of the "ROCm attention backends" blog: new query
// tokens attend to their own new K/V (causal) and to the request's cached
// context, which lives in the shuffled cache.  The context is processed in
// chunks: each iteration gathers every request's next chunk from the
// shuffled cache into the standard [tokens, kv_heads, head_dim] layout,
// runs attention of the new queries over it without a mask, and merges the
// result into the running one by log-sum-exp (merge_attn_states semantics).
//
// gather_chunk_kernel  K vectors copy 16 bytes at a time; a V vector of the
//   cache holds 8 tokens of one dim, so 8 of them (8 dims) are transposed
//   in registers into 8 standard-layout vectors (8 dims of one token).
// fa_kernel  flash attention on gfx950 MFMA (v_mfma_f32_32x32x16_bf16),
//   head_dim 128, bf16 inputs, fp32 accumulation.  A workgroup takes 128
//   query rows of one (request, q head), 32 per wave, and walks the keys 64
//   at a time through LDS:
//     S^T = K Q^T   (keys x queries): lane l owns query l % 32, so the
//                   online softmax state of a query sits in one lane pair
//                   (l, l + 32) and needs no shuffles beyond one swap;
//     O^T += V^T P^T (dims x queries): P is split into bf16 hi + lo parts
//                   (two MFMAs, ~2^-16 relative accuracy of the weights),
//                   regrouped between the lane halves with v_permlane32_swap
//                   into the MFMA operand layout; V^T is read from an LDS
//                   tile that the workgroup writes transposed.
//   The epilogue either writes the result, merges it into the running
//   (output, LSE) state, or (last step) writes the bf16 output and LSE.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kD = 128;
constexpr int kBM = 128;       // query rows per workgroup
constexpr int kBN = 64;        // keys per tile
constexpr int kKRow = kD + 8;  // LDS K row stride in bf16 (272 bytes: conflict-free 16-byte reads)
constexpr int kVRow = kBN + 8; // LDS V^T row stride in bf16 (144 bytes)

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

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t &a, const bf16x8_t &b, const f32x16_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4 &v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

// MODE 0: write the result as the running state; 1: merge it into the
// running state; FINAL: write the bf16 output and LSE instead of the
// running state.  HILO: P is split into bf16 hi + lo parts (two MFMAs per
// step, ~2^-16 relative accuracy) for attention over few keys, where a
// single bf16 rounding of a dominant weight would show in the output.
template <bool CAUSAL, int MODE, bool FINAL, bool HILO>
__global__ __launch_bounds__(256, 2) void fa_kernel(FAParams p) {
    const int qb = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
    const int q0 = p.q_start[r];
    const int nq = p.q_start[r + 1] - q0;
    if (qb * kBM >= nq) return;
    int k0, nk;
    if (p.chunk > 0) {  // keys: this iteration's gathered context chunk
        k0 = chunk_start(p.context_lens, r, p.iteration, p.chunk);
        nk = chunk_len(p.context_lens, r, p.iteration, p.chunk);
    } else {            // keys: the request's new tokens
        k0 = q0;
        nk = nq;
    }
    const int g = h / (p.Hq / p.Hkv);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31, hl = lane >> 5;
    const int qi = qb * kBM + wave * 32 + l32;  // this lane's query, request-relative
    const bool q_ok = qi < nq;
    const size_t qrow = (size_t)q0 + (q_ok ? qi : 0);

    __shared__ __align__(16) uint16_t sK[kBN * kKRow];
    __shared__ __align__(16) uint16_t sVt[kD * kVRow];

    // Q^T operand for the 8 k-steps of head_dim: dims 16 ks + 8 hl .. + 7
    bf16x8_t qf[8];
    {
        const uint4 *qp = reinterpret_cast<const uint4 *>(
            reinterpret_cast<const uint16_t *>(p.q) + (qrow * p.Hq + h) * kD) + hl;
#pragma unroll
        for (int ks = 0; ks < 8; ks++) qf[ks] = as_bf16x8(q_ok ? qp[2 * ks] : make_uint4(0, 0, 0, 0));
    }

    f32x16_t o[4];
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
        for (int i = 0; i < 16; i++) o[db][i] = 0.f;
    float m = kNegInf, lsum = 0.f;
    const float sl2 = p.scale * kLog2e;

    // keys past the block's last query are never visible under the causal mask
    const int nk_eff = CAUSAL ? min(nk, (qb + 1) * kBM + (nk - nq)) : nk;
    const uint16_t *kbase = reinterpret_cast<const uint16_t *>(p.k) + ((size_t)k0 * p.Hkv + g) * kD;
    const uint16_t *vbase = reinterpret_cast<const uint16_t *>(p.v) + ((size_t)k0 * p.Hkv + g) * kD;
    const size_t kstride = (size_t)p.Hkv * kD;

    // K and V of a tile go global -> registers -> LDS; the next tile's loads
    // are issued right after the current tile is in LDS, so they overlap its
    // math.  K: thread -> (key, vector) for 4 keys; V: thread -> (key pair,
    // 8 dims) for 2 pairs (past the end: zeros, no memory access).
    uint4 kreg[4], va[2], vb[2];
    auto load_kv = [&](int kt0) {
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int idx = threadIdx.x + 256 * u, key = idx >> 4, c = idx & 15;
            kreg[u] = kt0 + key < nk
                          ? *reinterpret_cast<const uint4 *>(kbase + (size_t)(kt0 + key) * kstride + 8 * c)
                          : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int idx = threadIdx.x + 256 * u, pr = idx & 31, c = idx >> 5;
            const int key = 2 * pr;
            va[u] = kt0 + key < nk
                        ? *reinterpret_cast<const uint4 *>(vbase + (size_t)(kt0 + key) * kstride + 8 * c)
                        : make_uint4(0, 0, 0, 0);
            vb[u] = kt0 + key + 1 < nk
                        ? *reinterpret_cast<const uint4 *>(vbase + (size_t)(kt0 + key + 1) * kstride + 8 * c)
                        : make_uint4(0, 0, 0, 0);
        }
    };
    // K rows as they are (16-byte LDS writes); V transposed: for each dim the
    // key pair's two values form one 4-byte LDS write
    auto store_kv = [&]() {
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int idx = threadIdx.x + 256 * u, key = idx >> 4, c = idx & 15;
            *reinterpret_cast<uint4 *>(&sK[key * kKRow + 8 * c]) = kreg[u];
        }
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int idx = threadIdx.x + 256 * u, pr = idx & 31, c = idx >> 5;
            const int key = 2 * pr;
            const uint32_t aw[4] = {va[u].x, va[u].y, va[u].z, va[u].w};
            const uint32_t bw[4] = {vb[u].x, vb[u].y, vb[u].z, vb[u].w};
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const uint32_t lo = (aw[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                const uint32_t hi = (bw[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                *reinterpret_cast<uint32_t *>(&sVt[(8 * c + e) * kVRow + key]) = lo | (hi << 16);
            }
        }
    };

    load_kv(0);
    for (int kt0 = 0; kt0 < nk_eff; kt0 += kBN) {
        store_kv();
        __syncthreads();
        load_kv(kt0 + kBN);

        // S^T = K Q^T for the two 32-key blocks of the tile
        f32x16_t s[2];
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
#pragma unroll
            for (int i = 0; i < 16; i++) s[kb][i] = 0.f;
            const uint16_t *kr = &sK[(kb * 32 + l32) * kKRow + 8 * hl];
#pragma unroll
            for (int ks = 0; ks < 8; ks++)
                s[kb] = mfma32(as_bf16x8(*reinterpret_cast<const uint4 *>(kr + 16 * ks)), qf[ks], s[kb]);
        }
        // s[kb][i]: key kt0 + 32 kb + 8 (i / 4) + 4 hl + i % 4 of query qi
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int key = kt0 + 32 * kb + 8 * (i >> 2) + 4 * hl + (i & 3);
                const bool vis = key < nk && (!CAUSAL || key <= qi + (nk - nq));
                s[kb][i] = vis ? s[kb][i] * sl2 : kNegInf;
                mx = fmax_nc(mx, s[kb][i]);
            }
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                             false, false);
            mx = fmax_nc(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float mn = fmax_nc(m, mx);
        const float mref = mn == kNegInf ? 0.f : mn;
        const float alpha = fast_exp2(m - mref);
        m = mn;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
            for (int i = 0; i < 16; i++) o[db][i] *= alpha;
        // P^T as the B operand of O^T += V^T P^T: bf16 pairs (i, i + 1),
        // regrouped so that lane half 0 holds keys 0-7 and half 1 keys 8-15
        // of each 16-key step
        uint32_t pk[2][8], pl[2][8];
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const float a = fast_exp2(s[kb][2 * j] - mref), b = fast_exp2(s[kb][2 * j + 1] - mref);
                pk[kb][j] = pack_bf16x2(a, b);
                if constexpr (HILO) {
                    pl[kb][j] = pack_bf16x2(a - bf16_lo(pk[kb][j]), b - bf16_hi(pk[kb][j]));
                    lsum += a + b;
                } else {
                    lsum += bf16_lo(pk[kb][j]) + bf16_hi(pk[kb][j]);
                }
            }
#pragma unroll
            for (int j = 0; j < 8; j += 4) {
#pragma unroll
                for (int jj = 0; jj < 2; jj++) {
                    auto x = __builtin_amdgcn_permlane32_swap(pk[kb][j + jj], pk[kb][j + jj + 2], false, false);
                    pk[kb][j + jj] = x[0];
                    pk[kb][j + jj + 2] = x[1];
                    if constexpr (HILO) {
                        auto y = __builtin_amdgcn_permlane32_swap(pl[kb][j + jj], pl[kb][j + jj + 2], false, false);
                        pl[kb][j + jj] = y[0];
                        pl[kb][j + jj + 2] = y[1];
                    }
                }
            }
        }
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int st = 0; st < 2; st++) {
                const bf16x8_t pb = as_bf16x8(make_uint4(pk[kb][4 * st], pk[kb][4 * st + 1],
                                                         pk[kb][4 * st + 2], pk[kb][4 * st + 3]));
                bf16x8_t pbl;
                if constexpr (HILO)
                    pbl = as_bf16x8(make_uint4(pl[kb][4 * st], pl[kb][4 * st + 1],
                                               pl[kb][4 * st + 2], pl[kb][4 * st + 3]));
                const int kk = 32 * kb + 16 * st + 8 * hl;
#pragma unroll
                for (int db = 0; db < 4; db++) {
                    const bf16x8_t va = as_bf16x8(
                        *reinterpret_cast<const uint4 *>(&sVt[(32 * db + l32) * kVRow + kk]));
                    o[db] = mfma32(va, pb, o[db]);
                    if constexpr (HILO) o[db] = mfma32(va, pbl, o[db]);
                }
            }
        __syncthreads();
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
    // o[db][i]: dim 32 db + 8 (i / 4) + 4 hl + i % 4 of query qi
    const size_t orow = qrow * p.Hq + h;
    float *run_o = p.run_out + orow * kD;
    float Lr = kNegInf, wr = 0.f, wn = 1.f, invd = inv;
    if constexpr (MODE == 1) {
        Lr = p.run_lse[orow];
        const float M = fmax_nc(Lr, L);
        const float Mr = M == kNegInf ? 0.f : M;
        wr = fast_exp2((Lr - Mr) * kLog2e);
        wn = fast_exp2((L - Mr) * kLog2e);
        const float den = wr + wn;
        const float id = den > 0.f ? 1.f / den : 0.f;
        wr *= id;
        wn *= id;
        invd = inv * wn;
        Lr = den > 0.f ? Mr + fast_log2(den) * kLn2 : kNegInf;
    } else {
        Lr = L;
    }
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
            const int d = 32 * db + 8 * (i >> 2) + 4 * hl;
            float4 v = make_float4(o[db][i] * invd, o[db][i + 1] * invd, o[db][i + 2] * invd,
                                   o[db][i + 3] * invd);
            if constexpr (MODE == 1) {
                const float4 pr = *reinterpret_cast<const float4 *>(run_o + d);
                v.x += wr * pr.x;
                v.y += wr * pr.y;
                v.z += wr * pr.z;
                v.w += wr * pr.w;
            }
            if constexpr (FINAL) {
                uint2 b;
                b.x = pack_bf16x2(v.x, v.y);
                b.y = pack_bf16x2(v.z, v.w);
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.out) + orow * kD + d) = b;
            } else {
                *reinterpret_cast<float4 *>(run_o + d) = v;
            }
        }
    if (hl == 0) {
        if constexpr (FINAL) {
            if (p.lse) p.lse[orow] = Lr;
        } else {
            p.run_lse[orow] = Lr;
        }
    }
}

}  // namespace

hipError_t launch_gather_chunk(const GatherParams &p, int max_chunk_len, hipStream_t stream) {
    if (max_chunk_len <= 0 || p.S <= 0) return hipSuccess;
    const unsigned gx = (unsigned)((max_chunk_len + 7) / 8);
    hipLaunchKernelGGL(gather_chunk_kernel, dim3(gx, (unsigned)p.S), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_fa(const FAParams &p, int max_q_len, bool causal, int mode, bool final_,
                     hipStream_t stream) {
    if (max_q_len <= 0 || p.S <= 0) return hipSuccess;
    const dim3 grid((unsigned)((max_q_len + kBM - 1) / kBM), (unsigned)p.Hq, (unsigned)p.S);
    // hi / lo weights everywhere: a single bf16 rounding of the weights
    // misses the output tolerance when a few keys dominate (short contexts,
    // the first causal rows, small chunks)
#define PA_FA(C, M, F) hipLaunchKernelGGL((fa_kernel<C, M, F, true>), grid, dim3(256), 0, stream, p)
    if (causal) {
        if (mode == 0) { if (final_) PA_FA(true, 0, true); else PA_FA(true, 0, false); }
        else { if (final_) PA_FA(true, 1, true); else PA_FA(true, 1, false); }
    } else {
        if (mode == 0) { if (final_) PA_FA(false, 0, true); else PA_FA(false, 0, false); }
        else { if (final_) PA_FA(false, 1, true); else PA_FA(false, 1, false); }
    }
#undef PA_FA
    return hipGetLastError();
}

}  // namespace pa
