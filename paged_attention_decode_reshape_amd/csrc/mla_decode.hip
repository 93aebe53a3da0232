// Absorbed MLA paged decode attention over the latent cache.
//
// In absorbed MLA every query head attends over the same per-token latent
// ("ROCm attention backends" blog, MLA section: decode runs directly on the
// compressed 576-wide latent, 512 no-rope + 64 rope dims, and keeps the
// cache in that form): the key of token t is its whole latent row c_t and
// the value is the row's first 512 entries, so
//   out_h = sum_t softmax_t(scale * q_h . c_t) * c_t[0:512].
// A latent row (1152 bytes) is read from HBM once and used by all heads.
//
// Work unit: one workgroup of 4 waves per (partition, sequence), all query
// heads together; wave w owns heads 4w .. 4w + 3 for QK, softmax and PV, so
// the waves never merge with each other.  The partition's tokens go through
// LDS 32 at a time: the workgroup loads a tile of latent rows (rows padded
// to 1168 bytes so that 8 lanes reading 8 rows at one column hit distinct
// banks), and the next tile's loads are in flight while the current one is
// used.
//   QK  lane (half f, token t): the 288 latent dims of half f of token t's
//       row, against query dwords broadcast by DPP from registers that stay
//       resident (9 per head); one permlane swap adds the halves.
//   PV  lane l: output dims 8l .. 8l + 7; per token one 16-byte LDS read of
//       its latent and one of its 4 heads' weights (which the token's lane
//       wrote to LDS: a broadcast read, so the FMAs take plain registers),
//       fp32 FMAs.
// Two ways to split the sequences over workgroups: fixed-length partitions
// (one workgroup per (partition, sequence)) or the balanced split (a grid of
// the resident workgroups, each sequence cut into pieces proportional to its
// length, as for GQA decode).  A sequence split over several workgroups
// writes fp32 partials (normalised output, LSE); the last workgroup of the
// sequence to finish merges them by log-sum-exp in token order.
#include <type_traits>

#include "common.h"
#include "decode_common.h"
#include "fp8.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kDl = 576;                  // latent width (keys)
constexpr int kDv = 512;                  // value width
constexpr int kWaves = 4;
constexpr int kHPW = 4;                   // heads per wave
constexpr int kTile = 32;                 // tokens per LDS tile
constexpr int kRowDw = kDl / 2 + 4;       // LDS row stride in dwords (1168 bytes)
constexpr int kHalfDw = kDl / 4;          // dwords per half row (144)
constexpr int kSlices = kHalfDw / 16;     // 16-dword query slices per half (9)
constexpr int kRowVec = kDl / 8;          // 16-byte vectors per latent row (72)
constexpr int kLoadVec = kTile * kRowVec / 256;  // vectors each thread loads per tile (9)
constexpr int kMaxPartition = 4096;       // tokens per partition, at most
constexpr int kPVAhead = 2;               // P.V: tokens whose V rows are read ahead
constexpr float kLazyLog2 = 8.f;          // softmax reference lag (log2 units)

// context length limited to the host's bound and what the block table covers
__device__ __forceinline__ int clamp_ctx(const MLAParams &p, int ctx) {
    const int64_t cap = min((int64_t)p.max_blocks * p.B, (int64_t)p.max_ctx);
    return ctx < 0 ? 0 : ((int64_t)ctx > cap ? (int)cap : ctx);
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), unrolled
template <typename F, int... E>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, E...>) {
    (f(std::integral_constant<int, E>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Max over the 16 lanes of each row (v must not be NaN).
__device__ __forceinline__ float row_max16(float v) {
    int k = f2ord(v);
    k = max(k, dpp_i<kQuadXor1>(k));
    k = max(k, dpp_i<kQuadXor2>(k));
    k = max(k, dpp_i<kRowRor4>(k));
    k = max(k, dpp_i<kRowRor8>(k));
    return ord2f(k);
}

// Log-sum-exp merge of a sequence's partials (in token order), by the
// workgroup that finished last.  Partial k of head h sits at
// po + h * hs + k * ks (floats, rows of 512 stored as 16-byte vectors
// v = 64 i + lane holding dims 8 lane + 4 i .. + 3) with its LSE at
// pl + h * lhs + k * lks; `extent` floats from po are readable.  Thread ->
// (head tid / 16, vectors 16 k + tid % 16, k < 8); 4 partials per round trip.
__device__ __forceinline__ void merge_mla_partials(const MLAParams &p, int s, const float *po,
                                                   size_t hs, size_t ks, uint32_t extent,
                                                   const float *pl, size_t lhs, size_t lks,
                                                   int nparts) {
    constexpr int kBatch = 4;
    const int h = threadIdx.x >> 4, c = threadIdx.x & 15;
    if (h >= p.Hq) return;
    const size_t row = (size_t)s * p.Hq + h;
    const auto rs = coherent_rsrc(po, extent * 4);
    float M = kNegInf, den = 0.f, o[8][4];
#pragma unroll
    for (int k = 0; k < 8; k++)
#pragma unroll
        for (int e = 0; e < 4; e++) o[k][e] = 0.f;
    for (int b = 0; b < nparts; b += kBatch) {
        float L[kBatch];
        float4 x[kBatch][8];
#pragma unroll
        for (int u = 0; u < kBatch; u++) {
            const int pu = b + u < nparts ? b + u : b;  // always an in-range address
            L[u] = load_coherent(&pl[h * lhs + pu * lks]);
            const uint32_t base = (uint32_t)(h * hs + pu * ks);
#pragma unroll
            for (int k = 0; k < 8; k++) x[u][k] = load_coherent4(rs, (base + 4 * (16 * k + c)) * 4);
        }
#pragma unroll
        for (int u = 0; u < kBatch; u++)
            if (b + u >= nparts) L[u] = kNegInf;
        float Mb = M;
#pragma unroll
        for (int u = 0; u < kBatch; u++) Mb = fmax_nc(Mb, L[u]);
        const float Mr = Mb == kNegInf ? 0.f : Mb;
        const float r = fast_exp2((M - Mr) * kLog2e);
        den *= r;
#pragma unroll
        for (int k = 0; k < 8; k++)
#pragma unroll
            for (int e = 0; e < 4; e++) o[k][e] *= r;
#pragma unroll
        for (int u = 0; u < kBatch; u++) {
            const float w = fast_exp2((L[u] - Mr) * kLog2e);
            den += w;
#pragma unroll
            for (int k = 0; k < 8; k++) {
                o[k][0] += w * x[u][k].x;
                o[k][1] += w * x[u][k].y;
                o[k][2] += w * x[u][k].z;
                o[k][3] += w * x[u][k].w;
            }
        }
        M = Mb;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    uint16_t *out = reinterpret_cast<uint16_t *>(p.out) + row * kDv;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const int v = 16 * k + c, d = 8 * (v & 63) + 4 * (v >> 6);  // vector v -> its 4 dims
        uint2 w;
        w.x = pack_bf16x2(o[k][0] * inv, o[k][1] * inv);
        w.y = pack_bf16x2(o[k][2] * inv, o[k][3] * inv);
        *reinterpret_cast<uint2 *>(out + d) = w;
    }
    if (c == 0 && p.lse) p.lse[row] = den > 0.f ? M + fast_log2(den) * kLn2 : kNegInf;
}

// Fused cache write of one decode token's latent (reshape_and_cache, MLA
// layout: the row of slot = block * B + o is kv_cache[block][o][0..576)),
// by the workgroup that reads the sequence's last token: threads 0..71 copy
// the 72 16-byte vectors, the stores complete and the workgroup meets at a
// barrier before any wave reads the cache.  Called by every thread.
// FP8 cache: threads 0..35 quantise 16 values each into one vector of codes.
template <bool F8>
__device__ __forceinline__ void mla_write_new_token(const MLAParams &p, int s) {
    const int64_t slot = as_const<int64_t>(p.slot_mapping)[s];
    if constexpr (F8) {
        constexpr int kRowVec8 = kDl / kFp8X;  // 36
        if (slot >= 0 && slot < p.num_blocks * p.B && (int)threadIdx.x < kRowVec8) {
            const uint4 *src = reinterpret_cast<const uint4 *>(p.new_latent) +
                               (size_t)s * kRowVec + 2 * threadIdx.x;
            reinterpret_cast<uint4 *>(const_cast<void *>(p.kv_cache))[(size_t)slot * kRowVec8 +
                                                                      threadIdx.x] =
                quantize16(src[0], src[1], p.kv_inv);
            wait_stores();
        }
        __syncthreads();
        return;
    }
    if (slot >= 0 && slot < p.num_blocks * p.B && (int)threadIdx.x < kRowVec) {
        const uint4 v = reinterpret_cast<const uint4 *>(p.new_latent)[(size_t)s * kRowVec + threadIdx.x];
        reinterpret_cast<uint4 *>(const_cast<void *>(p.kv_cache))[(size_t)slot * kRowVec + threadIdx.x] = v;
        wait_stores();
    }
    __syncthreads();
}

struct MLASmem {
    __align__(16) uint32_t tile[kTile * kRowDw];
    // latent row of every token of the current window (-1: past the end or
    // an out-of-range block id), resolved once per window so that the tile
    // loop issues no dependent block-table reads
    int32_t row[kMaxPartition];
    // P.V weights of each wave's 4 heads for the tile's tokens (written and
    // read by the same wave only)
    float4 w[kWaves][kTile];
};

// Query registers of the wave's heads (past num_q_heads: repeats of real
// heads, not stored): slice k of head j, lane n of a row of half f holds
// dword 144 f + 16 k + n of the head's query.
__device__ __forceinline__ void mla_load_queries(const MLAParams &p, int s,
                                                 uint32_t (&qreg)[kHPW][kSlices]) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, col = lane & 15, hf = lane >> 5;
#pragma unroll
    for (int j = 0; j < kHPW; j++) {
        const int head = (kHPW * wave + j) % p.Hq;
        const uint32_t *qh = reinterpret_cast<const uint32_t *>(p.query) +
                             ((size_t)s * p.Hq + head) * (kDl / 2) + kHalfDw * hf + col;
#pragma unroll
        for (int k = 0; k < kSlices; k++) qreg[j][k] = qh[16 * k];
    }
}

// Attention of the wave's heads over tokens [start, end) of sequence s,
// accumulated into (m, lsum, acc): windows of at most kMaxPartition tokens
// whose latent rows are resolved into LDS, then 32-token tiles.
template <bool F8>
__device__ __forceinline__ void mla_attend(const MLAParams &p, MLASmem &sm, int s, int start,
                                           int end, const uint32_t (&qreg)[kHPW][kSlices],
                                           float (&m)[kHPW], float (&lsum)[kHPW],
                                           float (&acc)[kHPW][8]) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int hf = lane >> 5;  // QK: half of the latent row
    const int tk = lane & 31;  // QK: token of the tile
    const float sl2 = p.scale * kLog2e * (F8 ? p.kv_scale : 1.f);
    const uint4 *kv = reinterpret_cast<const uint4 *>(p.kv_cache);
    const uint2 *kv8 = reinterpret_cast<const uint2 *>(p.kv_cache);  // FP8: 8 codes per uint2
    const int ld_tok = 8 * wave + (lane >> 3), ld_vec = lane & 7;

    for (int w0 = start; w0 < end; w0 += kMaxPartition) {
        const int wend = min(w0 + kMaxPartition, end);
        __syncthreads();  // the previous window's rows and tile are no longer read
        for (int i = threadIdx.x; i < wend - w0; i += kWaves * 64) {
            const int t = w0 + i;
            const int b = p.block_table[(size_t)s * p.max_blocks + t / p.B];
            sm.row[i] = b >= 0 && (int64_t)b < p.num_blocks ? b * p.B + t % p.B : -1;
        }
        // Tile loader: thread (wave w, lane) moves vectors (lane & 7) + 8 i of
        // the latent row of tile token 8 w + (lane >> 3); tokens past the end
        // (or with an out-of-range block id) become zero rows.
        // FP8: the same 16-byte bf16 vectors come from 8 codes each (half a
        // 16-code vector), converted exactly on the way to LDS.
        auto load_tile = [&](int t0, uint4 (&r)[kLoadVec]) {
            const int t = t0 + ld_tok;
            const int rowi = t < wend ? sm.row[t - w0] : -1;
            if constexpr (F8) {
                const uint2 *src = kv8 + (size_t)(rowi < 0 ? 0 : rowi) * (kDl / 8) + ld_vec;
#pragma unroll
                for (int i = 0; i < kLoadVec; i++) {
                    const uint2 c = rowi < 0 ? make_uint2(0, 0) : src[8 * i];
                    fp8x4_to_bf16x2(c.x, r[i].x, r[i].y);
                    fp8x4_to_bf16x2(c.y, r[i].z, r[i].w);
                }
            } else {
                const uint4 *src = kv + (size_t)(rowi < 0 ? 0 : rowi) * kRowVec + ld_vec;
#pragma unroll
                for (int i = 0; i < kLoadVec; i++)
                    r[i] = rowi < 0 ? make_uint4(0, 0, 0, 0) : src[8 * i];
            }
        };
        auto store_tile = [&](const uint4 (&r)[kLoadVec]) {
            uint4 *dst = reinterpret_cast<uint4 *>(&sm.tile[ld_tok * kRowDw]) + ld_vec;
#pragma unroll
            for (int i = 0; i < kLoadVec; i++) dst[8 * i] = r[i];
        };
        // validity of QK token tk of the tile starting at t0 (same test as the loader)
        auto token_ok = [&](int t0) {
            const int t = t0 + tk;
            return t < wend && sm.row[t - w0] >= 0;
        };

        __syncthreads();  // rows complete
        uint4 next[kLoadVec];
        load_tile(w0, next);
        for (int t0 = w0; t0 < wend; t0 += kTile) {
            __syncthreads();  // the previous tile is no longer read
            store_tile(next);
            const bool tok_ok = token_ok(t0);
            __syncthreads();

            // QK: half f of the row of token tk against the wave's heads
            float za[kHPW], zb[kHPW];
#pragma unroll
            for (int j = 0; j < kHPW; j++) za[j] = zb[j] = 0.f;
            const uint4 *kr = reinterpret_cast<const uint4 *>(&sm.tile[tk * kRowDw + kHalfDw * hf]);
#pragma unroll
            for (int k = 0; k < kSlices; k++) {
                const uint4 k0 = kr[4 * k], k1 = kr[4 * k + 1], k2 = kr[4 * k + 2], k3 = kr[4 * k + 3];
#pragma unroll
                for (int j = 0; j < kHPW; j++) qk16<false>(za[j], zb[j], qreg[j][k], k0, k1, k2, k3);
            }
            dpp_result_fence<kHPW>(za);
            dpp_result_fence<kHPW>(zb);
            // softmax: the tile's exact max; the reference maximum m moves only
            // when the tile's passes it by more than 8 (log2 units), so weights
            // stay <= 2^8 and most tiles skip the rescale of the running state
            float pw[kHPW];
#pragma unroll
            for (int j = 0; j < kHPW; j++) {
                const float z = za[j] + zb[j];
                const auto zz = __builtin_amdgcn_permlane32_swap(__float_as_uint(z), __float_as_uint(z),
                                                                 false, false);
                const float sc = tok_ok ? (__uint_as_float(zz[0]) + __uint_as_float(zz[1])) * sl2 : kNegInf;
                const float rm = row_max16(sc);
                const auto mm = __builtin_amdgcn_permlane16_swap(__float_as_uint(rm),
                                                                 __float_as_uint(rm), false, false);
                const float mx = uniform_f(fmax_nc(__uint_as_float(mm[0]), __uint_as_float(mm[1])));
                if (mx > m[j] + kLazyLog2) {  // uniform
                    const float alpha = fast_exp2(m[j] - mx);
                    m[j] = mx;
                    lsum[j] *= alpha;
#pragma unroll
                    for (int i = 0; i < 8; i++) acc[j][i] *= alpha;
                }
                const float mref = m[j] == kNegInf ? 0.f : m[j];
                pw[j] = fast_exp2(sc - mref);
                lsum[j] += pw[j];
            }
            // the next tile's loads overlap P.V (issued after QK, so their
            // registers are not live during QK)
            if (t0 + kTile < wend) load_tile(t0 + kTile, next);
            // PV: dims 8 lane .. 8 lane + 7 of every token of the tile; the
            // LDS reads run kPVAhead tokens ahead of their use
            const uint4 *vr = reinterpret_cast<const uint4 *>(sm.tile) + lane;
            // token lane t publishes its weights; every lane reads them back
            if (lane < kTile) sm.w[wave][lane] = make_float4(pw[0], pw[1], pw[2], pw[3]);
            float4 wbuf[kPVAhead];
            static_for<kPVAhead>([&](auto u_c) {
                constexpr int u = decltype(u_c)::value;
                wbuf[u] = sm.w[wave][u];
            });
            uint4 vbuf[kPVAhead];
            static_for<kPVAhead>([&](auto u_c) {
                constexpr int u = decltype(u_c)::value;
                vbuf[u] = vr[u * (kRowDw / 4)];
            });
            static_for<kTile>([&](auto t_c) {
                constexpr int t = decltype(t_c)::value;
                const uint4 v = vbuf[t % kPVAhead];
                const float4 wt = wbuf[t % kPVAhead];
                if constexpr (t + kPVAhead < kTile) {
                    vbuf[t % kPVAhead] = vr[(t + kPVAhead) * (kRowDw / 4)];
                    wbuf[t % kPVAhead] = sm.w[wave][t + kPVAhead];
                }
                const float wts[4] = {wt.x, wt.y, wt.z, wt.w};
                const float vf[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                                     bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
                for (int j = 0; j < kHPW; j++) {
                    const float w = wts[j];
#pragma unroll
                    for (int i = 0; i < 8; i++) acc[j][i] = __builtin_fmaf(w, vf[i], acc[j][i]);
                }
            });
        }
    }
    if constexpr (F8) {  // the value rows were summed as unscaled codes
#pragma unroll
        for (int j = 0; j < kHPW; j++)
#pragma unroll
            for (int i = 0; i < 8; i++) acc[j][i] *= p.kv_scale;
    }
}

// Normalise the wave's heads and write them: as output rows (whole = true)
// or as partials at po + h * hs (floats) with LSEs at pl + h * lhs.
__device__ __forceinline__ void mla_emit(const MLAParams &p, int s, bool whole,
                                         const float (&m)[kHPW], const float (&lsum)[kHPW],
                                         const float (&acc)[kHPW][8], float *po, size_t hs,
                                         float *pl, size_t lhs) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    uint16_t *out = reinterpret_cast<uint16_t *>(p.out);
    // lanes 32-63 repeat the weights of 0-31
    float L[kHPW], inv[kHPW];
#pragma unroll
    for (int j = 0; j < kHPW; j++) {
        const float l = wave_sum(lsum[j]) * 0.5f;
        inv[j] = l > 0.f ? 1.f / l : 0.f;
        L[j] = l > 0.f ? (m[j] + fast_log2(l)) * kLn2 : kNegInf;
    }
#pragma unroll
    for (int j = 0; j < kHPW; j++) {
        const int h = kHPW * wave + j;
        if (h >= p.Hq) continue;
        const size_t orow = (size_t)s * p.Hq + h;
        if (whole) {
            uint4 o;
            o.x = pack_bf16x2(acc[j][0] * inv[j], acc[j][1] * inv[j]);
            o.y = pack_bf16x2(acc[j][2] * inv[j], acc[j][3] * inv[j]);
            o.z = pack_bf16x2(acc[j][4] * inv[j], acc[j][5] * inv[j]);
            o.w = pack_bf16x2(acc[j][6] * inv[j], acc[j][7] * inv[j]);
            reinterpret_cast<uint4 *>(out + orow * kDv)[lane] = o;
            if (lane == 0 && p.lse) p.lse[orow] = L[j];
        } else {
            // partial row stored as 16-byte vectors v = 64 i + lane (dims
            // 8 lane + 4 i .. + 3), so each store instruction writes 1 KB
            const auto rs = coherent_rsrc(po + h * hs, kDv * 4);
#pragma unroll
            for (int i = 0; i < 2; i++)
                store_coherent4(rs, (64 * i + lane) * 16, acc[j][4 * i] * inv[j],
                                acc[j][4 * i + 1] * inv[j], acc[j][4 * i + 2] * inv[j],
                                acc[j][4 * i + 3] * inv[j]);
            if (lane == 0) store_coherent(&pl[h * lhs], L[j]);
        }
    }
}

// Counts one finished piece of sequence s; true in the workgroup that
// finished last (which then merges).  Each thread first waits for its
// partial stores to complete.  The last workgroup leaves the counter zero.
__device__ __forceinline__ bool mla_count(const MLAParams &p, int s, int nparts) {
    __shared__ int sm_last;
    wait_stores();
    __syncthreads();
    int *counter = p.counters + s;
    if (threadIdx.x == 0) {
        const int prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm_last = prev == nparts - 1;
        if (prev == nparts - 1) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return sm_last;
}

__device__ __forceinline__ void mla_write_empty(const MLAParams &p, int s) {
    uint16_t *out = reinterpret_cast<uint16_t *>(p.out);
    for (int idx = threadIdx.x; idx < p.Hq * kDv; idx += kWaves * 64) {
        out[((size_t)s * p.Hq + idx / kDv) * kDv + idx % kDv] = 0;
        if (idx % kDv == 0 && p.lse) p.lse[(size_t)s * p.Hq + idx / kDv] = kNegInf;
    }
}

// ---------------------------------------------------------------------------
// Matrix-core engine.  The 16 query heads over one shared latent make QK a
// dense [16 x 576] x [576 x T] product and P.V a [16 x T] x [T x 512] one,
// computed with v_mfma_f32_16x16x32_bf16 (QK, 18 steps of 32 dims per 16
// tokens) and v_mfma_f32_16x16x16_bf16 (P.V, P in bf16 hi + lo parts).  A
// workgroup of 4 waves walks its range 64 tokens at a time (a round); wave w
// owns tokens 16 w .. 16 w + 15 of each round and never exchanges data with
// the other waves until the final merge.
//   load  each lane of a wave gathers 16-byte vectors of its own token's
//         latent row (lane (g, m): token m, vectors 4 j + g) straight into
//         one of the wave's two stage buffers (global_load_lds: per-lane
//         64-bit addresses, so any pool size and block size): block j holds,
//         at slot 16 g + m, vector 4 j + g of token m.  The next round's
//         gather is in flight while the current round is computed; the two
//         stages are separate LDS objects, so a read of one need not wait
//         for a gather into the other.
//   QK    S^T = K Q^T: A = the 16 tokens' latents, B = the queries (resident
//         registers: lane (g, m) holds head m's dims 32 j + 8 g .. + 7);
//         lane (g, m) then holds head m's scores of tokens 4 g .. 4 g + 3.
//   P.V   O = P V: A = P (lane (g, m): head m, tokens 4 g .. 4 g + 3, i.e.
//         the lane's own weights), B = V through LDS transpose reads; 32
//         output tiles of 16 dims, whose accumulators (lane (g, n): heads
//         4 g .. 4 g + 3, dim 16 N + n) stay in registers.
// bf16 latents: 18 blocks (18 KB) per stage, 144 KB of stages per workgroup
// (one workgroup per compute unit); operand j of QK is one conflict-free
// 1 KB read of block j; the P.V operand of tile N comes from
// ds_read_b64_tr_b16 (within 16 lanes, lane 4 k + q reads token 4 g + k,
// dims 4 q .. 4 q + 3 of the tile, and lane n receives dim n of the 4
// tokens).
// FP8 latents (576 codes a row): 9 blocks (9 KB) per stage, 72 KB per
// workgroup (two per compute unit); codes are widened to bf16 in registers
// (exact: every E4M3 value is a bf16): the QK operand of step j is 8 codes
// (one 64-bit read) of dims 32 j + 8 g .. + 7; the B operands of tiles N
// and N + 1 (N even) come from one ds_read_b64_tr_b8 (within 16 lanes,
// lane 2 b + h gives the address of row b, lane n receives byte n of every
// row) whose row b is token 4 g + b % 4 at dims 16 (N + b / 4) + 8 h .. + 7,
// so lane (g, n) receives dim 16 N + n (first word) and 16 (N + 1) + n
// (second word) of tokens 4 g .. 4 g + 3; the cache scale folds into the
// softmax scale and the output.
// Every round issues exactly one block-table load (for two rounds ahead,
// index clamped) and one gather load per stage block, so "all but the
// newest (blocks + 1) vector memory operations are done" means the current
// round has landed.  Lanes whose token is past the end (or whose block id
// is out of range) gather a stand-in in-pool row; their scores are masked
// and their values zeroed before the P.V products.  Online softmax with the
// lazy reference of the VALU engine.  Query heads beyond num_q_heads are
// zero rows whose outputs are not written.
// ---------------------------------------------------------------------------
constexpr int kMTok = 16;              // tokens per wave per round
constexpr int kMRound = kWaves * kMTok;  // 64 tokens per round
constexpr int kMSteps = kDl / 32;      // 18 QK steps
constexpr int kMTiles = kDv / 16;      // 32 output tiles of 16 dims
constexpr int kMMergeDims = 256;       // output dims merged per pass

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Workgroup state of the matrix-core engine besides its stage buffers.
struct MLAMfmaSmem {
    float m[kWaves][16], l[kWaves][16];
    float alpha[kWaves][16];  // rescale factors of the wave's heads (lazy softmax)
};
template <bool F8, bool MFMA>
using MLASmemOf = std::conditional_t<MFMA, MLAMfmaSmem, MLASmem>;
typedef int v2i32_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4 &v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

// Query operand registers: lane (g, m), step j: dims 32 j + 8 g .. + 7 of head m
// (zero for heads >= num_q_heads).
__device__ __forceinline__ void mla_mfma_queries(const MLAParams &p, int s, uint4 (&q)[kMSteps]) {
    const int lane = threadIdx.x & 63, g = lane >> 4, m = lane & 15;
    const uint4 *qh = reinterpret_cast<const uint4 *>(p.query) + ((size_t)s * p.Hq + min(m, p.Hq - 1)) * kRowVec;
#pragma unroll
    for (int j = 0; j < kMSteps; j++) q[j] = m < p.Hq ? qh[4 * j + g] : make_uint4(0, 0, 0, 0);
}

// Latent row of token t of sequence s (-1: past `end` or an out-of-range block id).
__device__ __forceinline__ int64_t mla_row(const MLAParams &p, int s, int t, int end) {
    if (t >= end) return -1;
    const int b = p.block_table[(size_t)s * p.max_blocks + min(t / p.B, p.max_blocks - 1)];
    return b >= 0 && (int64_t)b < p.num_blocks ? (int64_t)b * p.B + t % p.B : -1;
}

// Merge of the 4 waves of a matrix-core workgroup and the output: each
// wave's accumulators (lane (g, n): heads 4 g .. 4 g + 3, dim 16 N + n of tile
// N), reference maxima (mh, head m) and weight sums (lsum, lane's share of
// head m) are combined by log-sum-exp, written as output rows (whole) or as
// partials at po + h * hs (16-byte vector 64 i + c holding dims 8 c + 4 i ..
// + 3) with LSEs at pl + h * lhs.  The output dims go through LDS in passes of
// kMMergeDims; obuf(w) is wave w's [16][kMMergeDims + 4] float area.
template <typename OBuf>
__device__ __forceinline__ void mla_mfma_emit(const MLAParams &p, int s, bool whole, float *po,
                                              size_t hs, float *pl, size_t lhs,
                                              const f32x4_t (&o)[kMTiles], float mh, float lsum,
                                              float (&sm_m)[kWaves][16],
                                              float (&sm_l)[kWaves][16], OBuf obuf) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, m = lane & 15;
    {  // weight sums of head m over the 4 rows of lanes
        auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
        float l2 = __uint_as_float(x[0]) + __uint_as_float(x[1]);
        auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(l2), __float_as_uint(l2), false, false);
        lsum = __uint_as_float(y[0]) + __uint_as_float(y[1]);
    }
    lds_barrier();  // every wave is done with the LDS that obuf reuses
    if (g == 0) {
        sm_m[wave][m] = mh;
        sm_l[wave][m] = lsum;
    }
    uint16_t *out = reinterpret_cast<uint16_t *>(p.out);
    // partials of all heads through one descriptor made outside the loops
    // (a per-head descriptor is per-lane to the compiler, which then wraps
    // each store in a loop over distinct descriptors)
    const auto prs = coherent_rsrc(po, whole ? 0u : (uint32_t)(((p.Hq - 1) * hs + kDv) * 4));
    constexpr int kStride = kMMergeDims + 4;
    float *mine = obuf(wave);
    for (int pass = 0; pass < kDv / kMMergeDims; pass++) {
        constexpr int kTilesPerPass = kMMergeDims / 16;
#pragma unroll
        for (int n = 0; n < kTilesPerPass; n++)
#pragma unroll
            for (int i = 0; i < 4; i++) mine[(4 * g + i) * kStride + 16 * n + m] = o[kTilesPerPass * pass + n][i];
        lds_barrier();
        // a wave's 64 consecutive indices share one head (the bound is a
        // multiple of 64)
        for (int idx = threadIdx.x; idx < p.Hq * (kMMergeDims / 4); idx += kWaves * 64) {
            const int h = __builtin_amdgcn_readfirstlane(idx / (kMMergeDims / 4));
            const int d = 4 * (idx % (kMMergeDims / 4));
            float M = kNegInf;
#pragma unroll
            for (int w = 0; w < kWaves; w++) M = fmax_nc(M, sm_m[w][h]);
            const float Mr = M == kNegInf ? 0.f : M;
            float acc[4] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; w++) {
                const float wt = fast_exp2(sm_m[w][h] - Mr);
                const float4 a = *reinterpret_cast<const float4 *>(obuf(w) + h * kStride + d);
                acc[0] += wt * a.x;
                acc[1] += wt * a.y;
                acc[2] += wt * a.z;
                acc[3] += wt * a.w;
                den += wt * sm_l[w][h];
            }
            const float inv = den > 0.f ? 1.f / den : 0.f;
            const float L = den > 0.f ? (M + fast_log2(den)) * kLn2 : kNegInf;
            const int dim = kMMergeDims * pass + d;
            const size_t orow = (size_t)s * p.Hq + h;
            if (whole) {
                uint2 v;
                v.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
                v.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
                *reinterpret_cast<uint2 *>(out + orow * kDv + dim) = v;
                if (dim == 0 && p.lse) p.lse[orow] = L;
            } else {
                // vector 64 i + c holds dims 8 c + 4 i .. + 3
                const int vec = 64 * ((dim & 7) >> 2) + (dim >> 3);
                store_coherent4(prs, (uint32_t)(h * hs * 4 + vec * 16), acc[0] * inv,
                                acc[1] * inv, acc[2] * inv, acc[3] * inv);
                if (dim == 0) store_coherent(&pl[h * lhs], L);
            }
        }
        // the pass's LDS is read before the next one is written (its partial
        // stores stay in flight: the count that publishes them waits for them)
        lds_barrier();
    }
}

// Stage blocks of 64 16-byte vectors per wave and round: 9 of codes, 18 of bf16.
template <bool F8>
constexpr int kStageBlocks = F8 ? kDl / 64 : kDl / 32;

template <bool F8>
struct MfmaStage {
    __align__(16) uint4 t[kWaves][kStageBlocks<F8>][64];
};

// "All but the newest n vector memory operations have completed."
#define PA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

// Attention of all heads over tokens [start, end) of sequence s, then the
// merge of the 4 waves and the output (mla_mfma_emit).
template <bool F8>
__device__ __forceinline__ void mla_mfma_piece(const MLAParams &p, MLAMfmaSmem &sm, int s,
                                                  int start, int end, bool whole, float *po,
                                                  size_t hs, float *pl, size_t lhs) {
    // two objects: a read of one need not wait for a gather into the other
    __shared__ MfmaStage<F8> st0, st1;
    constexpr int kLoads = kStageBlocks<F8>;  // gather loads per round
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, m = lane & 15;
    const float sl2 = p.scale * kLog2e * (F8 ? p.kv_scale : 1.f);
    const char *kv = reinterpret_cast<const char *>(p.kv_cache);
    char *const b0 = reinterpret_cast<char *>(&st0.t[wave][0][0]);
    char *const b1 = reinterpret_cast<char *>(&st1.t[wave][0][0]);
    const int nr = end > start ? (end - start + kMRound - 1) / kMRound : 0;  // rounds of the piece
    const int32_t *bt = p.block_table + (size_t)s * p.max_blocks;

    // the lane's token in round r, its block-table entry (always loaded: the
    // index is clamped) and its latent row (-1: no token)
    auto token = [&](int r) { return start + kMRound * r + kMTok * wave + m; };
    auto entry = [&](int r) {
        const int t = min(token(r), end - 1);
        return bt[min(t / p.B, p.max_blocks - 1)];
    };
    auto row_of = [&](int r, int b) -> int64_t {
        const int t = token(r);
        return t < end && b >= 0 && (int64_t)b < p.num_blocks ? (int64_t)b * p.B + t % p.B : -1;
    };
    auto gather = [&](char *stage, int64_t row) {
        const char *src = kv + (size_t)(row < 0 ? 0 : row) * (F8 ? kDl : 2 * kDl) + 16 * g;
#pragma unroll
        for (int j = 0; j < kLoads; j++)
            __builtin_amdgcn_global_load_lds(src + 64 * j, (lds_void_t *)(stage + 1024 * j), 16, 0, 0);
    };

    // FP8 QK operand of steps j, j + 1 (j even): vector 2 j + g / 2 (+ 2),
    // i.e. block j / 2, slot 16 (g / 2) (+ 32) + m, half g % 2
    const int qk_off = (16 * (g >> 1) + m) * 16 + 8 * (g & 1);
    // FP8 transpose row (tb) and half (th) of the lane: tile pair N, N + 1
    // (N even) reads vector N + tb / 4 of token 4 g + tb % 4
    const int tb = (lane & 15) >> 1, th = lane & 1;
    const int tr_tok = 4 * g + (tb & 3);
    // bf16 transpose read of tile N: lane (g, 4 k + q) reads token 4 g + k,
    // dims 4 q .. 4 q + 3 (vector 2 N + q / 2, half q % 2)
    const int kq = lane & 15, tk = 4 * g + (kq >> 2), qd = kq & 3;

    uint4 q[kMSteps];
    f32x4_t o[kMTiles];
#pragma unroll
    for (int n = 0; n < kMTiles; n++) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float mh = kNegInf, lsum = 0.f;

    int e1 = 0;  // entry of round r + 1
    int64_t row = -1;
    if (nr > 0) {
        row = row_of(0, entry(0));
        e1 = entry(min(1, nr - 1));
        gather(b0, row);
        mla_mfma_queries(p, s, q);
    }
    // one round; which stage is current is a compile-time fact, so that the
    // compiler can tell the stage read from the one being gathered into
    auto round = [&](int r, auto in_st0) {
        constexpr bool kSt0 = decltype(in_st0)::value;
        char *cur = kSt0 ? b0 : b1;
        char *nxt = kSt0 ? b1 : b0;
        const uint32_t valid = (uint32_t)__ballot(row >= 0) & 0xffffu;
        int64_t row1 = -1;
        asm volatile("" ::: "memory");
        if (r + 1 < nr) {
            // the next round: its entry is in (loaded before this round's
            // gather), the one after is requested first
            PA_WAIT_VM(kLoads);  // e1, loaded before the current round's gather
            asm volatile("" ::: "memory");
            const int e2 = entry(min(r + 2, nr - 1));
            row1 = row_of(r + 1, e1);
            gather(nxt, row1);
            e1 = e2;
            asm volatile("" ::: "memory");
            PA_WAIT_VM(kLoads + 1);
        } else {
            PA_WAIT_VM(0);
        }
        asm volatile("" ::: "memory");
        if (valid != 0) {
            // QK: two accumulator chains over the 18 steps
            f32x4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kMSteps; j += 2) {
                if constexpr (F8) {
                    uint4 ka, kb;
                    const char *base = cur + 1024 * (j / 2) + qk_off;
                    const uint2 ca = *reinterpret_cast<const uint2 *>(base);
                    const uint2 cb = *reinterpret_cast<const uint2 *>(base + 2 * 16 * 16);
                    fp8x4_to_bf16x2(ca.x, ka.x, ka.y);
                    fp8x4_to_bf16x2(ca.y, ka.z, ka.w);
                    fp8x4_to_bf16x2(cb.x, kb.x, kb.y);
                    fp8x4_to_bf16x2(cb.y, kb.z, kb.w);
                    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka), as_bf16x8(q[j]), sa, 0, 0, 0);
                    sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kb), as_bf16x8(q[j + 1]), sb, 0, 0, 0);
                } else if (j % 6 == 0) {
                    // six steps at a time: their operand reads are issued
                    // together (block j, slot lane: vector 4 j + g of token m)
                    uint4 kk[6];
#pragma unroll
                    for (int i = 0; i < 6; i++)
                        kk[i] = *reinterpret_cast<const uint4 *>(cur + 1024 * (j + i) + 16 * lane);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < 6; i += 2) {
                        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kk[i]), as_bf16x8(q[j + i]), sa, 0, 0, 0);
                        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kk[i + 1]), as_bf16x8(q[j + i + 1]), sb, 0, 0, 0);
                    }
                }
            }
            float z[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const bool ok = (valid >> (4 * g + i)) & 1u;
                z[i] = ok ? (sa[i] + sb[i]) * sl2 : kNegInf;
            }
            float zm = fmax_nc(fmax_nc(z[0], z[1]), fmax_nc(z[2], z[3]));
            {
                auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(zm), __float_as_uint(zm), false, false);
                zm = fmax_nc(__uint_as_float(x[0]), __uint_as_float(x[1]));
                auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(zm), __float_as_uint(zm), false, false);
                zm = fmax_nc(__uint_as_float(y[0]), __uint_as_float(y[1]));
            }
            if (__ballot(zm > mh + kLazyLog2)) {
                float alpha = 1.f;
                if (zm > mh + kLazyLog2) {
                    alpha = fast_exp2(mh - zm);  // 0 from -inf
                    mh = zm;
                }
                lsum *= alpha;
                if (g == 0) sm.alpha[wave][m] = alpha;
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the LDS writes have landed
                float a4[4];
#pragma unroll
                for (int i = 0; i < 4; i++) a4[i] = sm.alpha[wave][4 * g + i];
#pragma unroll
                for (int n = 0; n < kMTiles; n++)
#pragma unroll
                    for (int i = 0; i < 4; i++) o[n][i] *= a4[i];
            }
            float pw[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                pw[i] = fast_exp2(z[i] - mh);  // mh is finite here
                lsum += pw[i];
            }
            uint2 ph, pl_;
            ph.x = pack_bf16x2(pw[0], pw[1]);
            ph.y = pack_bf16x2(pw[2], pw[3]);
            pl_.x = pack_bf16x2(pw[0] - bf16_lo(ph.x), pw[1] - bf16_hi(ph.x));
            pl_.y = pack_bf16x2(pw[2] - bf16_lo(ph.y), pw[3] - bf16_hi(ph.y));
            const bf16x4_t pa = __builtin_bit_cast(bf16x4_t, ph), pb = __builtin_bit_cast(bf16x4_t, pl_);
            // values of tokens 4 g .. 4 g + 3 that are not this round's are
            // zeroed (the gathered stand-in row may hold any bits)
            const uint32_t nib = (valid >> (4 * g)) & 0xfu;
            if constexpr (F8) {
                const uint32_t bm = ((nib * 0x00204081u) & 0x01010101u) * 0xffu;  // byte k: token k
#pragma unroll
                for (int n = 0; n < kMTiles; n += 2) {
                    const int v = n + (tb >> 2);  // code vector of the lane's transpose row
                    const int off = (v >> 2) * 1024 + (16 * (v & 3) + tr_tok) * 16 + 8 * th;
                    const v2i32_t c = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) v2i32_t *)(cur + off));
                    uint2 w0, w1;
                    fp8x4_to_bf16x2((uint32_t)c[0] & bm, w0.x, w0.y);
                    fp8x4_to_bf16x2((uint32_t)c[1] & bm, w1.x, w1.y);
                    const bf16x4_t v0 = __builtin_bit_cast(bf16x4_t, w0), v1 = __builtin_bit_cast(bf16x4_t, w1);
                    o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, v0, o[n], 0, 0, 0);
                    o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pb, v0, o[n], 0, 0, 0);
                    o[n + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, v1, o[n + 1], 0, 0, 0);
                    o[n + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pb, v1, o[n + 1], 0, 0, 0);
                }
            } else {
                // 16-bit half k of the pair: token k (first word 0, 1; second 2, 3)
                const uint32_t hm0 = ((nib & 1u) ? 0xffffu : 0u) | ((nib & 2u) ? 0xffff0000u : 0u);
                const uint32_t hm1 = ((nib & 4u) ? 0xffffu : 0u) | ((nib & 8u) ? 0xffff0000u : 0u);
#pragma unroll
                for (int n0 = 0; n0 < kMTiles; n0 += 8) {  // 8 tiles' reads issued together
                    uint2 w[8];
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        const int v = 2 * (n0 + i) + (qd >> 1);
                        const int off = (v >> 2) * 1024 + (16 * (v & 3) + tk) * 16 + 8 * (qd & 1);
                        w[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4_t *)(cur + off)));
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        w[i].x &= hm0;
                        w[i].y &= hm1;
                        const bf16x4_t vb = __builtin_bit_cast(bf16x4_t, w[i]);
                        o[n0 + i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, o[n0 + i], 0, 0, 0);
                        o[n0 + i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pb, vb, o[n0 + i], 0, 0, 0);
                    }
                }
            }
        }
        // every LDS read of this round's stage is done before the gather two
        // rounds on overwrites it (the gather's LDS writes are not ordered
        // after reads)
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("" ::: "memory");
        row = row1;
    };
    for (int r = 0; r < nr; r += 2) {
        round(r, std::true_type{});
        if (r + 1 < nr) round(r + 1, std::false_type{});
    }
    if constexpr (F8) {  // the value rows were summed as unscaled codes
#pragma unroll
        for (int n = 0; n < kMTiles; n++)
#pragma unroll
            for (int i = 0; i < 4; i++) o[n][i] *= p.kv_scale;
    }

    // the stages, no longer read, hold each wave's pass of output dims:
    // waves 0, 1 in st0, 2, 3 in st1
    mla_mfma_emit(p, s, whole, po, hs, pl, lhs, o, mh, lsum, sm.m, sm.l, [&](int w) -> float * {
        return reinterpret_cast<float *>(w < 2 ? &st0 : &st1) + (w & 1) * 16 * (kMMergeDims + 4);
    });
}

__device__ __forceinline__ void mla_reset(float (&m)[kHPW], float (&lsum)[kHPW], float (&acc)[kHPW][8]) {
#pragma unroll
    for (int j = 0; j < kHPW; j++) {
        m[j] = kNegInf;
        lsum[j] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) acc[j][i] = 0.f;
    }
}

// Fixed partitions: one workgroup per (partition, sequence).
template <bool F8, bool MFMA>
__global__ __launch_bounds__(256, (MFMA && !F8) ? 1 : 2) void mla_decode_kernel(MLAParams p) {
    const int part = blockIdx.x / p.S;
    const int s = blockIdx.x - part * p.S;
    const int P = p.partition;
    const int start = part * P;
    __shared__ MLASmemOf<F8, MFMA> sm;

    const int ctx = clamp_ctx(p, as_const<int32_t>(p.context_lens)[s]);
    if (start >= ctx) {
        if (ctx == 0 && part == 0) {
            if (p.slot_mapping) mla_write_new_token<F8>(p, s);
            mla_write_empty(p, s);
        }
        return;
    }
    const int end = min(start + P, ctx);
    const int nparts = (ctx + P - 1) / P;
    // the partition holding the last token writes the new token first
    if (p.slot_mapping && end == ctx) mla_write_new_token<F8>(p, s);
    // partials [S, Hq, max_parts, Dv] and [S, Hq, max_parts]
    float *po = nparts == 1 ? nullptr : p.part_out + ((size_t)s * p.Hq * p.max_parts + part) * kDv;
    float *pl = nparts == 1 ? nullptr : p.part_lse + (size_t)s * p.Hq * p.max_parts + part;
    if constexpr (MFMA) {
        mla_mfma_piece<F8>(p, sm, s, start, end, nparts == 1, po, (size_t)p.max_parts * kDv,
                              pl, p.max_parts);
    } else {
        uint32_t qreg[kHPW][kSlices];
        mla_load_queries(p, s, qreg);
        float m[kHPW], lsum[kHPW], acc[kHPW][8];
        mla_reset(m, lsum, acc);
        mla_attend<F8>(p, sm, s, start, end, qreg, m, lsum, acc);
        mla_emit(p, s, nparts == 1, m, lsum, acc, po, (size_t)p.max_parts * kDv, pl, p.max_parts);
    }
    if (nparts == 1) return;
    if (!mla_count(p, s, nparts)) return;
    merge_mla_partials(p, s, p.part_out + (size_t)s * p.Hq * p.max_parts * kDv,
                       (size_t)p.max_parts * kDv, kDv, (uint32_t)p.Hq * p.max_parts * kDv,
                       p.part_lse + (size_t)s * p.Hq * p.max_parts, p.max_parts, 1, nparts);
}

// Inclusive prefix sum over the wave's lanes: Hillis-Steele inside each
// 16-lane row (DPP row shifts, zero shifted in), then rows 1 and 3 add the
// last lane of the row before (row_bcast:15) and rows 2 and 3 that of row 1
// (row_bcast:31).
__device__ __forceinline__ int wave_prefix_sum_i(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Balanced split: NW resident workgroups; every non-empty sequence (U of
// them, SB 32-token tiles in all) is cut into
//   n_s = min(nsb_s, 1 + floor(nsb_s (NW - U) / SB))   pieces if U <= NW,
// else one, numbered sequence-major; workgroup w takes piece w (+ NW, ...).
// Pieces P_u .. P_u + n - 1 of a sequence leave partials in those slots of
// [NW, Hq, Dv] and [NW, Hq]; the last to finish merges them in order.
template <bool F8, bool MFMA>
__global__ __launch_bounds__(256, (MFMA && !F8) ? 1 : 2) void mla_decode_balanced_kernel(MLAParams p) {
    const int NW = gridDim.x, w = blockIdx.x;
    const int lane = threadIdx.x & 63;
    __shared__ MLASmemOf<F8, MFMA> sm;
    auto ctx_of = [&](int s) { return s < p.S ? clamp_ctx(p, p.context_lens[min(s, p.S - 1)]) : 0; };
    const int ctx_w0 = ctx_of(lane);
    auto ctx_in = [&](int c0) { return c0 == 0 ? ctx_w0 : ctx_of(c0 + lane); };

    for (int s = w; s < p.S; s += NW)
        if (readlane_i32(ctx_in(s & ~63), s & 63) == 0) {
            if (p.slot_mapping) mla_write_new_token<F8>(p, s);
            mla_write_empty(p, s);
        }

    // pass 1 (every wave): tiles and non-empty sequences
    int64_t SB = 0;
    int U = 0;
    for (int c0 = 0; c0 < p.S; c0 += 64) {
        const int nsb = (ctx_in(c0) + kTile - 1) / kTile;
        SB += readlane_i32(wave_prefix_sum_i(nsb), 63);
        U += __popcll(__ballot(nsb > 0));
    }
    if (U == 0) return;
    const bool split = U <= NW;
    // when split, SB <= NW * 2^15 and the arithmetic fits 32 bits
    const uint32_t spare = split ? (uint32_t)(NW - U) : 0u, SB32 = split ? (uint32_t)SB : 1u;
    auto pieces_of = [&](int nsb) -> int {
        if (nsb == 0) return 0;
        if (!split) return 1;
        const uint32_t n = 1u + (uint32_t)nsb * spare / SB32;
        return n < (uint32_t)nsb ? (int)n : nsb;
    };

    for (int64_t v = w; ; v += NW) {
        // find piece v (every wave computes the same)
        int s = -1, k = 0, n = 1, a = 0, b = 0, ctx = 0, P_u = 0;
        int64_t base = 0;  // pieces of the sequences before window c0
        for (int c0 = 0; c0 < p.S; c0 += 64) {
            const int ctx_l = ctx_in(c0);
            const int nsb_l = (ctx_l + kTile - 1) / kTile;
            const int np_l = pieces_of(nsb_l);
            const int incl = wave_prefix_sum_i(np_l);
            const uint64_t past = __ballot(base + incl > v);
            if (past) {
                const int i = __builtin_ctzll(past);
                n = readlane_i32(np_l, i);
                const int nsb = readlane_i32(nsb_l, i);
                const int64_t first = base + readlane_i32(incl, i) - n;
                k = (int)(v - first);
                s = c0 + i;
                a = (int)((uint32_t)k * (uint32_t)nsb / (uint32_t)n);
                b = (int)((uint32_t)(k + 1) * (uint32_t)nsb / (uint32_t)n);
                P_u = (int)first;
                ctx = readlane_i32(ctx_l, i);
                if (s >= p.S || n < 1 || k >= n || (split && (int64_t)P_u + n > NW)) s = -1;
                break;
            }
            base += readlane_i32(incl, 63);
        }
        if (s < 0) break;  // no piece left for this workgroup

        if (v != w) __syncthreads();  // the previous piece's LDS has been read
        // the piece holding the last token writes the new token first
        if (p.slot_mapping && min(b * kTile, ctx) == ctx) mla_write_new_token<F8>(p, s);
        if constexpr (MFMA) {
            mla_mfma_piece<F8>(p, sm, s, a * kTile, min(b * kTile, ctx), n == 1,
                                  p.part_out + (size_t)v * p.Hq * kDv, kDv,
                                  p.part_lse + (size_t)v * p.Hq, 1);
        } else {
            uint32_t qreg[kHPW][kSlices];
            mla_load_queries(p, s, qreg);
            float m[kHPW], lsum[kHPW], acc[kHPW][8];
            mla_reset(m, lsum, acc);
            mla_attend<F8>(p, sm, s, a * kTile, min(b * kTile, ctx), qreg, m, lsum, acc);
            mla_emit(p, s, n == 1, m, lsum, acc, p.part_out + (size_t)v * p.Hq * kDv, kDv,
                     p.part_lse + (size_t)v * p.Hq, 1);
        }
        if (n > 1 && mla_count(p, s, n))
            merge_mla_partials(p, s, p.part_out + (size_t)P_u * p.Hq * kDv, kDv,
                               (size_t)p.Hq * kDv, (uint32_t)n * p.Hq * kDv,
                               p.part_lse + (size_t)P_u * p.Hq, 1, p.Hq, n);
        if (split) break;  // one piece per workgroup
    }
}

}  // namespace

namespace {

template <bool F8, bool MFMA>
hipError_t launch_mla(const MLAParams &p, hipStream_t stream) {
    if (p.balanced_workgroups > 0) {
        // one wave of workgroups: as many as are resident together
        static const int per_cu = [] {
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &n, reinterpret_cast<const void *>(&mla_decode_balanced_kernel<F8, MFMA>), 256, 0) !=
                    hipSuccess || n < 1)
                n = 1;
            return n;
        }();
        const int nw = min(p.balanced_workgroups, per_cu * p.num_cus);
        hipLaunchKernelGGL((mla_decode_balanced_kernel<F8, MFMA>), dim3((unsigned)nw), dim3(256), 0,
                           stream, p);
        return hipGetLastError();
    }
    const int64_t units = (int64_t)p.max_parts * p.S;
    if (units > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((mla_decode_kernel<F8, MFMA>), dim3((unsigned)units), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mla_decode(const MLAParams &p, hipStream_t stream) {
    if (p.mfma) return p.fp8 ? launch_mla<true, true>(p, stream) : launch_mla<false, true>(p, stream);
    return p.fp8 ? launch_mla<true, false>(p, stream) : launch_mla<false, false>(p, stream);
}

}  // namespace pa
