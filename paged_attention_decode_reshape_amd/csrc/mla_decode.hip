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
//   PV  lane l: output dims 8l .. 8l + 7; per token one 16-byte LDS read,
//       the weight taken from the token's lane with v_readlane, fp32 FMAs.
// A sequence longer than one partition writes fp32 partials (normalised
// output, LSE); the last workgroup of the sequence to finish merges them by
// log-sum-exp in partition order.
#include <type_traits>

#include "common.h"
#include "decode_common.h"
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

__device__ __forceinline__ int clamp_ctx(int ctx, int max_blocks, int B, int max_parts, int P) {
    const int64_t cap = min((int64_t)max_blocks * B, (int64_t)max_parts * P);
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

// Log-sum-exp merge of a sequence's partitions (in partition order), by the
// workgroup that finished last: thread -> (head tid / 16, 16-byte vectors
// v = 16 k + tid % 16, k < 8) of the partial rows; a batch of 4 partitions is
// fetched before any is used.
__device__ __forceinline__ void merge_mla_partitions(const MLAParams &p, int s, int nparts) {
    constexpr int kBatch = 4;
    const int h = threadIdx.x >> 4, c = threadIdx.x & 15;
    if (h >= p.Hq) return;
    const size_t row = (size_t)s * p.Hq + h;
    const auto rs = coherent_rsrc(p.part_out + row * p.max_parts * kDv, p.max_parts * kDv * 4);
    const float *pl = p.part_lse + row * p.max_parts;
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
            L[u] = load_coherent(&pl[pu]);
#pragma unroll
            for (int k = 0; k < 8; k++) x[u][k] = load_coherent4(rs, (pu * kDv + 4 * (16 * k + c)) * 4);
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

__global__ __launch_bounds__(256, 2) void mla_decode_kernel(MLAParams p) {
    const int part = blockIdx.x / p.S;
    const int s = blockIdx.x - part * p.S;
    const int P = p.partition;
    const int start = part * P;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;
    const int hf = lane >> 5;  // QK: half of the latent row
    const int tk = lane & 31;  // QK: token of the tile
    uint16_t *out = reinterpret_cast<uint16_t *>(p.out);

    __shared__ __align__(16) uint32_t sm_tile[kTile * kRowDw];
    // latent row of every token of the partition (-1: past the end or an
    // out-of-range block id), resolved once so that the tile loop issues no
    // dependent block-table reads
    __shared__ int32_t sm_row[kMaxPartition];

    const int ctx = clamp_ctx(as_const<int32_t>(p.context_lens)[s], p.max_blocks, p.B,
                              p.max_parts, P);
    if (start >= ctx) {
        if (ctx == 0 && part == 0) {
            // no keys: out = 0, lse = -inf
            for (int idx = threadIdx.x; idx < p.Hq * kDv; idx += blockDim.x) {
                out[((size_t)s * p.Hq + idx / kDv) * kDv + idx % kDv] = 0;
                if (idx % kDv == 0 && p.lse) p.lse[(size_t)s * p.Hq + idx / kDv] = kNegInf;
            }
        }
        return;
    }
    const int end = min(start + P, ctx);
    const int nparts = (ctx + P - 1) / P;
    const float sl2 = p.scale * kLog2e;

    for (int i = threadIdx.x; i < end - start; i += blockDim.x) {
        const int t = start + i;
        const int b = p.block_table[(size_t)s * p.max_blocks + t / p.B];
        sm_row[i] = b >= 0 && (int64_t)b < p.num_blocks ? b * p.B + t % p.B : -1;
    }

    // this wave's heads (past num_q_heads: repeats of real heads, not stored)
    int head[kHPW];
#pragma unroll
    for (int j = 0; j < kHPW; j++) head[j] = (kHPW * wave + j) % p.Hq;
    // query slice k of head j: lane n of a row of half f holds dword
    // 144 f + 16 k + n of the head's query
    uint32_t qreg[kHPW][kSlices];
#pragma unroll
    for (int j = 0; j < kHPW; j++) {
        const uint32_t *qh = reinterpret_cast<const uint32_t *>(p.query) +
                             ((size_t)s * p.Hq + head[j]) * (kDl / 2) + kHalfDw * hf + col;
#pragma unroll
        for (int k = 0; k < kSlices; k++) qreg[j][k] = qh[16 * k];
    }

    // Tile loader: thread (wave w, lane) moves vectors (lane & 7) + 8 i of
    // the latent row of tile token 8 w + (lane >> 3); tokens past the end
    // (or with an out-of-range block id) become zero rows.
    const uint4 *kv = reinterpret_cast<const uint4 *>(p.kv_cache);
    const int ld_tok = 8 * wave + (lane >> 3), ld_vec = lane & 7;
    auto load_tile = [&](int t0, uint4 (&r)[kLoadVec]) {
        const int t = t0 + ld_tok;
        const int rowi = t < end ? sm_row[t - start] : -1;
        const uint4 *src = kv + (size_t)(rowi < 0 ? 0 : rowi) * kRowVec + ld_vec;
#pragma unroll
        for (int i = 0; i < kLoadVec; i++)
            r[i] = rowi < 0 ? make_uint4(0, 0, 0, 0) : src[8 * i];
    };
    auto store_tile = [&](const uint4 (&r)[kLoadVec]) {
        uint4 *dst = reinterpret_cast<uint4 *>(&sm_tile[ld_tok * kRowDw]) + ld_vec;
#pragma unroll
        for (int i = 0; i < kLoadVec; i++) dst[8 * i] = r[i];
    };
    // validity of QK token tk of the tile starting at t0 (same test as the loader)
    auto token_ok = [&](int t0) {
        const int t = t0 + tk;
        return t < end && sm_row[t - start] >= 0;
    };

    float m[kHPW], lsum[kHPW], acc[kHPW][8];
#pragma unroll
    for (int j = 0; j < kHPW; j++) {
        m[j] = kNegInf;
        lsum[j] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) acc[j][i] = 0.f;
    }

    __syncthreads();  // sm_row complete
    uint4 next[kLoadVec];
    load_tile(start, next);
    for (int t0 = start; t0 < end; t0 += kTile) {
        __syncthreads();  // the previous tile is no longer read
        store_tile(next);
        const bool tok_ok = token_ok(t0);
        __syncthreads();
        if (t0 + kTile < end) load_tile(t0 + kTile, next);

        // QK: half f of the row of token tk against the wave's heads
        float za[kHPW], zb[kHPW];
#pragma unroll
        for (int j = 0; j < kHPW; j++) za[j] = zb[j] = 0.f;
        const uint4 *kr = reinterpret_cast<const uint4 *>(&sm_tile[tk * kRowDw + kHalfDw * hf]);
#pragma unroll
        for (int k = 0; k < kSlices; k++) {
            const uint4 k0 = kr[4 * k], k1 = kr[4 * k + 1], k2 = kr[4 * k + 2], k3 = kr[4 * k + 3];
#pragma unroll
            for (int j = 0; j < kHPW; j++) qk16<false>(za[j], zb[j], qreg[j][k], k0, k1, k2, k3);
        }
        dpp_result_fence<kHPW>(za);
        dpp_result_fence<kHPW>(zb);
        // softmax: exact max of the tile, one rescale of the running state
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
            const float mn = fmax_nc(m[j], mx);
            const float mref = mn == kNegInf ? 0.f : mn;
            const float alpha = fast_exp2(m[j] - mref);
            m[j] = mn;
            pw[j] = fast_exp2(sc - mref);
            lsum[j] = lsum[j] * alpha + pw[j];
#pragma unroll
            for (int i = 0; i < 8; i++) acc[j][i] *= alpha;
        }
        // PV: dims 8 lane .. 8 lane + 7 of every token of the tile
        const uint4 *vr = reinterpret_cast<const uint4 *>(sm_tile) + lane;
        static_for<kTile>([&](auto t_c) {
            constexpr int t = decltype(t_c)::value;
            const uint4 v = vr[t * (kRowDw / 4)];
            const float vf[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                                 bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
            for (int j = 0; j < kHPW; j++) {
                const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw[j]), t));
#pragma unroll
                for (int i = 0; i < 8; i++) acc[j][i] = __builtin_fmaf(w, vf[i], acc[j][i]);
            }
        });
    }

    // every wave finishes its own heads (lanes 32-63 repeat the weights of 0-31)
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
        if (nparts == 1) {
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
            const auto rs = coherent_rsrc(p.part_out + (orow * p.max_parts + part) * kDv, kDv * 4);
#pragma unroll
            for (int i = 0; i < 2; i++)
                store_coherent4(rs, (64 * i + lane) * 16, acc[j][4 * i] * inv[j],
                                acc[j][4 * i + 1] * inv[j], acc[j][4 * i + 2] * inv[j],
                                acc[j][4 * i + 3] * inv[j]);
            if (lane == 0) store_coherent(&p.part_lse[orow * p.max_parts + part], L[j]);
        }
    }
    if (nparts == 1) return;

    // The last workgroup of the sequence to finish merges all partitions
    // (partials are written and read with device-coherent accesses; each
    // thread waits for its stores to complete before one thread counts).
    __shared__ int sm_last;
    wait_stores();
    __syncthreads();
    int *counter = p.counters + s;
    if (threadIdx.x == 0)
        sm_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  nparts - 1;
    __syncthreads();
    if (!sm_last) return;
    if (threadIdx.x == 0)  // leave the counter zero for the next call
        __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    merge_mla_partitions(p, s, nparts);
}

}  // namespace

hipError_t launch_mla_decode(const MLAParams &p, hipStream_t stream) {
    const int64_t units = (int64_t)p.max_parts * p.S;
    if (units > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mla_decode_kernel, dim3((unsigned)units), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa
