// GQA / MHA paged decode attention over the preshuffled KV cache.
//
// Decode is memory-bound: every step streams the whole KV cache of every
// sequence once ("ROCm attention backends" blog, phase taxonomy; the
// decode path reads the shuffled cache directly).  Each K/V byte is read
// exactly once, as a 16-byte vector, and the arithmetic runs on the VALU as
// bf16 dot2 instructions whose broadcast operand comes through DPP.
//
// Work unit: one workgroup of 4 waves per (partition, kv head, sequence);
// the 1-D grid is ordered partition-major so the units of one partition
// index spread over all XCDs.  A wave processes 64 tokens per step:
//   QK  lane l owns token t0 + l and loads its head_dim / 8 K vectors
//       (k_cache[p][g][c][o][0..8), 8 consecutive dims of one token), so a
//       lane accumulates whole dot products with no cross-lane reduction.
//       The group's queries sit in VGPRs laid out so that lane n of every
//       16-lane row holds query dword n of a 16-dword slice; DPP
//       row_newbcast hands it to the whole row inside v_dot2c.
//   softmax  one wave max per head (integer-ordered DPP max + gfx950
//       permlane swaps), online rescale, p = exp2(z - m) with log2(e)
//       folded into the scale.
//   PV  lane l owns dims l (and l + 64).  A V vector
//       (v_cache[p][g][j][d][0..8), 8 consecutive tokens of one dim) makes
//       P.V a reduction over tokens inside a lane.  p is split as
//       hi + lo (two bf16) so that bf16 dot2 keeps ~2^-17 relative accuracy
//       per weight; the pairs are permuted (ds_bpermute) so that lane n of
//       every row holds token pair n and are broadcast by DPP as above.
// Groups of more than 8 query heads are processed 8 heads at a time with
// the queries re-read from LDS.  The 4 waves' states merge in LDS.  A
// sequence longer than one partition writes fp32 partials (normalised
// output, LSE) that a second kernel merges by log-sum-exp in partition
// order, so results are deterministic.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kStep = 64;  // tokens per wave step

// context length limited to what the block table and the grid can cover
__device__ __forceinline__ int clamp_ctx(int ctx, int max_blocks, int B, int max_parts, int P) {
    const int64_t cap = min((int64_t)max_blocks * B, (int64_t)max_parts * P);
    return ctx < 0 ? 0 : ((int64_t)ctx > cap ? (int)cap : ctx);
}

__device__ __forceinline__ uint32_t mask_pair(uint32_t w, int first, int nvalid) {
    // w holds tokens first (lo) and first + 1 (hi)
    return first >= nvalid ? 0u : (first + 1 >= nvalid ? (w & 0xffffu) : w);
}

// One v_dot2c whose first operand is lane `n` of the same 16-lane row.
#define PA_DOT2_BC(acc, r, v, n) \
    "v_dot2c_f32_bf16_dpp " acc ", " r ", " v " row_newbcast:" n " row_mask:0xf bank_mask:0xf\n\t"

// Hazards the compiler cannot see inside inline asm:
//  - the leading s_nop covers the VALU-write -> DPP-read hazard on the
//    broadcast registers (nothing inside a block writes them);
//  - an ordinary VALU instruction that reads a v_dot2c_dpp result within a
//    few instructions sees a stale value on gfx950 (measured: results were
//    wrong and timing-dependent without it), so a block whose outputs plain
//    code reads next ends with s_nop 4 (TAIL).  Chains of these blocks feed
//    each other through the accumulator operand, which needs no wait.

// QK for two heads over 4 K vectors (16 dwords): lane n of qa / qb holds
// query dword n of the slice.  Two accumulator chains per head.
#define PA_QK2H_BODY                                                                        \
    "s_nop 1\n\t"                                                                           \
    PA_DOT2_BC("%0", "%4", "%6", "0") PA_DOT2_BC("%2", "%5", "%6", "0")                     \
    PA_DOT2_BC("%1", "%4", "%7", "1") PA_DOT2_BC("%3", "%5", "%7", "1")                     \
    PA_DOT2_BC("%0", "%4", "%8", "2") PA_DOT2_BC("%2", "%5", "%8", "2")                     \
    PA_DOT2_BC("%1", "%4", "%9", "3") PA_DOT2_BC("%3", "%5", "%9", "3")                     \
    PA_DOT2_BC("%0", "%4", "%10", "4") PA_DOT2_BC("%2", "%5", "%10", "4")                   \
    PA_DOT2_BC("%1", "%4", "%11", "5") PA_DOT2_BC("%3", "%5", "%11", "5")                   \
    PA_DOT2_BC("%0", "%4", "%12", "6") PA_DOT2_BC("%2", "%5", "%12", "6")                   \
    PA_DOT2_BC("%1", "%4", "%13", "7") PA_DOT2_BC("%3", "%5", "%13", "7")                   \
    PA_DOT2_BC("%0", "%4", "%14", "8") PA_DOT2_BC("%2", "%5", "%14", "8")                   \
    PA_DOT2_BC("%1", "%4", "%15", "9") PA_DOT2_BC("%3", "%5", "%15", "9")                   \
    PA_DOT2_BC("%0", "%4", "%16", "10") PA_DOT2_BC("%2", "%5", "%16", "10")                 \
    PA_DOT2_BC("%1", "%4", "%17", "11") PA_DOT2_BC("%3", "%5", "%17", "11")                 \
    PA_DOT2_BC("%0", "%4", "%18", "12") PA_DOT2_BC("%2", "%5", "%18", "12")                 \
    PA_DOT2_BC("%1", "%4", "%19", "13") PA_DOT2_BC("%3", "%5", "%19", "13")                 \
    PA_DOT2_BC("%0", "%4", "%20", "14") PA_DOT2_BC("%2", "%5", "%20", "14")                 \
    PA_DOT2_BC("%1", "%4", "%21", "15") PA_DOT2_BC("%3", "%5", "%21", "15")
#define PA_QK2H_OPERANDS                                                                    \
    : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1)                                                \
    : "v"(qa), "v"(qb), "v"(k0.x), "v"(k0.y), "v"(k0.z), "v"(k0.w), "v"(k1.x), "v"(k1.y),   \
      "v"(k1.z), "v"(k1.w), "v"(k2.x), "v"(k2.y), "v"(k2.z), "v"(k2.w), "v"(k3.x),          \
      "v"(k3.y), "v"(k3.z), "v"(k3.w)

template <bool TAIL>
__device__ __forceinline__ void qk_2h(float &a0, float &a1, float &b0, float &b1, uint32_t qa,
                                      uint32_t qb, const uint4 &k0, const uint4 &k1,
                                      const uint4 &k2, const uint4 &k3) {
    if constexpr (TAIL)
        asm volatile(PA_QK2H_BODY "s_nop 4\n\t" PA_QK2H_OPERANDS);
    else
        asm volatile(PA_QK2H_BODY PA_QK2H_OPERANDS);
}

#define PA_QK1H_BODY                                                                        \
    "s_nop 1\n\t"                                                                           \
    PA_DOT2_BC("%0", "%2", "%3", "0") PA_DOT2_BC("%1", "%2", "%4", "1")                     \
    PA_DOT2_BC("%0", "%2", "%5", "2") PA_DOT2_BC("%1", "%2", "%6", "3")                     \
    PA_DOT2_BC("%0", "%2", "%7", "4") PA_DOT2_BC("%1", "%2", "%8", "5")                     \
    PA_DOT2_BC("%0", "%2", "%9", "6") PA_DOT2_BC("%1", "%2", "%10", "7")                    \
    PA_DOT2_BC("%0", "%2", "%11", "8") PA_DOT2_BC("%1", "%2", "%12", "9")                   \
    PA_DOT2_BC("%0", "%2", "%13", "10") PA_DOT2_BC("%1", "%2", "%14", "11")                 \
    PA_DOT2_BC("%0", "%2", "%15", "12") PA_DOT2_BC("%1", "%2", "%16", "13")                 \
    PA_DOT2_BC("%0", "%2", "%17", "14") PA_DOT2_BC("%1", "%2", "%18", "15")
#define PA_QK1H_OPERANDS                                                                    \
    : "+v"(a0), "+v"(a1)                                                                    \
    : "v"(qa), "v"(k0.x), "v"(k0.y), "v"(k0.z), "v"(k0.w), "v"(k1.x), "v"(k1.y), "v"(k1.z), \
      "v"(k1.w), "v"(k2.x), "v"(k2.y), "v"(k2.z), "v"(k2.w), "v"(k3.x), "v"(k3.y), "v"(k3.z), \
      "v"(k3.w)

template <bool TAIL>
__device__ __forceinline__ void qk_1h(float &a0, float &a1, uint32_t qa, const uint4 &k0,
                                      const uint4 &k1, const uint4 &k2, const uint4 &k3) {
    if constexpr (TAIL)
        asm volatile(PA_QK1H_BODY "s_nop 4\n\t" PA_QK1H_OPERANDS);
    else
        asm volatile(PA_QK1H_BODY PA_QK1H_OPERANDS);
}

__device__ __forceinline__ void qk_slice_2h(bool last, float &a0, float &a1, float &b0, float &b1,
                                            uint32_t qa, uint32_t qb, const uint4 &k0,
                                            const uint4 &k1, const uint4 &k2, const uint4 &k3) {
    if (last)
        qk_2h<true>(a0, a1, b0, b1, qa, qb, k0, k1, k2, k3);
    else
        qk_2h<false>(a0, a1, b0, b1, qa, qb, k0, k1, k2, k3);
}

__device__ __forceinline__ void qk_slice_1h(bool last, float &a0, float &a1, uint32_t qa,
                                            const uint4 &k0, const uint4 &k1, const uint4 &k2,
                                            const uint4 &k3) {
    if (last)
        qk_1h<true>(a0, a1, qa, k0, k1, k2, k3);
    else
        qk_1h<false>(a0, a1, qa, k0, k1, k2, k3);
}

// PV for one head over one group of 8 tokens: acc += sum over the group's
// 4 token pairs of (hi + lo) . v, where pair k sits in lane N0 + k of
// every row of rh / rl.  v holds the group's 8 tokens of one dim as pairs.
#define PA_PV2_BODY                                                                         \
    "s_nop 1\n\t"                                                                           \
    PA_DOT2_BC("%0", "%2", "%4", "%12") PA_DOT2_BC("%1", "%2", "%8", "%12")                 \
    PA_DOT2_BC("%0", "%3", "%4", "%12") PA_DOT2_BC("%1", "%3", "%8", "%12")                 \
    PA_DOT2_BC("%0", "%2", "%5", "%13") PA_DOT2_BC("%1", "%2", "%9", "%13")                 \
    PA_DOT2_BC("%0", "%3", "%5", "%13") PA_DOT2_BC("%1", "%3", "%9", "%13")                 \
    PA_DOT2_BC("%0", "%2", "%6", "%14") PA_DOT2_BC("%1", "%2", "%10", "%14")                \
    PA_DOT2_BC("%0", "%3", "%6", "%14") PA_DOT2_BC("%1", "%3", "%10", "%14")                \
    PA_DOT2_BC("%0", "%2", "%7", "%15") PA_DOT2_BC("%1", "%2", "%11", "%15")                \
    PA_DOT2_BC("%0", "%3", "%7", "%15") PA_DOT2_BC("%1", "%3", "%11", "%15")
#define PA_PV2_OPERANDS                                                                     \
    : "+v"(a0), "+v"(a1)                                                                    \
    : "v"(rh), "v"(rl), "v"(v0.x), "v"(v0.y), "v"(v0.z), "v"(v0.w), "v"(v1.x), "v"(v1.y),   \
      "v"(v1.z), "v"(v1.w), "n"(N0), "n"(N0 + 1), "n"(N0 + 2), "n"(N0 + 3)

template <int N0, bool TAIL>
__device__ __forceinline__ void pv_bcast2(float &a0, float &a1, uint32_t rh, uint32_t rl,
                                          const uint4 &v0, const uint4 &v1) {
    if constexpr (TAIL)
        asm volatile(PA_PV2_BODY "s_nop 4\n\t" PA_PV2_OPERANDS);
    else
        asm volatile(PA_PV2_BODY PA_PV2_OPERANDS);
}

#define PA_PV1_BODY                                                                         \
    "s_nop 1\n\t"                                                                           \
    PA_DOT2_BC("%0", "%1", "%3", "%7") PA_DOT2_BC("%0", "%2", "%3", "%7")                   \
    PA_DOT2_BC("%0", "%1", "%4", "%8") PA_DOT2_BC("%0", "%2", "%4", "%8")                   \
    PA_DOT2_BC("%0", "%1", "%5", "%9") PA_DOT2_BC("%0", "%2", "%5", "%9")                   \
    PA_DOT2_BC("%0", "%1", "%6", "%10") PA_DOT2_BC("%0", "%2", "%6", "%10")
#define PA_PV1_OPERANDS                                                                     \
    : "+v"(a0)                                                                              \
    : "v"(rh), "v"(rl), "v"(v0.x), "v"(v0.y), "v"(v0.z), "v"(v0.w), "n"(N0), "n"(N0 + 1),   \
      "n"(N0 + 2), "n"(N0 + 3)

template <int N0, bool TAIL>
__device__ __forceinline__ void pv_bcast1(float &a0, uint32_t rh, uint32_t rl, const uint4 &v0) {
    if constexpr (TAIL)
        asm volatile(PA_PV1_BODY "s_nop 4\n\t" PA_PV1_OPERANDS);
    else
        asm volatile(PA_PV1_BODY PA_PV1_OPERANDS);
}

// Dispatch on the (unrolled, hence constant) first pair index of the group.
template <int DV, bool TAIL>
__device__ __forceinline__ void pv_group(int n0, float (&a)[DV], uint32_t rh, uint32_t rl,
                                         const uint4 (&v)[DV]) {
    if constexpr (DV == 2) {
        switch (n0) {
        case 0: pv_bcast2<0, TAIL>(a[0], a[1], rh, rl, v[0], v[1]); break;
        case 4: pv_bcast2<4, TAIL>(a[0], a[1], rh, rl, v[0], v[1]); break;
        case 8: pv_bcast2<8, TAIL>(a[0], a[1], rh, rl, v[0], v[1]); break;
        default: pv_bcast2<12, TAIL>(a[0], a[1], rh, rl, v[0], v[1]); break;
        }
    } else {
        switch (n0) {
        case 0: pv_bcast1<0, TAIL>(a[0], rh, rl, v[0]); break;
        case 4: pv_bcast1<4, TAIL>(a[0], rh, rl, v[0]); break;
        case 8: pv_bcast1<8, TAIL>(a[0], rh, rl, v[0]); break;
        default: pv_bcast1<12, TAIL>(a[0], rh, rl, v[0]); break;
        }
    }
}

template <int D, int B, int G>
__global__ __launch_bounds__(256) void paged_decode_partition_kernel(DecodeParams p) {
    constexpr int C = D / 8;          // K vectors per token
    constexpr int DV = D / 64;        // output dims per lane
    constexpr int HG = G < 8 ? G : 8; // heads per pass
    constexpr int NPASS = G / HG;
    constexpr int QR = D / 32;        // query VGPRs per head (16 dwords each)

    const int units = p.S * p.Hkv;
    const int part = blockIdx.x / units;
    const int rem = blockIdx.x - part * units;
    const int s = rem / p.Hkv, g = rem - s * p.Hkv;
    const int Ga = p.Hq / p.Hkv;
    const int P = p.partition;
    const int ctx =
        clamp_ctx(as_const<int32_t>(p.context_lens)[s], p.max_blocks, B, p.max_parts, P);
    const int start = part * P;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint16_t *out = reinterpret_cast<uint16_t *>(p.out);

    if (start >= ctx) {
        if (ctx == 0 && part == 0) {
            // no keys: out = 0, lse = -inf
            for (int idx = threadIdx.x; idx < Ga * D; idx += blockDim.x) {
                const int hq = g * Ga + idx / D;
                out[((size_t)s * p.Hq + hq) * D + idx % D] = 0;
                if (idx % D == 0 && p.lse) p.lse[(size_t)s * p.Hq + hq] = kNegInf;
            }
        }
        return;
    }
    const int end = min(start + P, ctx);
    const int nparts = (ctx + P - 1) / P;
    const float sl2 = p.scale * kLog2e;

    // the group's queries in LDS; padded heads (h >= Ga) repeat real ones
    __shared__ uint32_t q_sm[G * D / 2];
    {
        const uint32_t *qg = reinterpret_cast<const uint32_t *>(p.query) +
                             ((size_t)s * p.Hq + (size_t)g * Ga) * (D / 2);
        for (int i = threadIdx.x; i < G * D / 2; i += blockDim.x) {
            const int h = i / (D / 2);
            q_sm[i] = qg[(h < Ga ? h : h - Ga) * (D / 2) + i % (D / 2)];
        }
    }
    __syncthreads();

    // ds_bpermute byte addresses: lane L reads pair L % 16 (lane 2 * (L % 16))
    // and pair 16 + L % 16 (lane 32 + 2 * (L % 16))
    const int src_pair0 = (2 * (lane & 15)) * 4;
    const int src_pair1 = (32 + 2 * (lane & 15)) * 4;
    const cptr<int32_t> bt = as_const<int32_t>(p.block_table) + (size_t)s * p.max_blocks;
    const uint4 *kc = reinterpret_cast<const uint4 *>(p.k_cache);
    const uint4 *vc = reinterpret_cast<const uint4 *>(p.v_cache);

    // query slices: qr[h][i] holds, in lane n of every row, dword 16 i + n of head h
    uint32_t qr[HG][QR];
    if constexpr (NPASS == 1) {
#pragma unroll
        for (int h = 0; h < HG; h++)
#pragma unroll
            for (int i = 0; i < QR; i++) qr[h][i] = q_sm[h * (D / 2) + 16 * i + (lane & 15)];
    }

    float m[G], lsum[G], acc[G][DV];
#pragma unroll
    for (int h = 0; h < G; h++) {
        m[h] = kNegInf;
        lsum[h] = 0.f;
#pragma unroll
        for (int jj = 0; jj < DV; jj++) acc[h][jj] = 0.f;
    }

    for (int t0 = start + wave * kStep; t0 < end; t0 += kWaves * kStep) {
        const int tok = t0 + lane;
        bool valid = tok < end;
        int phys = 0;
        if (valid) {
            phys = bt[tok / B];
            if (phys < 0 || (int64_t)phys >= p.num_blocks) {
                valid = false;
                phys = 0;
            }
        }
        // K: this lane's token, all head_dim / 8 vectors
        uint4 kx[C];
        {
            const uint4 *kp = kc + ((size_t)phys * p.Hkv + g) * (size_t)(C * B) + (tok % B);
            if (valid) {
#pragma unroll
                for (int c = 0; c < C; c++) kx[c] = kp[c * B];
            } else {
#pragma unroll
                for (int c = 0; c < C; c++) kx[c] = make_uint4(0, 0, 0, 0);
            }
        }
        // V: 8 token groups of 8; this lane's dims lane + 64 * jj
        uint4 vx[8][DV];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int tg0 = t0 + 8 * j;
            if (tg0 < end) {
                const int pj = readlane_i32(phys, 8 * j);
                const uint4 *vp =
                    vc + (((size_t)pj * p.Hkv + g) * (B / 8) + ((8 * j) % B) / 8) * D + lane;
#pragma unroll
                for (int jj = 0; jj < DV; jj++) vx[j][jj] = vp[64 * jj];
            } else {
#pragma unroll
                for (int jj = 0; jj < DV; jj++) vx[j][jj] = make_uint4(0, 0, 0, 0);
            }
        }
        // zero the V of tokens past the end (their weight is 0; the data may be anything)
        if (t0 + kStep > end) {
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const int nv = end - (t0 + 8 * j);
                if (nv > 0 && nv < 8) {
#pragma unroll
                    for (int jj = 0; jj < DV; jj++) {
                        vx[j][jj].x = mask_pair(vx[j][jj].x, 0, nv);
                        vx[j][jj].y = mask_pair(vx[j][jj].y, 2, nv);
                        vx[j][jj].z = mask_pair(vx[j][jj].z, 4, nv);
                        vx[j][jj].w = mask_pair(vx[j][jj].w, 6, nv);
                    }
                }
            }
        }

#pragma unroll
        for (int pass = 0; pass < NPASS; pass++) {
            const int hb = pass * HG;
            if constexpr (NPASS > 1) {
#pragma unroll
                for (int h = 0; h < HG; h++)
#pragma unroll
                    for (int i = 0; i < QR; i++)
                        qr[h][i] = q_sm[(hb + h) * (D / 2) + 16 * i + (lane & 15)];
            }
            // QK: whole dot products per lane
            float sc[HG];
            if constexpr (HG == 1) {
                float a0 = 0.f, a1 = 0.f;
#pragma unroll
                for (int i = 0; i < QR; i++)
                    qk_slice_1h(i == QR - 1, a0, a1, qr[0][i], kx[4 * i], kx[4 * i + 1],
                                kx[4 * i + 2], kx[4 * i + 3]);
                sc[0] = valid ? (a0 + a1) * sl2 : kNegInf;
            } else {
#pragma unroll
                for (int h = 0; h < HG; h += 2) {
                    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
                    for (int i = 0; i < QR; i++)
                        qk_slice_2h(i == QR - 1, a0, a1, b0, b1, qr[h][i], qr[h + 1][i], kx[4 * i],
                                    kx[4 * i + 1], kx[4 * i + 2], kx[4 * i + 3]);
                    sc[h] = valid ? (a0 + a1) * sl2 : kNegInf;
                    sc[h + 1] = valid ? (b0 + b1) * sl2 : kNegInf;
                }
            }
            // online softmax and the hi / lo pairs for P.V
            uint32_t r0hi[HG], r1hi[HG], r0lo[HG], r1lo[HG];
#pragma unroll
            for (int h = 0; h < HG; h++) {
                const int H = hb + h;
                const float mx = uniform_f(wave_max(sc[h]));
                const float mn = fmax_nc(m[H], mx);
                const float mref = mn == kNegInf ? 0.f : mn;
                const float alpha = fast_exp2(m[H] - mref);
                m[H] = mn;
                const float pr = fast_exp2(sc[h] - mref);
                lsum[H] = lsum[H] * alpha + pr;
#pragma unroll
                for (int jj = 0; jj < DV; jj++) acc[H][jj] *= alpha;
                const float pn = dpp_f<kQuadXor1>(pr);
                const uint32_t hi = pack_bf16x2(pr, pn);
                const uint32_t lo = pack_bf16x2(pr - bf16_lo(hi), pn - bf16_hi(hi));
                r0hi[h] = (uint32_t)__builtin_amdgcn_ds_bpermute(src_pair0, (int)hi);
                r1hi[h] = (uint32_t)__builtin_amdgcn_ds_bpermute(src_pair1, (int)hi);
                r0lo[h] = (uint32_t)__builtin_amdgcn_ds_bpermute(src_pair0, (int)lo);
                r1lo[h] = (uint32_t)__builtin_amdgcn_ds_bpermute(src_pair1, (int)lo);
            }
            // PV: token group j holds pairs 4j .. 4j+3
#pragma unroll
            for (int j = 0; j < 8; j++) {
                if (t0 + 8 * j < end) {
#pragma unroll
                    for (int h = 0; h < HG; h++) {
                        const uint32_t rh = j < 4 ? r0hi[h] : r1hi[h];
                        const uint32_t rl = j < 4 ? r0lo[h] : r1lo[h];
                        if (h == HG - 1)
                            pv_group<DV, true>((4 * j) % 16, acc[hb + h], rh, rl, vx[j]);
                        else
                            pv_group<DV, false>((4 * j) % 16, acc[hb + h], rh, rl, vx[j]);
                    }
                }
            }
        }
    }

    // merge the 4 waves of the workgroup
    __shared__ float sm_m[kWaves][G], sm_l[kWaves][G];
    __shared__ float sm_acc[kWaves][G][D];
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float l = wave_sum(lsum[h]);
        if (lane == 0) {
            sm_m[wave][h] = m[h];
            sm_l[wave][h] = l;
        }
#pragma unroll
        for (int jj = 0; jj < DV; jj++) sm_acc[wave][h][lane + 64 * jj] = acc[h][jj];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < Ga * D; idx += blockDim.x) {
        const int h = idx / D, d = idx % D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; w++) M = fmax_nc(M, sm_m[w][h]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            const float wt = fast_exp2(sm_m[w][h] - M);
            num += wt * sm_acc[w][h][d];
            den += wt * sm_l[w][h];
        }
        const float o = num / den;
        const float L = (M + fast_log2(den)) * kLn2;
        const size_t row = (size_t)s * p.Hq + (size_t)g * Ga + h;
        if (nparts == 1) {
            out[row * D + d] = f32_to_bf16(o);
            if (d == 0 && p.lse) p.lse[row] = L;
        } else {
            p.part_out[(row * p.max_parts + part) * D + d] = o;
            if (d == 0) p.part_lse[row * p.max_parts + part] = L;
        }
    }
}

// Log-sum-exp merge of a sequence's partitions, one wave per (seq, q head),
// in partition order: lane i holds partition i's LSE, the weights are
// broadcast with readlane and the partial outputs of 4 partitions are read
// together.
template <int D>
__global__ __launch_bounds__(256) void paged_decode_reduce_kernel(DecodeParams p, int B) {
    constexpr int DV = D / 64;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.S * p.Hq) return;
    const int lane = threadIdx.x & 63;
    const int s = row / p.Hq;
    const int P = p.partition;
    const int ctx = clamp_ctx(p.context_lens[s], p.max_blocks, B, p.max_parts, P);
    const int nparts = (ctx + P - 1) / P;
    if (nparts <= 1) return;
    const float *pl = p.part_lse + (size_t)row * p.max_parts;
    float M = kNegInf;
    for (int b = 0; b < nparts; b += 64) {
        const float v = b + lane < nparts ? pl[b + lane] : kNegInf;
        M = fmax_nc(M, wave_max(v));
    }
    float den = 0.f, o[DV];
#pragma unroll
    for (int jj = 0; jj < DV; jj++) o[jj] = 0.f;
    const float *po = p.part_out + (size_t)row * p.max_parts * D + lane;
    for (int b = 0; b < nparts; b += 64) {
        const float w = b + lane < nparts ? fast_exp2((pl[b + lane] - M) * kLog2e) : 0.f;
        den += wave_sum(w);
        const int n = min(64, nparts - b);
        int k = 0;
        for (; k + 4 <= n; k += 4) {
            float x[4][DV];
#pragma unroll
            for (int u = 0; u < 4; u++)
#pragma unroll
                for (int jj = 0; jj < DV; jj++) x[u][jj] = po[(size_t)(b + k + u) * D + 64 * jj];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const float wk = __int_as_float(readlane_i32(__float_as_int(w), k + u));
#pragma unroll
                for (int jj = 0; jj < DV; jj++) o[jj] += wk * x[u][jj];
            }
        }
        for (; k < n; k++) {
            const float wk = __int_as_float(readlane_i32(__float_as_int(w), k));
#pragma unroll
            for (int jj = 0; jj < DV; jj++) o[jj] += wk * po[(size_t)(b + k) * D + 64 * jj];
        }
    }
    uint16_t *out = reinterpret_cast<uint16_t *>(p.out) + (size_t)row * D + lane;
    const float inv = 1.f / den;
#pragma unroll
    for (int jj = 0; jj < DV; jj++) out[64 * jj] = f32_to_bf16(o[jj] * inv);
    if (lane == 0 && p.lse) p.lse[row] = M + fast_log2(den) * kLn2;
}

template <int D, int B, int G>
hipError_t launch_partition(const DecodeParams &p, hipStream_t stream) {
    const int64_t units = (int64_t)p.max_parts * p.S * p.Hkv;
    if (units > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((paged_decode_partition_kernel<D, B, G>), dim3((unsigned)units), dim3(256),
                       0, stream, p);
    return hipGetLastError();
}

template <int D, int B>
hipError_t dispatch_group(const DecodeParams &p, hipStream_t stream) {
    const int Ga = p.Hq / p.Hkv;
    if (Ga <= 1) return launch_partition<D, B, 1>(p, stream);
    if (Ga <= 2) return launch_partition<D, B, 2>(p, stream);
    if (Ga <= 4) return launch_partition<D, B, 4>(p, stream);
    if (Ga <= 8) return launch_partition<D, B, 8>(p, stream);
    return launch_partition<D, B, 16>(p, stream);
}

}  // namespace

hipError_t launch_paged_decode(const DecodeParams &p, hipStream_t stream) {
    hipError_t e;
    if (p.D == 128)
        e = p.B == 16 ? dispatch_group<128, 16>(p, stream) : dispatch_group<128, 32>(p, stream);
    else
        e = p.B == 16 ? dispatch_group<64, 16>(p, stream) : dispatch_group<64, 32>(p, stream);
    if (e != hipSuccess || p.max_parts <= 1) return e;
    const unsigned rows = (unsigned)p.S * (unsigned)p.Hq;
    dim3 grid((rows + 3) / 4);
    if (p.D == 128)
        hipLaunchKernelGGL(paged_decode_reduce_kernel<128>, grid, dim3(256), 0, stream, p, p.B);
    else
        hipLaunchKernelGGL(paged_decode_reduce_kernel<64>, grid, dim3(256), 0, stream, p, p.B);
    return hipGetLastError();
}

}  // namespace pa
