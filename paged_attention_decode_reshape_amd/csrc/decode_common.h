// Inline-asm building blocks shared by the decode kernels (internal):
// bf16 dot products whose broadcast operand comes through DPP, and the
// log-sum-exp merge of split-KV partition partials.
#pragma once

#include "common.h"

namespace pa {

// One v_dot2c whose first operand is lane `n` of the same 16-lane row.
#define PA_DOT2_BC(acc, r, v, n) \
    "v_dot2c_f32_bf16_dpp " acc ", " r ", " v " row_newbcast:" n " row_mask:0xf bank_mask:0xf\n\t"

// Hazards the compiler cannot see inside inline asm:
//  - the leading s_nop covers the VALU-write -> DPP-read hazard on the
//    broadcast register (nothing inside a block writes it);
//  - an ordinary VALU instruction that reads a v_dot2c_dpp result within a
//    few instructions sees a stale value on gfx950 (measured: results were
//    wrong and timing-dependent without it), so a block whose outputs plain
//    code reads next ends with s_nop 4 (TAIL).  Blocks that feed each other
//    through the accumulator operand need no wait.

// Waits out the DPP-result hazard for N accumulators before plain code reads
// them: the compiler cannot schedule a read of v[i] above this block, since
// the block (nominally) rewrites every v[i].
template <int N>
__device__ __forceinline__ void dpp_result_fence(float *v) {
    static_assert(N % 4 == 0 || N < 4, "groups of 4");
    if constexpr (N >= 4) {
        asm volatile("s_nop 4" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
#pragma unroll
        for (int i = 4; i < N; i += 4)
            asm volatile("" : "+v"(v[i]), "+v"(v[i + 1]), "+v"(v[i + 2]), "+v"(v[i + 3]));
    } else {
#pragma unroll
        for (int i = 0; i < N; i++) asm volatile("s_nop 4" : "+v"(v[i]));
    }
}

// a, b += dot products of 16 dwords (4 vectors k0..k3 of 8 bf16) with 16
// broadcast dwords: dword n comes from lane n of q's row.  Two accumulator
// chains (even / odd dwords).
#define PA_QK16                                                                             \
    "s_nop 1\n\t"                                                                           \
    PA_DOT2_BC("%0", "%2", "%3", "0") PA_DOT2_BC("%1", "%2", "%4", "1")                     \
    PA_DOT2_BC("%0", "%2", "%5", "2") PA_DOT2_BC("%1", "%2", "%6", "3")                     \
    PA_DOT2_BC("%0", "%2", "%7", "4") PA_DOT2_BC("%1", "%2", "%8", "5")                     \
    PA_DOT2_BC("%0", "%2", "%9", "6") PA_DOT2_BC("%1", "%2", "%10", "7")                    \
    PA_DOT2_BC("%0", "%2", "%11", "8") PA_DOT2_BC("%1", "%2", "%12", "9")                   \
    PA_DOT2_BC("%0", "%2", "%13", "10") PA_DOT2_BC("%1", "%2", "%14", "11")                 \
    PA_DOT2_BC("%0", "%2", "%15", "12") PA_DOT2_BC("%1", "%2", "%16", "13")                 \
    PA_DOT2_BC("%0", "%2", "%17", "14") PA_DOT2_BC("%1", "%2", "%18", "15")
#define PA_QK16_OPERANDS                                                                    \
    : "+v"(a), "+v"(b)                                                                      \
    : "v"(q), "v"(k0.x), "v"(k0.y), "v"(k0.z), "v"(k0.w), "v"(k1.x), "v"(k1.y), "v"(k1.z),  \
      "v"(k1.w), "v"(k2.x), "v"(k2.y), "v"(k2.z), "v"(k2.w), "v"(k3.x), "v"(k3.y), "v"(k3.z), \
      "v"(k3.w)

template <bool TAIL>
__device__ __forceinline__ void qk16(float &a, float &b, uint32_t q, const uint4 &k0,
                                     const uint4 &k1, const uint4 &k2, const uint4 &k3) {
    if constexpr (TAIL)
        asm volatile(PA_QK16 "s_nop 4\n\t" PA_QK16_OPERANDS);
    else
        asm volatile(PA_QK16 PA_QK16_OPERANDS);
}

// Two adjacent floats read / written as one 8-byte device-coherent access.
__device__ __forceinline__ float2 load_coherent2(const float *p) {
    const uint64_t w = __hip_atomic_load(reinterpret_cast<uint64_t *>(const_cast<float *>(p)),
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)w), __uint_as_float((uint32_t)(w >> 32)));
}
__device__ __forceinline__ void store_coherent2(float *p, float a, float b) {
    const uint64_t w = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), w, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte device-coherent global accesses (cache policy sc1: the access is
// coherent at agent scope, so data written by one workgroup is seen by
// another on any XCD) through a buffer resource covering `bytes` bytes from
// `base`.  0x00020000 is the gfx9 descriptor word 3 for raw (untyped)
// buffer access.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kCoherentSC1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float4 load_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kCoherentSC1);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                       __uint_as_float(v[3]));
}
__device__ __forceinline__ void store_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off,
                                                float a, float b, float c, float d) {
    const u32x4_t v = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)byte_off, 0, kCoherentSC1);
}

// Log-sum-exp merge of a split-KV partition set ("ROCm attention backends"
// blog, extend-path pseudocode: each chunk yields an output and an LSE and
// merge_attn_states combines them; the same merge combines decode
// partitions).  Rows row0 .. row0 + nrows - 1 of the output, each with
// nparts partials of D floats at part_out[(row * max_parts + k) * D] and
// LSEs at part_lse[row * max_parts + k].  Thread -> (row, DPT consecutive
// dims, DPT a multiple of 4); all partitions of a batch are fetched before
// any is used, so a batch costs one memory round trip.  Partitions combine
// in index order, so the result does not depend on which workgroup merges.
// Partials are read with device-coherent 16-byte loads (they were written by
// other workgroups of the same kernel), addressed from the first row so the
// offsets fit 32 bits.  NT: threads of the calling workgroup.
template <int D, int DPT, int BATCH, int NT>
__device__ __forceinline__ void merge_partition_rows(const float *part_out, const float *part_lse,
                                                     int max_parts, uint16_t *outp, float *lse,
                                                     size_t row0, int nrows, int nparts) {
    static_assert(DPT % 4 == 0, "16-byte partial loads");
    const auto rs = coherent_rsrc(part_out + row0 * max_parts * D,
                                  (uint32_t)nrows * max_parts * D * 4);
    for (int it = threadIdx.x; it < nrows * (D / DPT); it += NT) {
        const int h = it / (D / DPT), d0 = (it % (D / DPT)) * DPT;
        const size_t row = row0 + h;
        const float *pl = part_lse + row * max_parts;
        float M = kNegInf, den = 0.f, o[DPT];
#pragma unroll
        for (int e = 0; e < DPT; e++) o[e] = 0.f;
        for (int b = 0; b < nparts; b += BATCH) {
            float L[BATCH], x[BATCH][DPT];
#pragma unroll
            for (int u = 0; u < BATCH; u++) {
                const int pu = b + u < nparts ? b + u : b;  // always an in-range address
                L[u] = load_coherent(&pl[pu]);
#pragma unroll
                for (int e = 0; e < DPT; e += 4) {
                    const float4 v = load_coherent4(
                        rs, (uint32_t)(((h * max_parts + pu) * D + d0 + e) * 4));
                    x[u][e] = v.x;
                    x[u][e + 1] = v.y;
                    x[u][e + 2] = v.z;
                    x[u][e + 3] = v.w;
                }
            }
#pragma unroll
            for (int u = 0; u < BATCH; u++)
                if (b + u >= nparts) L[u] = kNegInf;
            float Mb = M;
#pragma unroll
            for (int u = 0; u < BATCH; u++) Mb = fmax_nc(Mb, L[u]);
            const float Mr = Mb == kNegInf ? 0.f : Mb;
            const float r = fast_exp2((M - Mr) * kLog2e);
            den *= r;
#pragma unroll
            for (int e = 0; e < DPT; e++) o[e] *= r;
#pragma unroll
            for (int u = 0; u < BATCH; u++) {
                const float w = fast_exp2((L[u] - Mr) * kLog2e);
                den += w;
#pragma unroll
                for (int e = 0; e < DPT; e++) o[e] += w * x[u][e];
            }
            M = Mb;
        }
        const float inv = den > 0.f ? 1.f / den : 0.f;
        uint32_t *out = reinterpret_cast<uint32_t *>(outp + row * D + d0);
#pragma unroll
        for (int e = 0; e < DPT; e += 2) out[e / 2] = pack_bf16x2(o[e] * inv, o[e + 1] * inv);
        if (d0 == 0 && lse) lse[row] = den > 0.f ? M + fast_log2(den) * kLn2 : kNegInf;
    }
}

}  // namespace pa
