// Pairwise log-sum-exp merge of two partial attention results
// (merge_attn_states in the extend-path pseudocode of the "ROCm attention
// backends" blog: every chunk yields an output and an LSE; the LSE carries
// the softmax denominator, so the merge is stable and the part with the
// larger scores dominates).
//
//   M = max(La, Lb), wa = exp(La - M), wb = exp(Lb - M)
//   O = (wa Oa + wb Ob) / (wa + wb),  L = M + log(wa + wb)
// A part with L = -inf has weight 0; two empty parts give O = 0, L = -inf.
//
// Pure streaming work: each thread moves one 8-element vector of a row
// (16 bytes of bf16 or 32 bytes of f32) from each input to the output.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

template <bool F32>
__device__ __forceinline__ void load8(const void *base, int64_t i, float v[8]) {
    if (F32) {
        const float4 *p = reinterpret_cast<const float4 *>(base) + 2 * i;
        const float4 x = p[0], y = p[1];
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
    } else {
        const uint4 w = reinterpret_cast<const uint4 *>(base)[i];
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    }
}

template <bool F32>
__device__ __forceinline__ void store8(void *base, int64_t i, const float v[8]) {
    if (F32) {
        float4 *p = reinterpret_cast<float4 *>(base) + 2 * i;
        p[0] = make_float4(v[0], v[1], v[2], v[3]);
        p[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
        uint4 w;
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        w.z = pack_bf16x2(v[4], v[5]);
        w.w = pack_bf16x2(v[6], v[7]);
        reinterpret_cast<uint4 *>(base)[i] = w;
    }
}

// out may alias a or b: each thread reads its vector of both inputs before
// writing the same vector of the output.
template <bool IN_F32, bool OUT_F32>
__global__ __launch_bounds__(256) void merge_pair_kernel(void *out, float *out_lse, const void *a,
                                                         const float *a_lse, const void *b,
                                                         const float *b_lse, int64_t rows,
                                                         int vecs_per_row) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * vecs_per_row) return;
    const int64_t row = idx / vecs_per_row;
    const int c = (int)(idx % vecs_per_row);
    const float la = a_lse[row], lb = b_lse[row];
    const float M = fmax_nc(la, lb);
    float o[8];
    float L;
    if (M == kNegInf) {
#pragma unroll
        for (int e = 0; e < 8; e++) o[e] = 0.f;
        L = kNegInf;
    } else {
        const float wa = fast_exp2((la - M) * kLog2e);  // la = -inf -> 0
        const float wb = fast_exp2((lb - M) * kLog2e);
        float va[8], vb[8];
        load8<IN_F32>(a, idx, va);
        load8<IN_F32>(b, idx, vb);
        const float inv = 1.f / (wa + wb);
        const float ca = wa * inv, cb = wb * inv;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            // an empty part may hold garbage: never multiply it by its zero weight
            const float x = wa == 0.f ? 0.f : ca * va[e];
            const float y = wb == 0.f ? 0.f : cb * vb[e];
            o[e] = x + y;
        }
        L = M + fast_log2(wa + wb) * kLn2;
    }
    store8<OUT_F32>(out, idx, o);
    if (c == 0 && out_lse) out_lse[row] = L;
}

}  // namespace

hipError_t launch_merge_pair(void *out, float *out_lse, int out_f32, const void *a,
                             const float *a_lse, const void *b, const float *b_lse, int in_f32,
                             int64_t rows, int D, hipStream_t stream) {
    const int vpr = D / 8;
    const int64_t total = rows * vpr;
    const int64_t grid = (total + 255) / 256;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
#define PA_MERGE_LAUNCH(I, O)                                                                   \
    hipLaunchKernelGGL((merge_pair_kernel<I, O>), dim3((unsigned)grid), dim3(256), 0, stream, out, \
                       out_lse, a, a_lse, b, b_lse, rows, vpr)
    if (in_f32) {
        if (out_f32) PA_MERGE_LAUNCH(true, true);
        else PA_MERGE_LAUNCH(true, false);
    } else {
        if (out_f32) PA_MERGE_LAUNCH(false, true);
        else PA_MERGE_LAUNCH(false, false);
    }
#undef PA_MERGE_LAUNCH
    return hipGetLastError();
}

}  // namespace pa
