// FP8 KV cache codes: OCP 8-bit E4M3 ("fn": no infinities, S.1111.111 is
// NaN, largest finite 448), one float32 scale per tensor.  The pages' MLA
// extend path gathers the context "and maybe dequantises" it ("vLLM ROCm
// attention backends" blog, AITER MLA section, extend pseudocode); the format
// is this library's reading:
//   value(code) = E4M3(code) * scale
//   code(x)     = nearest E4M3 to float32(x) * inv_scale, ties to the even
//                 code, saturating at +-448 (inv_scale = 1 / scale rounded
//                 to float32 once, on the host).
// In the shuffled layout an FP8 x-vector is 16 codes (16 bytes):
//   k_cache [num_blocks, kv_heads, head_dim / 16, block_size, 16]
//   v_cache [num_blocks, kv_heads, block_size / 16, head_dim, 16]
// gfx950's conversion instructions decode exactly this format
// (v_cvt_pk_f32_fp8, and v_cvt_scalef32_pk_bf16_fp8 with scale 1: every
// E4M3 value is a bf16).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace pa {

constexpr int kFp8X = 16;  // codes per 16-byte vector

// Nearest E4M3 code to y (finite), ties to the even code, saturating.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    if (a >= 448.f) return sign | 0x7Eu;
    if (a < 0.015625f)  // below 2^-6: multiples of 2^-9 (8 -> 0x08 = 2^-6)
        return sign | (uint32_t)__builtin_rintf(a * 512.f);
    const int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;  // -6 .. 8
    const float m = __uint_as_float(__float_as_uint(a) - ((uint32_t)e << 23));  // [1, 2)
    const uint32_t q = (uint32_t)__builtin_rintf((m - 1.f) * 8.f);  // 0 .. 8 (8 carries)
    const uint32_t code = ((uint32_t)(e + 7) << 3) + q;
    return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// Codes 4 w .. 4 w + 3 of a word -> two bf16 pairs (exact): lo gets codes 0, 1.
__device__ __forceinline__ void fp8x4_to_bf16x2(uint32_t w, uint32_t &lo, uint32_t &hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// Codes of a word -> 4 floats (exact).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float *f) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    f[0] = a[0];
    f[1] = a[1];
    f[2] = b[0];
    f[3] = b[1];
}

// float32 -> bf16 bits, round to nearest even (finite input).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// 16 bf16 (two 16-byte vectors) -> 16 codes under inv_scale.
__device__ __forceinline__ uint4 quantize16(const uint4 &a, const uint4 &b, float inv) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t w0 = w[2 * i], w1 = w[2 * i + 1];
        const uint32_t c0 = e4m3_encode(__uint_as_float(w0 << 16) * inv);
        const uint32_t c1 = e4m3_encode(__uint_as_float(w0 & 0xFFFF0000u) * inv);
        const uint32_t c2 = e4m3_encode(__uint_as_float(w1 << 16) * inv);
        const uint32_t c3 = e4m3_encode(__uint_as_float(w1 & 0xFFFF0000u) * inv);
        out[i] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

}  // namespace pa
