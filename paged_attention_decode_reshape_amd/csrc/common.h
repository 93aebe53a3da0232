// Internal device helpers shared by the gfx950 kernels of libpagedattn.
// Not part of the public ABI (that is include/pagedattn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// bf16 bits <-> f32 (bf16 -> f32 is exact; f32 -> bf16 rounds to nearest even).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 b = (__bf16)f;  // RNE (v_cvt_pk_bf16_f32 on gfx950)
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// c + a.lo * b.lo + a.hi * b.hi with bf16 pairs, f32 accumulate (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float fmax_nc(float a, float b) { return __builtin_fmaxf(a, b); }

// Read-only inputs viewed through the constant address space: the compiler
// then fetches wave-uniform addresses with scalar loads (s_load) into SGPRs.
template <typename T>
using cptr = __attribute__((address_space(4))) const T *;
template <typename T>
__device__ __forceinline__ cptr<T> as_const(const void *p) {
    return (cptr<T>)(p);
}

// Device-coherent (agent-scope) 4-byte accesses for data one workgroup
// writes and another, possibly on another XCD, reads in the same kernel.
// They bypass the per-XCD L2's write-back, so no cache-wide fence is needed.
__device__ __forceinline__ void store_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's outstanding stores have completed (been
// acknowledged); also a compiler barrier for memory.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier for reusing LDS: every wave's LDS accesses are done when
// any wave passes it.  Unlike __syncthreads() (whose workgroup-scope release
// also waits for the wave's global stores to be acknowledged) it leaves
// global stores in flight; a release that publishes them still has to wait
// for them itself.  Called by every wave of the workgroup.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A zero the compiler cannot see through.  Adding it to an address keeps a
// loop-invariant scalar load inside the loop (re-read from the scalar cache
// each iteration) instead of being hoisted and spilled.
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    return z;
}

// Cross-lane moves within a 16-lane row (DPP) and across rows (gfx950 swaps).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;   // row_ror:4
constexpr int kRowRor8 = 0x128;   // row_ror:8

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}

// Order-preserving map of non-NaN floats to int32 (and back): lets the max
// run on v_max_i32, which takes DPP operands directly.
__device__ __forceinline__ int f2ord(float f) {
    const int i = __float_as_int(f);
    return i >= 0 ? i : (i ^ 0x7fffffff);
}
__device__ __forceinline__ float ord2f(int i) { return __int_as_float(i >= 0 ? i : (i ^ 0x7fffffff)); }

// Every lane gets the max / sum over the 64 lanes of the wave (v must not be NaN).
__device__ __forceinline__ float wave_max(float v) {
    int k = f2ord(v);
    k = max(k, dpp_i<kQuadXor1>(k));
    k = max(k, dpp_i<kQuadXor2>(k));
    k = max(k, dpp_i<kRowRor4>(k));
    k = max(k, dpp_i<kRowRor8>(k));
    auto a = __builtin_amdgcn_permlane16_swap((unsigned)k, (unsigned)k, false, false);
    k = max((int)a[0], (int)a[1]);
    auto b = __builtin_amdgcn_permlane32_swap((unsigned)k, (unsigned)k, false, false);
    return ord2f(max((int)b[0], (int)b[1]));
}

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<kQuadXor1>(v);
    v += dpp_f<kQuadXor2>(v);
    v += dpp_f<kRowRor4>(v);
    v += dpp_f<kRowRor8>(v);
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}
__device__ __forceinline__ int readlane_i32(int v, int lane) {
    return __builtin_amdgcn_readlane(v, lane);
}
__device__ __forceinline__ float uniform_f(float v) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace pa
