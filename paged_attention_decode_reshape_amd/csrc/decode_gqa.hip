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
//       P.V a reduction over tokens inside a lane.  It runs as fp32 FMAs
//       (on gfx950 a wave64 fp32 FMA issues in half the cycles of a bf16
//       dot2, so fp32 weights cost no more than bf16 ones): each V vector is
//       widened once and shared by every head; the weights are permuted
//       (ds_bpermute) so that lane n of every row holds token 16 k + n and
//       are broadcast by DPP as above.
// Groups of more than 8 query heads are processed 8 heads at a time with
// the queries re-read from LDS.  The 4 waves' states merge in LDS.  A
// sequence longer than one partition writes fp32 partials (normalised
// output, LSE); the last workgroup of the sequence to finish merges them by
// log-sum-exp in partition order, so results are deterministic.
#include <type_traits>

#include "common.h"
#include "decode_common.h"
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


// head_dim 64: a lane holds 2 K vectors (8 dwords) and lane n (< 8) of its
// row holds the matching query dword.
#define PA_QK2H8_BODY                                                                       \
    "s_nop 1\n\t"                                                                           \
    PA_DOT2_BC("%0", "%4", "%6", "0") PA_DOT2_BC("%2", "%5", "%6", "0")                     \
    PA_DOT2_BC("%1", "%4", "%7", "1") PA_DOT2_BC("%3", "%5", "%7", "1")                     \
    PA_DOT2_BC("%0", "%4", "%8", "2") PA_DOT2_BC("%2", "%5", "%8", "2")                     \
    PA_DOT2_BC("%1", "%4", "%9", "3") PA_DOT2_BC("%3", "%5", "%9", "3")                     \
    PA_DOT2_BC("%0", "%4", "%10", "4") PA_DOT2_BC("%2", "%5", "%10", "4")                   \
    PA_DOT2_BC("%1", "%4", "%11", "5") PA_DOT2_BC("%3", "%5", "%11", "5")                   \
    PA_DOT2_BC("%0", "%4", "%12", "6") PA_DOT2_BC("%2", "%5", "%12", "6")                   \
    PA_DOT2_BC("%1", "%4", "%13", "7") PA_DOT2_BC("%3", "%5", "%13", "7") "s_nop 4\n\t"
#define PA_QK1H8_BODY                                                                       \
    "s_nop 1\n\t"                                                                           \
    PA_DOT2_BC("%0", "%2", "%3", "0") PA_DOT2_BC("%1", "%2", "%4", "1")                     \
    PA_DOT2_BC("%0", "%2", "%5", "2") PA_DOT2_BC("%1", "%2", "%6", "3")                     \
    PA_DOT2_BC("%0", "%2", "%7", "4") PA_DOT2_BC("%1", "%2", "%8", "5")                     \
    PA_DOT2_BC("%0", "%2", "%9", "6") PA_DOT2_BC("%1", "%2", "%10", "7") "s_nop 4\n\t"

__device__ __forceinline__ void qk8_2h(float &a0, float &a1, float &b0, float &b1, uint32_t qa,
                                       uint32_t qb, const uint4 &k0, const uint4 &k1) {
    asm volatile(PA_QK2H8_BODY
                 : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1)
                 : "v"(qa), "v"(qb), "v"(k0.x), "v"(k0.y), "v"(k0.z), "v"(k0.w), "v"(k1.x),
                   "v"(k1.y), "v"(k1.z), "v"(k1.w));
}

__device__ __forceinline__ void qk8_1h(float &a0, float &a1, uint32_t qa, const uint4 &k0,
                                       const uint4 &k1) {
    asm volatile(PA_QK1H8_BODY
                 : "+v"(a0), "+v"(a1)
                 : "v"(qa), "v"(k0.x), "v"(k0.y), "v"(k0.z), "v"(k0.w), "v"(k1.x), "v"(k1.y),
                   "v"(k1.z), "v"(k1.w));
}

// One v_fmac_f32 whose first operand is lane `n` of the same 16-lane row.
#define PA_FMA_BC(acc, r, v, n) \
    "v_fmac_f32_dpp " acc ", " r ", " v " row_newbcast:" n " row_mask:0xf bank_mask:0xf\n\t"

// PV over one group of 8 tokens: acc += p(token e) * v(token e), e = 0..7,
// where p of token e sits in lane N0 + e of every row of the p register
// (N0 = 0 or 8) and vf0 / vf1 hold the 8 tokens' values of dims lane and
// lane + 64 as fp32.  Bodies for two heads (a, b) and / or two dims.
#define PA_PV22_N0                                                                          \
    "s_nop 1\n\t"                                                                           \
    PA_FMA_BC("%0", "%4", "%6", "0") PA_FMA_BC("%2", "%5", "%6", "0")                       \
    PA_FMA_BC("%1", "%4", "%14", "0") PA_FMA_BC("%3", "%5", "%14", "0")                     \
    PA_FMA_BC("%0", "%4", "%7", "1") PA_FMA_BC("%2", "%5", "%7", "1")                       \
    PA_FMA_BC("%1", "%4", "%15", "1") PA_FMA_BC("%3", "%5", "%15", "1")                     \
    PA_FMA_BC("%0", "%4", "%8", "2") PA_FMA_BC("%2", "%5", "%8", "2")                       \
    PA_FMA_BC("%1", "%4", "%16", "2") PA_FMA_BC("%3", "%5", "%16", "2")                     \
    PA_FMA_BC("%0", "%4", "%9", "3") PA_FMA_BC("%2", "%5", "%9", "3")                       \
    PA_FMA_BC("%1", "%4", "%17", "3") PA_FMA_BC("%3", "%5", "%17", "3")                     \
    PA_FMA_BC("%0", "%4", "%10", "4") PA_FMA_BC("%2", "%5", "%10", "4")                     \
    PA_FMA_BC("%1", "%4", "%18", "4") PA_FMA_BC("%3", "%5", "%18", "4")                     \
    PA_FMA_BC("%0", "%4", "%11", "5") PA_FMA_BC("%2", "%5", "%11", "5")                     \
    PA_FMA_BC("%1", "%4", "%19", "5") PA_FMA_BC("%3", "%5", "%19", "5")                     \
    PA_FMA_BC("%0", "%4", "%12", "6") PA_FMA_BC("%2", "%5", "%12", "6")                     \
    PA_FMA_BC("%1", "%4", "%20", "6") PA_FMA_BC("%3", "%5", "%20", "6")                     \
    PA_FMA_BC("%0", "%4", "%13", "7") PA_FMA_BC("%2", "%5", "%13", "7")                     \
    PA_FMA_BC("%1", "%4", "%21", "7") PA_FMA_BC("%3", "%5", "%21", "7")
#define PA_PV22_N8                                                                          \
    "s_nop 1\n\t"                                                                           \
    PA_FMA_BC("%0", "%4", "%6", "8") PA_FMA_BC("%2", "%5", "%6", "8")                       \
    PA_FMA_BC("%1", "%4", "%14", "8") PA_FMA_BC("%3", "%5", "%14", "8")                     \
    PA_FMA_BC("%0", "%4", "%7", "9") PA_FMA_BC("%2", "%5", "%7", "9")                       \
    PA_FMA_BC("%1", "%4", "%15", "9") PA_FMA_BC("%3", "%5", "%15", "9")                     \
    PA_FMA_BC("%0", "%4", "%8", "10") PA_FMA_BC("%2", "%5", "%8", "10")                     \
    PA_FMA_BC("%1", "%4", "%16", "10") PA_FMA_BC("%3", "%5", "%16", "10")                   \
    PA_FMA_BC("%0", "%4", "%9", "11") PA_FMA_BC("%2", "%5", "%9", "11")                     \
    PA_FMA_BC("%1", "%4", "%17", "11") PA_FMA_BC("%3", "%5", "%17", "11")                   \
    PA_FMA_BC("%0", "%4", "%10", "12") PA_FMA_BC("%2", "%5", "%10", "12")                   \
    PA_FMA_BC("%1", "%4", "%18", "12") PA_FMA_BC("%3", "%5", "%18", "12")                   \
    PA_FMA_BC("%0", "%4", "%11", "13") PA_FMA_BC("%2", "%5", "%11", "13")                   \
    PA_FMA_BC("%1", "%4", "%19", "13") PA_FMA_BC("%3", "%5", "%19", "13")                   \
    PA_FMA_BC("%0", "%4", "%12", "14") PA_FMA_BC("%2", "%5", "%12", "14")                   \
    PA_FMA_BC("%1", "%4", "%20", "14") PA_FMA_BC("%3", "%5", "%20", "14")                   \
    PA_FMA_BC("%0", "%4", "%13", "15") PA_FMA_BC("%2", "%5", "%13", "15")                   \
    PA_FMA_BC("%1", "%4", "%21", "15") PA_FMA_BC("%3", "%5", "%21", "15")
#define PA_PV12_N0                                                                          \
    "s_nop 1\n\t"                                                                           \
    PA_FMA_BC("%0", "%2", "%3", "0") PA_FMA_BC("%1", "%2", "%11", "0")                      \
    PA_FMA_BC("%0", "%2", "%4", "1") PA_FMA_BC("%1", "%2", "%12", "1")                      \
    PA_FMA_BC("%0", "%2", "%5", "2") PA_FMA_BC("%1", "%2", "%13", "2")                      \
    PA_FMA_BC("%0", "%2", "%6", "3") PA_FMA_BC("%1", "%2", "%14", "3")                      \
    PA_FMA_BC("%0", "%2", "%7", "4") PA_FMA_BC("%1", "%2", "%15", "4")                      \
    PA_FMA_BC("%0", "%2", "%8", "5") PA_FMA_BC("%1", "%2", "%16", "5")                      \
    PA_FMA_BC("%0", "%2", "%9", "6") PA_FMA_BC("%1", "%2", "%17", "6")                      \
    PA_FMA_BC("%0", "%2", "%10", "7") PA_FMA_BC("%1", "%2", "%18", "7")
#define PA_PV12_N8                                                                          \
    "s_nop 1\n\t"                                                                           \
    PA_FMA_BC("%0", "%2", "%3", "8") PA_FMA_BC("%1", "%2", "%11", "8")                      \
    PA_FMA_BC("%0", "%2", "%4", "9") PA_FMA_BC("%1", "%2", "%12", "9")                      \
    PA_FMA_BC("%0", "%2", "%5", "10") PA_FMA_BC("%1", "%2", "%13", "10")                    \
    PA_FMA_BC("%0", "%2", "%6", "11") PA_FMA_BC("%1", "%2", "%14", "11")                    \
    PA_FMA_BC("%0", "%2", "%7", "12") PA_FMA_BC("%1", "%2", "%15", "12")                    \
    PA_FMA_BC("%0", "%2", "%8", "13") PA_FMA_BC("%1", "%2", "%16", "13")                    \
    PA_FMA_BC("%0", "%2", "%9", "14") PA_FMA_BC("%1", "%2", "%17", "14")                    \
    PA_FMA_BC("%0", "%2", "%10", "15") PA_FMA_BC("%1", "%2", "%18", "15")
#define PA_PV21_N0                                                                          \
    "s_nop 1\n\t"                                                                           \
    PA_FMA_BC("%0", "%2", "%4", "0") PA_FMA_BC("%1", "%3", "%4", "0")                       \
    PA_FMA_BC("%0", "%2", "%5", "1") PA_FMA_BC("%1", "%3", "%5", "1")                       \
    PA_FMA_BC("%0", "%2", "%6", "2") PA_FMA_BC("%1", "%3", "%6", "2")                       \
    PA_FMA_BC("%0", "%2", "%7", "3") PA_FMA_BC("%1", "%3", "%7", "3")                       \
    PA_FMA_BC("%0", "%2", "%8", "4") PA_FMA_BC("%1", "%3", "%8", "4")                       \
    PA_FMA_BC("%0", "%2", "%9", "5") PA_FMA_BC("%1", "%3", "%9", "5")                       \
    PA_FMA_BC("%0", "%2", "%10", "6") PA_FMA_BC("%1", "%3", "%10", "6")                     \
    PA_FMA_BC("%0", "%2", "%11", "7") PA_FMA_BC("%1", "%3", "%11", "7")
#define PA_PV21_N8                                                                          \
    "s_nop 1\n\t"                                                                           \
    PA_FMA_BC("%0", "%2", "%4", "8") PA_FMA_BC("%1", "%3", "%4", "8")                       \
    PA_FMA_BC("%0", "%2", "%5", "9") PA_FMA_BC("%1", "%3", "%5", "9")                       \
    PA_FMA_BC("%0", "%2", "%6", "10") PA_FMA_BC("%1", "%3", "%6", "10")                     \
    PA_FMA_BC("%0", "%2", "%7", "11") PA_FMA_BC("%1", "%3", "%7", "11")                     \
    PA_FMA_BC("%0", "%2", "%8", "12") PA_FMA_BC("%1", "%3", "%8", "12")                     \
    PA_FMA_BC("%0", "%2", "%9", "13") PA_FMA_BC("%1", "%3", "%9", "13")                     \
    PA_FMA_BC("%0", "%2", "%10", "14") PA_FMA_BC("%1", "%3", "%10", "14")                   \
    PA_FMA_BC("%0", "%2", "%11", "15") PA_FMA_BC("%1", "%3", "%11", "15")
#define PA_PV11_N0                                                                          \
    "s_nop 1\n\t"                                                                           \
    PA_FMA_BC("%0", "%1", "%2", "0")                                                        \
    PA_FMA_BC("%0", "%1", "%3", "1")                                                        \
    PA_FMA_BC("%0", "%1", "%4", "2")                                                        \
    PA_FMA_BC("%0", "%1", "%5", "3")                                                        \
    PA_FMA_BC("%0", "%1", "%6", "4")                                                        \
    PA_FMA_BC("%0", "%1", "%7", "5")                                                        \
    PA_FMA_BC("%0", "%1", "%8", "6")                                                        \
    PA_FMA_BC("%0", "%1", "%9", "7")
#define PA_PV11_N8                                                                          \
    "s_nop 1\n\t"                                                                           \
    PA_FMA_BC("%0", "%1", "%2", "8")                                                        \
    PA_FMA_BC("%0", "%1", "%3", "9")                                                        \
    PA_FMA_BC("%0", "%1", "%4", "10")                                                       \
    PA_FMA_BC("%0", "%1", "%5", "11")                                                       \
    PA_FMA_BC("%0", "%1", "%6", "12")                                                       \
    PA_FMA_BC("%0", "%1", "%7", "13")                                                       \
    PA_FMA_BC("%0", "%1", "%8", "14")                                                       \
    PA_FMA_BC("%0", "%1", "%9", "15")
#define PA_VF8(v) "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7])
#define PA_PV_ASM(BODY, ...)                             \
    do {                                                 \
        if constexpr (TAIL)                              \
            asm volatile(BODY "s_nop 4\n\t" __VA_ARGS__); \
        else                                             \
            asm volatile(BODY __VA_ARGS__);              \
    } while (0)

template <bool N8, bool TAIL>
__device__ __forceinline__ void pv22(float &a0, float &a1, float &b0, float &b1, uint32_t pa,
                                     uint32_t pb, const float (&v0)[8], const float (&v1)[8]) {
    if constexpr (N8)
        PA_PV_ASM(PA_PV22_N8, : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1) : "v"(pa), "v"(pb), PA_VF8(v0), PA_VF8(v1));
    else
        PA_PV_ASM(PA_PV22_N0, : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1) : "v"(pa), "v"(pb), PA_VF8(v0), PA_VF8(v1));
}

template <bool N8, bool TAIL>
__device__ __forceinline__ void pv12(float &a0, float &a1, uint32_t pa, const float (&v0)[8],
                                     const float (&v1)[8]) {
    if constexpr (N8)
        PA_PV_ASM(PA_PV12_N8, : "+v"(a0), "+v"(a1) : "v"(pa), PA_VF8(v0), PA_VF8(v1));
    else
        PA_PV_ASM(PA_PV12_N0, : "+v"(a0), "+v"(a1) : "v"(pa), PA_VF8(v0), PA_VF8(v1));
}

template <bool N8, bool TAIL>
__device__ __forceinline__ void pv21(float &a0, float &b0, uint32_t pa, uint32_t pb,
                                     const float (&v0)[8]) {
    if constexpr (N8)
        PA_PV_ASM(PA_PV21_N8, : "+v"(a0), "+v"(b0) : "v"(pa), "v"(pb), PA_VF8(v0));
    else
        PA_PV_ASM(PA_PV21_N0, : "+v"(a0), "+v"(b0) : "v"(pa), "v"(pb), PA_VF8(v0));
}

template <bool N8, bool TAIL>
__device__ __forceinline__ void pv11(float &a0, uint32_t pa, const float (&v0)[8]) {
    if constexpr (N8)
        PA_PV_ASM(PA_PV11_N8, : "+v"(a0) : "v"(pa), PA_VF8(v0));
    else
        PA_PV_ASM(PA_PV11_N0, : "+v"(a0) : "v"(pa), PA_VF8(v0));
}

// fp32 values of the 8 tokens in a V vector (token 2w in the low half of word w)
__device__ __forceinline__ void widen8(const uint4 &v, float (&f)[8]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// PV of one token group for one head pair (PAIRS) or one head; `odd`
// selects lanes 8..15 of the p registers, `last` ends the block with the
// wait that plain code reading the accumulators needs.
template <int DV, bool PAIRS>
__device__ __forceinline__ void pv_step(int odd, bool last, float (&a)[DV], float (&b)[DV],
                                        uint32_t pa, uint32_t pb, const float (&vf)[DV][8]) {
#define PA_PV_CALL(N8, T)                                                  \
    do {                                                                   \
        if constexpr (PAIRS && DV == 2) pv22<N8, T>(a[0], a[1], b[0], b[1], pa, pb, vf[0], vf[1]); \
        else if constexpr (PAIRS) pv21<N8, T>(a[0], b[0], pa, pb, vf[0]);  \
        else if constexpr (DV == 2) pv12<N8, T>(a[0], a[1], pa, vf[0], vf[1]); \
        else pv11<N8, T>(a[0], pa, vf[0]);                                 \
    } while (0)
    if (odd) {
        if (last) PA_PV_CALL(true, true);
        else PA_PV_CALL(true, false);
    } else {
        if (last) PA_PV_CALL(false, true);
        else PA_PV_CALL(false, false);
    }
#undef PA_PV_CALL
}

// Sum over the 4 rows of the wave (lanes n, n + 16, n + 32, n + 48); every
// lane gets the sum for its column.
__device__ __forceinline__ float row_sum4(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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

constexpr int kSub = 16;  // tokens per sub-block: one row of lanes

// K of one 16-token sub-block: lane (row, col) loads token `col`'s vectors
// row * CQ .. row * CQ + CQ - 1 (a quarter of the dims).  `half` selects the
// 16-token half of a 32-token block.
template <int D, int B>
__device__ __forceinline__ void load_k_sub(const uint4 *kc, size_t tile, int half, int row,
                                           int col, uint4 (&kq)[D / 32]) {
    constexpr int C = D / 8, CQ = D / 32;
    const uint4 *kt = kc + tile * (size_t)(C * B) + half * kSub + col;
#pragma unroll
    for (int i = 0; i < CQ; i++) kq[i] = kt[(row * CQ + i) * B];
}

// V of one 16-token sub-block: its two 8-token groups for dims lane + 64 jj.
template <int D, int B>
__device__ __forceinline__ void load_v_sub(const uint4 *vc, size_t tile, int half, int lane,
                                           uint4 (&vv)[2][D / 64]) {
    constexpr int DV = D / 64;
    const uint4 *vt = vc + (tile * (B / 8) + half * 2) * D + lane;
#pragma unroll
    for (int tg = 0; tg < 2; tg++)
#pragma unroll
        for (int jj = 0; jj < DV; jj++) vv[tg][jj] = vt[tg * D + 64 * jj];
}

// One workgroup (4 waves) per (partition, kv head, sequence).  A wave owns
// every 4th chunk of SUBS 16-token sub-blocks of the partition.  Per chunk
// it loads the sub-blocks' K (one 16-byte vector per lane per load) and V,
// computes all SUBS x G scores, takes their exact max, and accumulates P.V;
// the next chunk's K loads are issued as soon as the current K is consumed,
// and its V loads as soon as the current V is.
template <int D, int B, int G, int SUBS>
__global__ __launch_bounds__(256, 2) void paged_decode_kernel(DecodeParams p) {
    constexpr int CQ = D / 32;        // K vectors per lane per sub-block
    constexpr int DV = D / 64;        // output dims per lane
    constexpr int QW = 4 * CQ;        // query dwords per row
    constexpr int kChunk = kSub * SUBS;
    constexpr bool kPairs = G >= 2;
    constexpr int HS = kPairs ? 2 : 1;

    const int units = p.S * p.Hkv;
    const int part = blockIdx.x / units;
    const int rem = blockIdx.x - part * units;
    const int s = rem / p.Hkv, g = rem - s * p.Hkv;
    const int Ga = p.Hq / p.Hkv;
    const int P = p.partition;
    const int start = part * P;
    // the wave index as a scalar, so per-wave token offsets stay in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int row = lane >> 4, col = lane & 15;
    uint16_t *out = reinterpret_cast<uint16_t *>(p.out);

    // Issued together, before anything waits: the context length, the
    // block-table entry of this wave's sub-block `lane` (index clamped into
    // the table, validity decided once the length is known) and the queries.
    // Sub-block k of the wave is sub-block k % SUBS of its chunk k / SUBS.
    const int ctx_raw = as_const<int32_t>(p.context_lens)[s];
    const int t0_lane = start + (kWaves * (lane / SUBS) + wave) * kChunk + kSub * (lane % SUBS);
    const int bt_raw =
        p.block_table[(size_t)s * p.max_blocks + min(t0_lane / B, p.max_blocks - 1)];
    uint32_t qreg[G];
    {
        const uint32_t *qg = reinterpret_cast<const uint32_t *>(p.query) +
                             ((size_t)s * p.Hq + (size_t)g * Ga) * (D / 2) + row * QW + (col % QW);
#pragma unroll
        for (int h = 0; h < G; h++) qreg[h] = qg[(h < Ga ? h : h - Ga) * (D / 2)];
    }
    const int ctx = clamp_ctx(ctx_raw, p.max_blocks, B, p.max_parts, P);

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

    // lane k: physical block of sub-block k, -1 past the end or out of range.
    // Validity is monotone in k, so the valid sub-blocks are 0 .. nmine - 1.
    const bool lane_ok = t0_lane < end;
    const int bid = lane_ok && bt_raw >= 0 && (int64_t)bt_raw < p.num_blocks ? bt_raw : -1;
    const int nmine = __popcll(__ballot(lane_ok));
    const int nch = (nmine + SUBS - 1) / SUBS;
    const uint4 *kc = reinterpret_cast<const uint4 *>(p.k_cache);
    const uint4 *vc = reinterpret_cast<const uint4 *>(p.v_cache);

    float m[G], lsum[G], acc[G][DV];
#pragma unroll
    for (int h = 0; h < G; h++) {
        m[h] = kNegInf;
        lsum[h] = 0.f;
#pragma unroll
        for (int jj = 0; jj < DV; jj++) acc[h][jj] = 0.f;
    }

    uint4 kb[SUBS][CQ], vb[SUBS][2][DV];
    // Sub-block k's block and token offset; a sub-block past the end re-reads
    // the wave's last valid one (a cache hit) so every chunk issues the same loads.
    auto locate = [&](int k, size_t &tile, int &half) {
        const int kk = min(k, nmine - 1);
        const int b = readlane_i32(bid, kk);
        const int t0 = start + (kWaves * (kk / SUBS) + wave) * kChunk + kSub * (kk % SUBS);
        tile = (size_t)(b < 0 ? 0 : b) * p.Hkv + g;
        half = (t0 % B) / kSub;
    };
    auto issue_k = [&](int c) {
#pragma unroll
        for (int j = 0; j < SUBS; j++) {
            size_t tile;
            int half;
            locate(c * SUBS + j, tile, half);
            load_k_sub<D, B>(kc, tile, half, row, col, kb[j]);
        }
    };
    auto issue_v = [&](int c) {
#pragma unroll
        for (int j = 0; j < SUBS; j++) {
            size_t tile;
            int half;
            locate(c * SUBS + j, tile, half);
            load_v_sub<D, B>(vc, tile, half, lane, vb[j]);
        }
    };

    // One chunk: all of its K and V loads are issued first (V lands while
    // the scores are computed), then QK, softmax, PV.  Buffers are not
    // carried across chunks; the other waves of the SIMD cover the latency.
    auto chunk = [&](int c) {
        issue_k(c);
        issue_v(c);
        int nvalid[SUBS];
#pragma unroll
        for (int j = 0; j < SUBS; j++) {
            const int k = c * SUBS + j;
            const int t0 = start + (kWaves * c + wave) * kChunk + kSub * j;
            nvalid[j] = readlane_i32(bid, k) < 0 ? 0 : min(kSub, end - t0);
        }
        // QK: each lane sums a quarter of the dims; the rows are then summed,
        // leaving every row with the 16 scores of the sub-block
        float sc[SUBS][G];
#pragma unroll
        for (int j = 0; j < SUBS; j++) {
            float a[G][2];
#pragma unroll
            for (int h = 0; h < G; h++) a[h][0] = a[h][1] = 0.f;
#pragma unroll
            for (int h = 0; h < G; h += HS) {
                if constexpr (kPairs) {
                    if constexpr (CQ == 4) {
                        if (h + 2 >= G)
                            qk_2h<true>(a[h][0], a[h][1], a[h + 1][0], a[h + 1][1], qreg[h],
                                        qreg[h + 1], kb[j][0], kb[j][1], kb[j][2], kb[j][3]);
                        else
                            qk_2h<false>(a[h][0], a[h][1], a[h + 1][0], a[h + 1][1], qreg[h],
                                         qreg[h + 1], kb[j][0], kb[j][1], kb[j][2], kb[j][3]);
                    } else {
                        qk8_2h(a[h][0], a[h][1], a[h + 1][0], a[h + 1][1], qreg[h], qreg[h + 1],
                               kb[j][0], kb[j][1]);
                    }
                } else {
                    if constexpr (CQ == 4)
                        qk_1h<true>(a[h][0], a[h][1], qreg[h], kb[j][0], kb[j][1], kb[j][2],
                                    kb[j][3]);
                    else
                        qk8_1h(a[h][0], a[h][1], qreg[h], kb[j][0], kb[j][1]);
                }
            }
            dpp_result_fence<2 * G>(&a[0][0]);
            const bool ok = col < nvalid[j];
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float z = row_sum4(a[h][0] + a[h][1]);
                sc[j][h] = ok ? z * sl2 : kNegInf;
            }
        }
        // softmax: exact max over the chunk, one rescale of the running state
        uint32_t pw[SUBS][G];
#pragma unroll
        for (int h = 0; h < G; h++) {
            float mx = sc[0][h];
#pragma unroll
            for (int j = 1; j < SUBS; j++) mx = fmax_nc(mx, sc[j][h]);
            mx = uniform_f(row_max16(mx));
            const float mn = fmax_nc(m[h], mx);
            const float mref = mn == kNegInf ? 0.f : mn;
            const float alpha = fast_exp2(m[h] - mref);
            m[h] = mn;
            float l = lsum[h] * alpha;
#pragma unroll
            for (int j = 0; j < SUBS; j++) {
                const float pr = fast_exp2(sc[j][h] - mref);
                l += pr;
                pw[j][h] = __float_as_uint(pr);
            }
            lsum[h] = l;
#pragma unroll
            for (int jj = 0; jj < DV; jj++) acc[h][jj] *= alpha;
        }
        // PV: the V of tokens past the end is zeroed (weight 0, data may be anything)
#pragma unroll
        for (int j = 0; j < SUBS; j++) {
            if (nvalid[j] < kSub) {
#pragma unroll
                for (int tg = 0; tg < 2; tg++) {
                    const int nv = nvalid[j] - 8 * tg;
#pragma unroll
                    for (int jj = 0; jj < DV; jj++) {
                        uint4 &v = vb[j][tg][jj];
                        v.x = mask_pair(v.x, 0, nv);
                        v.y = mask_pair(v.y, 2, nv);
                        v.z = mask_pair(v.z, 4, nv);
                        v.w = mask_pair(v.w, 6, nv);
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < SUBS; j++) {
#pragma unroll
            for (int tg = 0; tg < 2; tg++) {
                float vf[DV][8];
#pragma unroll
                for (int jj = 0; jj < DV; jj++) widen8(vb[j][tg][jj], vf[jj]);
#pragma unroll
                for (int h = 0; h < G; h += HS) {
                    const bool last = j == SUBS - 1 && tg == 1 && h + HS >= G;
                    pv_step<DV, kPairs>(tg, last, acc[h], acc[h + HS - 1], pw[j][h],
                                        pw[j][h + HS - 1], vf);
                }
            }
        }
        dpp_result_fence<G * DV>(&acc[0][0]);
    };

    for (int c = 0; c < nch; c++) chunk(c);

    // merge the 4 waves of the workgroup (every row holds the same token
    // weights, so a wave's sum is 4 x the row sum)
    __shared__ float sm_m[kWaves][G], sm_l[kWaves][G];
    __shared__ float sm_acc[kWaves][G][D];
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float l = wave_sum(lsum[h]) * 0.25f;
        if (lane == 0) {
            sm_m[wave][h] = m[h];
            sm_l[wave][h] = l;
        }
#pragma unroll
        for (int jj = 0; jj < DV; jj++) sm_acc[wave][h][lane + 64 * jj] = acc[h][jj];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < Ga * (D / 2); idx += blockDim.x) {
        const int h = idx / (D / 2), d = 2 * (idx % (D / 2));
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; w++) M = fmax_nc(M, sm_m[w][h]);
        const float Mr = M == kNegInf ? 0.f : M;
        float n0 = 0.f, n1 = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            const float wt = fast_exp2(sm_m[w][h] - Mr);
            n0 += wt * sm_acc[w][h][d];
            n1 += wt * sm_acc[w][h][d + 1];
            den += wt * sm_l[w][h];
        }
        const float inv = den > 0.f ? 1.f / den : 0.f;
        const float L = den > 0.f ? (M + fast_log2(den)) * kLn2 : kNegInf;
        const size_t orow = (size_t)s * p.Hq + (size_t)g * Ga + h;
        if (nparts == 1) {
            reinterpret_cast<uint32_t *>(out + orow * D)[d / 2] = pack_bf16x2(n0 * inv, n1 * inv);
            if (d == 0 && p.lse) p.lse[orow] = L;
        } else {
            store_coherent2(&p.part_out[(orow * p.max_parts + part) * D + d], n0 * inv, n1 * inv);
            if (d == 0) store_coherent(&p.part_lse[orow * p.max_parts + part], L);
        }
    }
    if (nparts == 1) return;

    // The last workgroup of this (sequence, kv head) to finish merges all of
    // its partitions.  Partials are written and read with device-coherent
    // (agent-scope) accesses, so no cache-wide fence is needed: each thread
    // waits for its partial stores to complete, then one thread counts.
    __shared__ int sm_last;
    wait_stores();
    __syncthreads();
    int *counter = p.counters + (size_t)s * p.Hkv + g;
    if (threadIdx.x == 0)
        sm_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  nparts - 1;
    __syncthreads();
    if (!sm_last) return;
    if (threadIdx.x == 0)  // leave the counter zero for the next call
        __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    constexpr int kDPT = G * D / 256 > 4 ? G * D / 256 : 4;
    merge_partition_rows<D, kDPT, (kDPT > 4 ? 4 : 8)>(p.part_out, p.part_lse, p.max_parts,
                                                      reinterpret_cast<uint16_t *>(p.out), p.lse,
                                                      (size_t)s * p.Hq + (size_t)g * Ga, Ga, nparts);
}

template <int D, int B, int G>
hipError_t launch_partition(const DecodeParams &p, hipStream_t stream) {
    const int64_t units = (int64_t)p.max_parts * p.S * p.Hkv;
    if (units > 0x7fffffff) return hipErrorInvalidValue;
    constexpr int kSubs = G >= 16 ? 2 : 4;
    hipLaunchKernelGGL((paged_decode_kernel<D, B, G, kSubs>), dim3((unsigned)units), dim3(256), 0,
                       stream, p);
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
    if (p.D == 128)
        return p.B == 16 ? dispatch_group<128, 16>(p, stream) : dispatch_group<128, 32>(p, stream);
    return p.B == 16 ? dispatch_group<64, 16>(p, stream) : dispatch_group<64, 32>(p, stream);
}

}  // namespace pa
