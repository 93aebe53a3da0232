// GQA / MHA paged decode attention over the preshuffled KV cache.
//
// Decode is memory-bound: every step streams the whole KV cache of every
// sequence once ("ROCm attention backends" blog, phase taxonomy; the
// decode path reads the shuffled cache directly).  Each K/V byte is read
// exactly once, as a 16-byte vector, and the arithmetic runs on the VALU as
// bf16 dot2 instructions whose broadcast operand comes through DPP.
//
// Two ways to split the work over workgroups of 4 waves:
//   balanced  a fixed grid (a few workgroups per CU) shares the 16-token
//       sub-blocks of all (sequence, kv head) units equally, so every CU
//       streams the same number of bytes whatever the length mix;
//   partitioned  one workgroup per (fixed-length partition, kv head,
//       sequence), the 1-D grid ordered partition-major so the units of one
//       partition index spread over all XCDs.
// Within a range, the waves take chunks of SUBS 16-token sub-blocks
// round-robin.  A sub-block occupies a wave as 4 rows x 16 lanes:
//   QK  lane (row r, column n) loads token n's K vectors for a quarter of
//       head_dim (k_cache[p][g][c][o][0..8), 8 consecutive dims of one
//       token, as 16-byte loads).  The group's queries sit in VGPRs laid out
//       so that lane n of a row holds query dword n of the row's slice; DPP
//       row_newbcast hands it to the whole row inside v_dot2c.  The 4 rows'
//       partial dots are added with permlane swaps, which leaves every row
//       holding the 16 scores (column n: token n).
//   softmax  exact max over the chunk (integer-ordered DPP max), one online
//       rescale per chunk, p = exp2(z - m) with log2(e) folded into the
//       scale; the weights stay fp32.
//   PV  lane l owns dims l (and l + 64).  A V vector
//       (v_cache[p][g][j][d][0..8), 8 consecutive tokens of one dim) makes
//       P.V a reduction over tokens inside a lane: fp32 FMAs whose weight
//       operand (token n's p, in column n of every row) comes through DPP
//       row_newbcast.  Each V vector is widened once and shared by every head.
// The 4 waves' states merge in LDS.  A unit split over several workgroups
// writes fp32 partials (normalised output, LSE); the last workgroup of the
// unit to finish merges them by log-sum-exp in token order, so results are
// deterministic.
#include <type_traits>

#include "common.h"
#include "decode_common.h"
#include "fp8.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
// cache layouts the kernels are built for (DecodeParams::layout)
constexpr int kLayShuffled = 0, kLayStd = 1, kLayFp8 = 2;
constexpr int kStep = 64;  // tokens per wave step

// context length limited to the host's bound and what the block table covers
template <int B>
__device__ __forceinline__ int clamp_ctx(const DecodeParams &p, int ctx) {
    const int64_t cap = min((int64_t)p.max_blocks * B, (int64_t)p.max_ctx);
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

// s_waitcnt vmcnt(N) as a builtin, so the compiler's own wait insertion
// knows about it (expcnt and lgkmcnt left at their maximum: no wait).
template <int N>
__device__ __forceinline__ void wait_vm_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

constexpr int kSub = 16;  // tokens per sub-block: one row of lanes
constexpr float kLazyLog2 = 8.f;  // softmax reference lag allowed (log2 units)

// K and V of one 16-token sub-block come through buffer loads: the block's
// address is a scalar descriptor base and each lane's offset inside the
// block is the same for every sub-block, so no address register is
// rewritten while earlier loads are in flight (which would make the
// compiler wait for them).  `half` selects the 16-token half of a
// 32-token block.  The descriptor covers exactly the sub-block's bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
// Cache policy of the KV tile loads.  In the preshuffled layouts every load
// instruction covers whole cache lines (a K instruction 4 runs of 16 tokens'
// 16-byte vectors, a V instruction 64 consecutive vectors) and each line is
// read once per launch, so those loads skip the vector L1 (sc0) and are
// marked non-temporal in L2 (nt): 3% faster on the 64-request decode and 1-2%
// on the long-context one than the default policy.  The standard layout
// reads a token's row in four instructions, which the L1 serves together:
// there the default policy is kept (sc0 + nt made it 30% slower).
constexpr int kStreamPolicy = 1 | 2, kCachedPolicy = 0;
template <int POLICY = kStreamPolicy>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POLICY);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// K: lane (row, col) loads token `col`'s vectors row * CQ .. row * CQ + CQ - 1
// (a quarter of the dims) from k_cache[tile][c][o][0..8).
// A load that is not `live` gets a descriptor of 0 bytes: it is issued (so
// the buffers are redefined on every path) but touches no memory and
// returns zeros.
template <int D, int B>
__device__ __forceinline__ void load_k_sub(const char *k_cache, size_t tile, int half, bool live,
                                           uint32_t lane_off, uint4 (&kq)[D / 32]) {
    constexpr int CQ = D / 32;
    const char *base = k_cache + (tile * (size_t)(D * B) + half * kSub * 8) * 2;
    const auto r = tile_rsrc(base, live ? (uint32_t)(D * B * 2 - half * kSub * 16) : 0u);
#pragma unroll
    for (int i = 0; i < CQ; i++) kq[i] = buf_load16(r, lane_off + i * B * 16);
}
// byte offset of lane (row, col) inside a K tile
template <int D, int B>
__device__ __forceinline__ uint32_t k_lane_off(int row, int col) {
    return (uint32_t)((row * (D / 32) * B + col) * 16);
}

// V: the sub-block's two 8-token groups for dims lane + 64 jj, from
// v_cache[tile][j][d][0..8).
template <int D, int B>
__device__ __forceinline__ void load_v_sub(const char *v_cache, size_t tile, int half, bool live,
                                           uint32_t lane_off, uint4 (&vv)[2][D / 64]) {
    constexpr int DV = D / 64;
    const char *base = v_cache + ((tile * (B / 8) + half * 2) * (size_t)D) * 16;
    const auto r = tile_rsrc(base, live ? (uint32_t)(2 * D * 16) : 0u);
#pragma unroll
    for (int tg = 0; tg < 2; tg++)
#pragma unroll
        for (int jj = 0; jj < DV; jj++) vv[tg][jj] = buf_load16(r, lane_off + (tg * D + 64 * jj) * 16);
}

// Standard layout [num_blocks, block_size, kv_heads, head_dim] (the layout
// the shuffled one replaces, kept for comparing the two): token o of block
// b, head g, is the row of head_dim bf16 at ((b * B + o) * Hkv + g) * D.
// K and V are both read like the shuffled K: lane (row, col) loads token
// `col`'s vectors row * CQ .. row * CQ + CQ - 1 (CQ = D / 32), so K lands in
// the same registers as from the shuffled cache.  `first` is the
// sub-block's first row ((b * B + 16 half) * Hkv + g).
template <int D>
__device__ __forceinline__ void load_rows_std(const char *cache, size_t first, int Hkv, bool live,
                                              uint32_t lane_off, uint4 (&kq)[D / 32]) {
    constexpr int CQ = D / 32;
    const char *base = cache + first * (size_t)D * 2;
    const auto r = tile_rsrc(base, live ? (uint32_t)((15 * Hkv + 1) * D * 2) : 0u);
#pragma unroll
    for (int i = 0; i < CQ; i++) kq[i] = buf_load16<kCachedPolicy>(r, lane_off + i * 16);
}
// byte offset of lane (row, col) inside a standard-layout sub-block
template <int D>
__device__ __forceinline__ uint32_t std_lane_off(int row, int col, int Hkv) {
    return (uint32_t)((col * Hkv * D + row * (D / 32) * 8) * 2);
}

// FP8 shuffled layout (x = 16): lane (row, col) loads token `col`'s K vectors
// row * CQ8 .. row * CQ8 + CQ8 - 1 (CQ8 = D / 64; 16 dims each) from
// k_cache[tile][c][o][0..16), and lane l the V vector of dim l + 64 jj
// (the sub-block's 16 tokens) from v_cache[tile][o / 16][d][0..16).
template <int D, int B>
__device__ __forceinline__ void load_k_sub8(const char *k_cache, size_t tile, int half, bool live,
                                            uint32_t lane_off, uint4 (&kq)[D / 32]) {
    constexpr int CQ8 = D / 64;
    const char *base = k_cache + tile * (size_t)(D * B) + half * kSub * kFp8X;
    const auto r = tile_rsrc(base, live ? (uint32_t)(D * B - half * kSub * kFp8X) : 0u);
#pragma unroll
    for (int i = 0; i < CQ8; i++) kq[i] = buf_load16(r, lane_off + i * B * 16);
}
template <int D, int B>
__device__ __forceinline__ void load_v_sub8(const char *v_cache, size_t tile, int half, bool live,
                                            uint32_t lane_off, uint4 (&vv)[2][D / 64]) {
    constexpr int DV = D / 64;
    const char *base = v_cache + ((tile * (B / kFp8X) + half) * (size_t)D) * kFp8X;
    const auto r = tile_rsrc(base, live ? (uint32_t)(D * kFp8X) : 0u);
#pragma unroll
    for (int jj = 0; jj < DV; jj++) vv[0][jj] = buf_load16(r, lane_off + 64 * jj * 16);
}
// 16 FP8 K codes per vector -> the bf16 pairs the QK blocks read (exact)
template <int D>
__device__ __forceinline__ void k_fp8_to_bf16(const uint4 (&raw)[D / 32], uint4 (&kb)[D / 32]) {
    constexpr int CQ8 = D / 64;
#pragma unroll
    for (int i = 0; i < CQ8; i++) {
        fp8x4_to_bf16x2(raw[i].x, kb[2 * i].x, kb[2 * i].y);
        fp8x4_to_bf16x2(raw[i].y, kb[2 * i].z, kb[2 * i].w);
        fp8x4_to_bf16x2(raw[i].z, kb[2 * i + 1].x, kb[2 * i + 1].y);
        fp8x4_to_bf16x2(raw[i].w, kb[2 * i + 1].z, kb[2 * i + 1].w);
    }
}

// V from the standard layout, transposed through the wave's LDS region into
// the shuffled V registers: raw[i] (token col's dims 8 (row CQ + i) ..
// + 7) is scattered as 2-byte values to slot (token group col / 8, dim),
// 16 bytes of 8 tokens each; lane l then reads slot (tg, l + 64 jj) into
// vv[tg][jj], exactly what load_v_sub returns from the shuffled cache.
// Slots are padded every 32 dims and per token group so that a row's 16
// lanes and the 4 rows fall into different LDS banks.
template <int D>
struct StdVLayout {
    static constexpr int kGroupBytes = D * 16 + (D / 32) * 16 + 64;  // one 8-token group
    static constexpr int kWaveBytes = 2 * kGroupBytes;
    static __device__ __forceinline__ uint32_t slot(int tg, int dim) {
        return (uint32_t)(tg * kGroupBytes + dim * 16 + (dim / 32) * 16);
    }
};
template <int D>
__device__ __forceinline__ void transpose_v_std(char *region, const uint4 (&raw)[D / 32],
                                                uint4 (&vv)[2][D / 64]) {
    constexpr int CQ = D / 32, DV = D / 64;
    using L = StdVLayout<D>;
    const int lane = threadIdx.x & 63, row = lane >> 4, col = lane & 15;
    const uint32_t tok = (uint32_t)(col % 8) * 2;
#pragma unroll
    for (int i = 0; i < CQ; i++) {
        const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int dim = (row * CQ + i) * 8 + e;
            *reinterpret_cast<uint16_t *>(region + L::slot(col / 8, dim) + tok) =
                (uint16_t)(w[e / 2] >> ((e & 1) * 16));
        }
    }
    // the wave's own lanes wrote the slots: LDS operations of a wave are
    // performed in order, so only the compiler must not move reads up
    asm volatile("" ::: "memory");
#pragma unroll
    for (int tg = 0; tg < 2; tg++)
#pragma unroll
        for (int jj = 0; jj < DV; jj++)
            vv[tg][jj] = *reinterpret_cast<const uint4 *>(region + L::slot(tg, lane + 64 * jj));
    asm volatile("" ::: "memory");
}

// Token offset, from `start`, of a wave's sub-block k.  SHARED: the 4 waves
// of the workgroup take SUBS-sub-block chunks of the range round-robin
// (sub-block k of a wave is sub-block k % SUBS of its chunk k / SUBS);
// otherwise the wave owns the range and its sub-blocks are consecutive.
template <int SUBS, bool SHARED, int NWV = kWaves>
__device__ __forceinline__ int sub_t0(int k, int wave) {
    if constexpr (SHARED)
        return (NWV * (k / SUBS) + wave) * (kSub * SUBS) + kSub * (k % SUBS);
    else
        return kSub * k;
}

// Raw block-table entry of the wave's sub-block `lane` in the window that
// starts at token `start` (index clamped into the table; the caller decides
// validity).
template <int B, int SUBS, bool SHARED, int NWV = kWaves>
__device__ __forceinline__ int bt_entry(const DecodeParams &p, int s, int start) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int t0 = start + sub_t0<SUBS, SHARED, NWV>(lane, wave);
    return p.block_table[(size_t)s * p.max_blocks + min(t0 / B, p.max_blocks - 1)];
}

// The work of one wave on tokens [start, end) of sequence s, kv head g (start
// a multiple of 16), in chunks of SUBS sub-blocks; the online-softmax state
// (m, lsum, acc) accumulates across calls.  Per chunk a wave loads its
// sub-blocks' K (one 16-byte vector per lane per load) and V, computes all
// SUBS x G scores, takes their exact max and accumulates P.V.  A wave
// tracks the block ids of 64 sub-blocks at a time, so longer ranges are
// taken in windows; bt_first is bt_entry() of the first window, loaded
// early by the caller.
template <int D, int B, int G, int SUBS, bool SHARED, int LAY, int NBUF = 2, int NWV = kWaves>
__device__ __forceinline__ void attend_range(const DecodeParams &p, int s, int g, int range_start,
                                             int range_end, int bt_first, const uint32_t (&qreg)[G],
                                             float (&m)[G], float (&lsum)[G],
                                             float (&acc)[G][D / 64]) {
    constexpr int CQ = D / 32;        // K vectors per lane per sub-block
    constexpr int DV = D / 64;        // output dims per lane
    constexpr bool kPairs = G >= 2;
    constexpr int HS = kPairs ? 2 : 1;
    constexpr int kWindow = (SHARED ? NWV : 1) * 64 * kSub;  // tokens per window
    constexpr bool STD = LAY == kLayStd, FP8 = LAY == kLayFp8;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int row = lane >> 4, col = lane & 15;
    const float sl2 = p.scale * kLog2e * (FP8 ? p.k_scale : 1.f);
    const char *kc = reinterpret_cast<const char *>(p.k_cache);
    const char *vc = reinterpret_cast<const char *>(p.v_cache);
    const uint32_t k_off = STD ? std_lane_off<D>(row, col, p.Hkv)
                               : FP8 ? (uint32_t)((row * (D / 64) * B + col) * 16)
                                     : k_lane_off<D, B>(row, col);
    const uint32_t v_off = STD ? k_off : (uint32_t)lane * 16;
    char *vt_region = nullptr;
    if constexpr (STD) {
        __shared__ __align__(16) char vt_lds[NWV][StdVLayout<D>::kWaveBytes];
        vt_region = vt_lds[wave];
    }

    int bt_raw = bt_first;
    for (int start = range_start; start < range_end; start += kWindow) {
        const int end = min(start + kWindow, range_end);
        if (start != range_start) bt_raw = bt_entry<B, SUBS, SHARED, NWV>(p, s, start);
        // lane k: physical block of this wave's sub-block k, -1 past the end or
        // out of range.  Validity is monotone in k, so the sub-blocks in range
        // are 0 .. nmine - 1.
        const int t0_lane = start + sub_t0<SUBS, SHARED, NWV>(lane, wave);
        const bool lane_ok = t0_lane < end;
        const int bid = lane_ok && bt_raw >= 0 && (int64_t)bt_raw < p.num_blocks ? bt_raw : -1;
        const int nmine = __popcll(__ballot(lane_ok));

        // Sub-block k's block and token offset (k clamped into the window);
        // an invalid block id reads block 0 and is masked.
        auto locate = [&](int k, size_t &tile, int &half) {
            k = min(k, 63);
            const int b = readlane_i32(bid, k);
            const int t0 = start + sub_t0<SUBS, SHARED, NWV>(k, wave);
            tile = (size_t)(b < 0 ? 0 : b) * p.Hkv + g;
            half = (t0 % B) / kSub;
        };
        // standard layout: the sub-block's first row (block, 16-token half, head g)
        auto std_first = [&](int k) -> size_t {
            k = min(k, 63);
            const int b = readlane_i32(bid, k);
            const int t0 = start + sub_t0<SUBS, SHARED, NWV>(k, wave);
            return ((size_t)(b < 0 ? 0 : b) * B + (t0 % B) / kSub * kSub) * p.Hkv + g;
        };
        auto load_k = [&](int k, uint4 (&kq)[CQ]) {
            size_t tile;
            int half;
            locate(k, tile, half);
            if constexpr (STD)
                load_rows_std<D>(kc, std_first(k), p.Hkv, k < nmine, k_off, kq);
            else if constexpr (FP8)
                load_k_sub8<D, B>(kc, tile, half, k < nmine, k_off, kq);
            else
                load_k_sub<D, B>(kc, tile, half, k < nmine, k_off, kq);
        };
        auto load_v = [&](int k, uint4 (&vv)[2][DV]) {
            size_t tile;
            int half;
            locate(k, tile, half);
            if constexpr (STD)
                load_rows_std<D>(vc, std_first(k), p.Hkv, k < nmine,
                                 v_off, reinterpret_cast<uint4(&)[CQ]>(vv));
            else if constexpr (FP8)
                load_v_sub8<D, B>(vc, tile, half, k < nmine, v_off, vv);
            else
                load_v_sub<D, B>(vc, tile, half, k < nmine, v_off, vv);
        };

        // One sub-block: QK, a lazy softmax update, PV (skipped, by uniform
        // branches, for sub-blocks past the end or with an invalid block).
        // When it starts, the loads in flight are, oldest first: this
        // sub-block's K and V, then the other buffer's K and V; the explicit
        // waits say exactly that to the compiler.
        // load instructions per sub-block
        constexpr int LK = FP8 ? D / 64 : CQ, LV = FP8 ? DV : 2 * DV;
        // loads issued after sub-block k's, still in flight when k starts
        constexpr int kAhead = (NBUF - 1) * (LK + LV);
        static_assert(NBUF == 2 || NBUF == 4, "ring of 2 or 4 sub-blocks");
        static_assert(LV + kAhead < 64, "vmcnt range");
        auto compute_sub = [&](int k, const uint4 (&kin)[CQ], const uint4 (&vv)[2][DV]) {
            const int t0 = start + sub_t0<SUBS, SHARED, NWV>(k, wave);
            const int nvalid =
                k < nmine && readlane_i32(bid, min(k, 63)) >= 0 ? min(kSub, end - t0) : 0;
            float z[G];
            if (nvalid > 0) {
                wait_vm_loads<LV + kAhead>();
                uint4 kconv[CQ];
                if constexpr (FP8) k_fp8_to_bf16<D>(kin, kconv);
                const uint4 (&kq)[CQ] = FP8 ? kconv : kin;
                // QK: each lane sums a quarter of the dims; the rows are then
                // summed, leaving every row with the 16 scores of the sub-block
                float a[G][2];
#pragma unroll
                for (int h = 0; h < G; h++) a[h][0] = a[h][1] = 0.f;
#pragma unroll
                for (int h = 0; h < G; h += HS) {
                    if constexpr (kPairs) {
                        if constexpr (CQ == 4) {
                            if (h + 2 >= G)
                                qk_2h<true>(a[h][0], a[h][1], a[h + 1][0], a[h + 1][1], qreg[h],
                                            qreg[h + 1], kq[0], kq[1], kq[2], kq[3]);
                            else
                                qk_2h<false>(a[h][0], a[h][1], a[h + 1][0], a[h + 1][1], qreg[h],
                                             qreg[h + 1], kq[0], kq[1], kq[2], kq[3]);
                        } else {
                            qk8_2h(a[h][0], a[h][1], a[h + 1][0], a[h + 1][1], qreg[h],
                                   qreg[h + 1], kq[0], kq[1]);
                        }
                    } else {
                        if constexpr (CQ == 4)
                            qk_1h<true>(a[h][0], a[h][1], qreg[h], kq[0], kq[1], kq[2], kq[3]);
                        else
                            qk8_1h(a[h][0], a[h][1], qreg[h], kq[0], kq[1]);
                    }
                }
                dpp_result_fence<2 * G>(&a[0][0]);
                const bool ok = col < nvalid;
#pragma unroll
                for (int h = 0; h < G; h++) {
                    const float t = row_sum4(a[h][0] + a[h][1]);
                    z[h] = ok ? t * sl2 : kNegInf;
                }
            }
            if (nvalid > 0) {
                // Lazy softmax: the reference m[h] (log2 units) moves only when
                // a score exceeds it by more than kLazyLog2, so weights stay
                // <= 2^kLazyLog2 and most sub-blocks need no rescale.
                uint64_t over = 0;
#pragma unroll
                for (int h = 0; h < G; h++) over |= __ballot(z[h] > m[h] + kLazyLog2);
                if (over) {
                    dpp_result_fence<G * DV>(&acc[0][0]);
#pragma unroll
                    for (int h = 0; h < G; h++) {
                        const float mx = uniform_f(row_max16(z[h]));
                        if (mx > m[h] + kLazyLog2) {
                            const float alpha = fast_exp2(m[h] - mx);  // 0 from -inf
                            lsum[h] *= alpha;
#pragma unroll
                            for (int jj = 0; jj < DV; jj++) acc[h][jj] *= alpha;
                            m[h] = mx;
                        }
                    }
                }
                uint32_t pw[G];
#pragma unroll
                for (int h = 0; h < G; h++) {
                    const float mref = m[h] == kNegInf ? 0.f : m[h];
                    const float pr = fast_exp2(z[h] - mref);
                    lsum[h] += pr;
                    pw[h] = __float_as_uint(pr);
                }
                // PV: the V of tokens past the end is zeroed (weight 0, data may
                // be anything); the buffers themselves are only read
                wait_vm_loads<kAhead>();
                uint4 vt[2][DV];
                if constexpr (STD)
                    transpose_v_std<D>(vt_region, reinterpret_cast<const uint4(&)[CQ]>(vv), vt);
                const uint4 (&vsrc)[2][DV] = STD ? vt : vv;
#pragma unroll
                for (int tg = 0; tg < 2; tg++) {
                    const int nv = nvalid - 8 * tg;
                    float vf[DV][8];
#pragma unroll
                    for (int jj = 0; jj < DV; jj++) {
                        if constexpr (FP8) {  // tokens 8 tg .. 8 tg + 7 of the 16-code vector
                            const uint4 raw = vv[0][jj];
                            fp8x4_to_f32(tg ? raw.z : raw.x, vf[jj]);
                            fp8x4_to_f32(tg ? raw.w : raw.y, vf[jj] + 4);
                            if (nvalid < kSub) {
#pragma unroll
                                for (int e = 0; e < 8; e++)
                                    if (e >= nv) vf[jj][e] = 0.f;
                            }
                        } else {
                            uint4 v = vsrc[tg][jj];
                            if (nvalid < kSub) {
                                v.x = mask_pair(v.x, 0, nv);
                                v.y = mask_pair(v.y, 2, nv);
                                v.z = mask_pair(v.z, 4, nv);
                                v.w = mask_pair(v.w, 6, nv);
                            }
                            widen8(v, vf[jj]);
                        }
                    }
#pragma unroll
                    for (int h = 0; h < G; h += HS) {
                        const bool last = tg == 1 && h + HS >= G;
                        pv_step<DV, kPairs>(tg, last, acc[h], acc[h + HS - 1], pw[h],
                                            pw[h + HS - 1], vf);
                    }
                }
                dpp_result_fence<G * DV>(&acc[0][0]);
            }
        };

        // Two buffers: sub-block k + 1 is requested before k is computed, so
        // requests reach memory spread over the wave's work and computation
        // overlaps the stream (loads complete in issue order).  Every load is
        // issued on every path (a load past the end touches no memory), so
        // the buffers are plain loop-carried registers.
        if constexpr (NBUF == 2) {
            uint4 kA[CQ], vA[2][DV], kB[CQ], vB[2][DV];
            load_k(0, kA);
            load_v(0, vA);
            for (int k = 0; k < nmine; k += 2) {
                load_k(k + 1, kB);
                load_v(k + 1, vB);
                compute_sub(k, kA, vA);
                load_k(k + 2, kA);
                load_v(k + 2, vA);
                compute_sub(k + 1, kB, vB);
            }
        } else {
            // four sub-blocks in flight: a wave's whole share of a short
            // piece is requested before its first sub-block is computed
            uint4 kA[CQ], vA[2][DV], kB[CQ], vB[2][DV], kC[CQ], vC[2][DV], kD[CQ], vD[2][DV];
            load_k(0, kA);
            load_v(0, vA);
            load_k(1, kB);
            load_v(1, vB);
            load_k(2, kC);
            load_v(2, vC);
            for (int k = 0; k < nmine; k += 4) {
                load_k(k + 3, kD);
                load_v(k + 3, vD);
                compute_sub(k, kA, vA);
                load_k(k + 4, kA);
                load_v(k + 4, vA);
                compute_sub(k + 1, kB, vB);
                load_k(k + 5, kB);
                load_v(k + 5, vB);
                compute_sub(k + 2, kC, vC);
                load_k(k + 6, kC);
                load_v(k + 6, vC);
                compute_sub(k + 3, kD, vD);
            }
        }
    }
    if constexpr (FP8) {  // V codes were summed unscaled
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int jj = 0; jj < DV; jj++) acc[h][jj] *= p.v_scale;
    }
}

// Query registers of kv head g's query heads: lane (row r, column n) holds
// dword r * QW + n of each head's query; padded heads (h >= Ga) repeat real ones.
template <int D, int G>
__device__ __forceinline__ void load_queries(const DecodeParams &p, int s, int g, int Ga,
                                             uint32_t (&qreg)[G]) {
    constexpr int QW = D / 8;
    const int lane = threadIdx.x & 63, row = lane >> 4, col = lane & 15;
    const uint32_t *qg = reinterpret_cast<const uint32_t *>(p.query) +
                         ((size_t)s * p.Hq + (size_t)g * Ga) * (D / 2) + row * QW + (col % QW);
#pragma unroll
    for (int h = 0; h < G; h++) qreg[h] = qg[(h < Ga ? h : h - Ga) * (D / 2)];
}

template <int G, int DV>
__device__ __forceinline__ void reset_state(float (&m)[G], float (&lsum)[G], float (&acc)[G][DV]) {
#pragma unroll
    for (int h = 0; h < G; h++) {
        m[h] = kNegInf;
        lsum[h] = 0.f;
#pragma unroll
        for (int jj = 0; jj < DV; jj++) acc[h][jj] = 0.f;
    }
}

template <int D, int G, int NWV = kWaves>
struct WaveMergeLDS {
    float m[NWV][G], l[NWV][G];
    __align__(16) float acc[NWV][G][D];
};

// Merge the 4 waves' states in LDS; thread (head h, dims d .. d + 3) then
// calls emit(h, d, o, L) with the normalised output o[0..3] and the LSE
// (natural log).  Every row holds the same token weights, so a wave's sum
// of weights is 4 x the row sum.  Ends with the workgroup synchronised only
// before the emits: callers that reuse the LDS must synchronise again.
template <int D, int G, int NWV, typename Emit>
__device__ __forceinline__ void merge_waves(WaveMergeLDS<D, G, NWV> &sm, int Ga, const float (&m)[G],
                                            const float (&lsum)[G], const float (&acc)[G][D / 64],
                                            Emit emit) {
    constexpr int DV = D / 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float l = wave_sum(lsum[h]) * 0.25f;
        if (lane == 0) {
            sm.m[wave][h] = m[h];
            sm.l[wave][h] = l;
        }
#pragma unroll
        for (int jj = 0; jj < DV; jj++) sm.acc[wave][h][lane + 64 * jj] = acc[h][jj];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < Ga * (D / 4); idx += NWV * 64) {
        const int h = idx / (D / 4), d = 4 * (idx % (D / 4));
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < NWV; w++) M = fmax_nc(M, sm.m[w][h]);
        const float Mr = M == kNegInf ? 0.f : M;
        float o[4] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; w++) {
            const float wt = fast_exp2(sm.m[w][h] - Mr);
            const float4 a = *reinterpret_cast<const float4 *>(&sm.acc[w][h][d]);
            o[0] += wt * a.x;
            o[1] += wt * a.y;
            o[2] += wt * a.z;
            o[3] += wt * a.w;
            den += wt * sm.l[w][h];
        }
        const float inv = den > 0.f ? 1.f / den : 0.f;
        const float L = den > 0.f ? (M + fast_log2(den)) * kLn2 : kNegInf;
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] *= inv;
        emit(h, d, o, L);
    }
}

// ---------------------------------------------------------------------------
// Row-per-head softmax with gathered weights (bf16 caches, 4, 8 or 16 query
// heads per kv head).  QK is computed as above (lane (row r, column n): token
// n, the r-th quarter of head_dim), but the four rows' partial dot products
// of four heads are summed with two-register permlane swaps, after which row
// r holds head r's 16 scores: 3 swaps and 3 adds per 4 heads instead of 8 and
// 8, and each softmax weight is computed once, not once per row.  The
// weights of token pairs are split into bf16 hi + lo parts and gathered so
// that every row holds every head's (3 permlane swaps per register); P.V then
// runs in the V cache's own layout (lane l: dims l and l + 64) as v_dot2c over
// the bf16 pairs of a V vector, so V is neither widened nor loaded twice.
//
// Wait states the compiler cannot see inside the asm blocks (gfx950):
//  - a VALU write of a VGPR followed by a DPP read of it needs 2 wait
//    states: every block that reads an operand through DPP starts with
//    s_nop 1 (the compiler may place the producer right before it);
//  - a v_dot2c result read by any other VALU instruction, or by a dot as its
//    A or B operand, needs 3 wait states; read by the same dot opcode as its
//    accumulator it needs none.  Blocks whose results plain code reads next
//    end with s_nop 4 (5 wait states), or the caller fences them
//    (dpp_result_fence).
// ---------------------------------------------------------------------------

// 4 heads, one accumulator each, over the lane's 16 (D = 128) or 8 (D = 64)
// K dwords; dword n of the row slice comes from lane n of each head's query
// register.
#define PA_QK4_N(kd, n) \
    PA_DOT2_BC("%0", "%4", kd, n) PA_DOT2_BC("%1", "%5", kd, n) \
    PA_DOT2_BC("%2", "%6", kd, n) PA_DOT2_BC("%3", "%7", kd, n)
#define PA_QK4_D128                                                                         \
    "s_nop 1\n\t"                                                                           \
    PA_QK4_N("%8", "0") PA_QK4_N("%9", "1") PA_QK4_N("%10", "2") PA_QK4_N("%11", "3")       \
    PA_QK4_N("%12", "4") PA_QK4_N("%13", "5") PA_QK4_N("%14", "6") PA_QK4_N("%15", "7")     \
    PA_QK4_N("%16", "8") PA_QK4_N("%17", "9") PA_QK4_N("%18", "10") PA_QK4_N("%19", "11")   \
    PA_QK4_N("%20", "12") PA_QK4_N("%21", "13") PA_QK4_N("%22", "14") PA_QK4_N("%23", "15") \
    "s_nop 4\n\t"
#define PA_QK4_D64                                                                          \
    "s_nop 1\n\t"                                                                           \
    PA_QK4_N("%8", "0") PA_QK4_N("%9", "1") PA_QK4_N("%10", "2") PA_QK4_N("%11", "3")       \
    PA_QK4_N("%12", "4") PA_QK4_N("%13", "5") PA_QK4_N("%14", "6") PA_QK4_N("%15", "7")     \
    "s_nop 4\n\t"

template <int D>
__device__ __forceinline__ void qk_4h(float (&a)[4], const uint32_t *q, const uint4 (&k)[D / 32]) {
    if constexpr (D == 128)
        asm volatile(PA_QK4_D128
                     : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
                     : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(k[0].x), "v"(k[0].y),
                       "v"(k[0].z), "v"(k[0].w), "v"(k[1].x), "v"(k[1].y), "v"(k[1].z),
                       "v"(k[1].w), "v"(k[2].x), "v"(k[2].y), "v"(k[2].z), "v"(k[2].w),
                       "v"(k[3].x), "v"(k[3].y), "v"(k[3].z), "v"(k[3].w));
    else
        asm volatile(PA_QK4_D64
                     : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
                     : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(k[0].x), "v"(k[0].y),
                       "v"(k[0].z), "v"(k[0].w), "v"(k[1].x), "v"(k[1].y), "v"(k[1].z),
                       "v"(k[1].w));
}

// Sum over the 4 rows of 4 heads' partial dots: row r of the result holds
// head r's totals (column n: token n).  A permlane16 swap of two registers
// exchanges the odd rows of the first with the even rows of the second, a
// permlane32 swap the upper half of the first with the lower half of the
// second.
__device__ __forceinline__ float rows_to_heads(float a0, float a1, float a2, float a3) {
    auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
    const float s01 = __uint_as_float(x[0]) + __uint_as_float(x[1]);  // h0 r01, h1 r01, h0 r23, h1 r23
    auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(a2), __float_as_uint(a3), false, false);
    const float s23 = __uint_as_float(y[0]) + __uint_as_float(y[1]);  // h2 r01, h3 r01, h2 r23, h3 r23
    auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(s01), __float_as_uint(s23), false, false);
    return __uint_as_float(z[0]) + __uint_as_float(z[1]);             // h0, h1, h2, h3
}

// P.V in the V cache's own layout once every row holds every head's weights
// (gather_rows below): lane l owns dims l and l + 64 of all heads, a V
// vector is 8 tokens of one dim as 4 bf16 pairs, and the weights of token
// pair w of token group tg come from lane 8 tg + 2 w of the row, in bf16 hi
// and lo parts.  One block: two heads (a, b), both token groups.
//   D = 128: %0 %1 a (dims l, l + 64), %2 %3 b; %4 %5 a hi / lo, %6 %7 b hi /
//   lo; %8..%11 V of (tg 0, dim l), %12..%15 (tg 0, l + 64), %16..%19
//   (tg 1, l), %20..%23 (tg 1, l + 64).
#define PA_PVG2_W128(L, va0, va1)                                                           \
    PA_DOT2_BC("%0", "%4", va0, L) PA_DOT2_BC("%1", "%4", va1, L)                           \
    PA_DOT2_BC("%2", "%6", va0, L) PA_DOT2_BC("%3", "%6", va1, L)                           \
    PA_DOT2_BC("%0", "%5", va0, L) PA_DOT2_BC("%1", "%5", va1, L)                           \
    PA_DOT2_BC("%2", "%7", va0, L) PA_DOT2_BC("%3", "%7", va1, L)
#define PA_PVG2_D128                                                                        \
    "s_nop 1\n\t"                                                                           \
    PA_PVG2_W128("0", "%8", "%12") PA_PVG2_W128("2", "%9", "%13")                           \
    PA_PVG2_W128("4", "%10", "%14") PA_PVG2_W128("6", "%11", "%15")                         \
    PA_PVG2_W128("8", "%16", "%20") PA_PVG2_W128("10", "%17", "%21")                        \
    PA_PVG2_W128("12", "%18", "%22") PA_PVG2_W128("14", "%19", "%23")
//   D = 64: %0 a, %1 b (dim l); %2 %3 a hi / lo, %4 %5 b hi / lo; %6..%9 V of
//   (tg 0, dim l), %10..%13 (tg 1, dim l).
#define PA_PVG2_W64(L, va)                                                                  \
    PA_DOT2_BC("%0", "%2", va, L) PA_DOT2_BC("%1", "%4", va, L)                             \
    PA_DOT2_BC("%0", "%3", va, L) PA_DOT2_BC("%1", "%5", va, L)
#define PA_PVG2_D64                                                                         \
    "s_nop 1\n\t"                                                                           \
    PA_PVG2_W64("0", "%6") PA_PVG2_W64("2", "%7") PA_PVG2_W64("4", "%8") PA_PVG2_W64("6", "%9") \
    PA_PVG2_W64("8", "%10") PA_PVG2_W64("10", "%11") PA_PVG2_W64("12", "%12")              \
    PA_PVG2_W64("14", "%13")

template <int D>
__device__ __forceinline__ void pv_2h(float (&a)[D / 64], float (&b)[D / 64], uint32_t ah,
                                      uint32_t al, uint32_t bh, uint32_t bl,
                                      const uint4 (&v)[2][D / 64]) {
    if constexpr (D == 128)
        asm volatile(PA_PVG2_D128
                     : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1])
                     : "v"(ah), "v"(al), "v"(bh), "v"(bl), "v"(v[0][0].x), "v"(v[0][0].y),
                       "v"(v[0][0].z), "v"(v[0][0].w), "v"(v[0][1].x), "v"(v[0][1].y),
                       "v"(v[0][1].z), "v"(v[0][1].w), "v"(v[1][0].x), "v"(v[1][0].y),
                       "v"(v[1][0].z), "v"(v[1][0].w), "v"(v[1][1].x), "v"(v[1][1].y),
                       "v"(v[1][1].z), "v"(v[1][1].w));
    else
        asm volatile(PA_PVG2_D64
                     : "+v"(a[0]), "+v"(b[0])
                     : "v"(ah), "v"(al), "v"(bh), "v"(bl), "v"(v[0][0].x), "v"(v[0][0].y),
                       "v"(v[0][0].z), "v"(v[0][0].w), "v"(v[1][0].x), "v"(v[1][0].y),
                       "v"(v[1][0].z), "v"(v[1][0].w));
}

// bf16 hi and lo parts of the weights of token pairs: lane 2w of a row gets
// (p[2w], p[2w + 1]) (its own weight and its right neighbour's), so that
// p = hi + lo to 16 significant bits.
__device__ __forceinline__ void split_pairs(float p, uint32_t &ph, uint32_t &pl) {
    const float pn = dpp_f<kQuadXor1>(p);
    ph = pack_bf16x2(p, pn);
    pl = pack_bf16x2(p - bf16_lo(ph), pn - bf16_hi(ph));
}

// Every row gets every row's values: out[r] holds row r of v in all four
// rows (one permlane32 swap and two permlane16 swaps).
__device__ __forceinline__ void gather_rows(uint32_t v, uint32_t (&out)[4]) {
    auto x = __builtin_amdgcn_permlane32_swap(v, v, false, false);        // r0 r1 r0 r1 | r2 r3 r2 r3
    auto y = __builtin_amdgcn_permlane16_swap(x[0], x[0], false, false);  // r0 x4 | r1 x4
    auto z = __builtin_amdgcn_permlane16_swap(x[1], x[1], false, false);  // r2 x4 | r3 x4
    out[0] = y[0];
    out[1] = y[1];
    out[2] = z[0];
    out[3] = z[1];
}

// Sum over the 16 lanes of each row (every lane gets its row's sum).
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp_f<kQuadXor1>(v);
    v += dpp_f<kQuadXor2>(v);
    v += dpp_f<kRowRor4>(v);
    v += dpp_f<kRowRor8>(v);
    return v;
}

// The gathered-weight counterpart of attend_range (bf16 caches, G a multiple
// of 4).  State per lane: for the NR = G / 4 heads 4 i + r of its row r, the
// reference maximum m[i] (log2 units, the same in every lane of the row) and
// the lane's share of the weight sum lsum[i] (summed over the row at the
// end); acc[h][jj] for every head h and dims l + 64 jj, as in attend_range.
template <int D, int B, int G, int SUBS, bool SHARED, int LAY, int NWV = kWaves>
__device__ __forceinline__ void attend_range_rh(const DecodeParams &p, int s, int g,
                                                int range_start, int range_end, int bt_first,
                                                const uint32_t (&qreg)[G], float (&m)[G / 4],
                                                float (&lsum)[G / 4], float (&acc)[G][D / 64]) {
    constexpr int CQ = D / 32;        // K vectors per lane per sub-block
    constexpr int DV = D / 64;        // output dims per lane
    constexpr int NR = G / 4;         // heads per row
    constexpr int kWindow = (SHARED ? NWV : 1) * 64 * kSub;  // tokens per window
    constexpr bool STD = LAY == kLayStd, FP8 = LAY == kLayFp8;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int row = lane >> 4, col = lane & 15;
    // FP8: the codes are widened to bf16 exactly; K's scale goes into the
    // score scale and V's multiplies the output at the end
    const float sl2 = p.scale * kLog2e * (FP8 ? p.k_scale : 1.f);
    const char *kc = reinterpret_cast<const char *>(p.k_cache);
    const char *vc = reinterpret_cast<const char *>(p.v_cache);
    const uint32_t k_off = STD   ? std_lane_off<D>(row, col, p.Hkv)
                           : FP8 ? (uint32_t)((row * (D / 64) * B + col) * 16)
                                 : k_lane_off<D, B>(row, col);
    const uint32_t v_off = STD ? k_off : (uint32_t)lane * 16;
    char *vt_region = nullptr;
    if constexpr (STD) {
        __shared__ __align__(16) char vt_lds[NWV][StdVLayout<D>::kWaveBytes];
        vt_region = vt_lds[wave];
    }

    int bt_raw = bt_first;
    for (int start = range_start; start < range_end; start += kWindow) {
        const int end = min(start + kWindow, range_end);
        if (start != range_start) bt_raw = bt_entry<B, SUBS, SHARED, NWV>(p, s, start);
        const int t0_lane = start + sub_t0<SUBS, SHARED, NWV>(lane, wave);
        const bool lane_ok = t0_lane < end;
        const int bid = lane_ok && bt_raw >= 0 && (int64_t)bt_raw < p.num_blocks ? bt_raw : -1;
        const int nmine = __popcll(__ballot(lane_ok));

        auto locate = [&](int k, size_t &tile, int &half) {
            k = min(k, 63);
            const int b = readlane_i32(bid, k);
            const int t0 = start + sub_t0<SUBS, SHARED, NWV>(k, wave);
            tile = (size_t)(b < 0 ? 0 : b) * p.Hkv + g;
            half = (t0 % B) / kSub;
        };
        // standard layout: the sub-block's first row (block, 16-token half, head g)
        auto std_first = [&](int k) -> size_t {
            k = min(k, 63);
            const int b = readlane_i32(bid, k);
            const int t0 = start + sub_t0<SUBS, SHARED, NWV>(k, wave);
            return ((size_t)(b < 0 ? 0 : b) * B + (t0 % B) / kSub * kSub) * p.Hkv + g;
        };
        auto load_kv = [&](int k, uint4 (&kq)[CQ], uint4 (&vv)[2][DV]) {
            if constexpr (STD) {
                const size_t first = std_first(k);
                load_rows_std<D>(kc, first, p.Hkv, k < nmine, k_off, kq);
                load_rows_std<D>(vc, first, p.Hkv, k < nmine, v_off,
                                 reinterpret_cast<uint4(&)[CQ]>(vv));
            } else {
                size_t tile;
                int half;
                locate(k, tile, half);
                if constexpr (FP8) {
                    load_k_sub8<D, B>(kc, tile, half, k < nmine, k_off, kq);
                    load_v_sub8<D, B>(vc, tile, half, k < nmine, v_off, vv);
                } else {
                    load_k_sub<D, B>(kc, tile, half, k < nmine, k_off, kq);
                    load_v_sub<D, B>(vc, tile, half, k < nmine, v_off, vv);
                }
            }
        };
        // loads per sub-block (FP8: CQ / 2 K vectors of 16 codes, one V vector
        // of the sub-block's 16 tokens per dim)
        constexpr int LK = FP8 ? CQ / 2 : CQ, LV = FP8 ? DV : 2 * DV;

        auto compute_sub = [&](int k, const uint4 (&kq)[CQ], const uint4 (&vin)[2][DV]) {
            const int t0 = start + sub_t0<SUBS, SHARED, NWV>(k, wave);
            const int nvalid =
                k < nmine && readlane_i32(bid, min(k, 63)) >= 0 ? min(kSub, end - t0) : 0;
            if (nvalid <= 0) return;
            // in flight: this sub-block's K and V, then the next one's
            wait_vm_loads<LV + LK + LV>();
            uint4 kconv[CQ];
            if constexpr (FP8) k_fp8_to_bf16<D>(kq, kconv);
            const uint4 (&kb)[CQ] = FP8 ? kconv : kq;
            float z[NR];
#pragma unroll
            for (int i = 0; i < NR; i++) {
                float a[4] = {0.f, 0.f, 0.f, 0.f};
                qk_4h<D>(a, &qreg[4 * i], kb);
                z[i] = rows_to_heads(a[0], a[1], a[2], a[3]) * sl2;
            }
            if (nvalid < kSub) {
#pragma unroll
                for (int i = 0; i < NR; i++) z[i] = col < nvalid ? z[i] : kNegInf;
            }
            // lazy softmax: a row's reference moves only when one of its
            // scores passes it by more than kLazyLog2
            uint64_t over = 0;
#pragma unroll
            for (int i = 0; i < NR; i++) over |= __ballot(z[i] > m[i] + kLazyLog2);
            if (over) {
                dpp_result_fence<G * DV>(&acc[0][0]);
#pragma unroll
                for (int i = 0; i < NR; i++) {
                    const float mx = row_max16(z[i]);
                    float alpha = 1.f;
                    if (mx > m[i] + kLazyLog2) {
                        alpha = fast_exp2(m[i] - mx);  // 0 from -inf
                        m[i] = mx;
                    }
                    lsum[i] *= alpha;
                    uint32_t al[4];
                    gather_rows(__float_as_uint(alpha), al);
#pragma unroll
                    for (int r = 0; r < 4; r++)
#pragma unroll
                        for (int jj = 0; jj < DV; jj++) acc[4 * i + r][jj] *= __uint_as_float(al[r]);
                }
            }
            uint32_t ph[G], pl[G];
#pragma unroll
            for (int i = 0; i < NR; i++) {
                const float pr = fast_exp2(z[i] - m[i]);  // m[i] is finite here
                lsum[i] += pr;
                uint32_t h, l;
                split_pairs(pr, h, l);
                gather_rows(h, reinterpret_cast<uint32_t(&)[4]>(ph[4 * i]));
                gather_rows(l, reinterpret_cast<uint32_t(&)[4]>(pl[4 * i]));
            }
            // in flight: this sub-block's V, then the next sub-block's K and V
            wait_vm_loads<LK + LV>();
            uint4 vv[2][DV];
            if constexpr (STD) {
                transpose_v_std<D>(vt_region, reinterpret_cast<const uint4(&)[CQ]>(vin), vv);
            } else if constexpr (FP8) {
                // the 16-token vector of dim l + 64 jj -> the two 8-token
                // groups' bf16 pairs (token 2 w in the low half of word w)
#pragma unroll
                for (int jj = 0; jj < DV; jj++) {
                    const uint4 raw = vin[0][jj];
                    fp8x4_to_bf16x2(raw.x, vv[0][jj].x, vv[0][jj].y);
                    fp8x4_to_bf16x2(raw.y, vv[0][jj].z, vv[0][jj].w);
                    fp8x4_to_bf16x2(raw.z, vv[1][jj].x, vv[1][jj].y);
                    fp8x4_to_bf16x2(raw.w, vv[1][jj].z, vv[1][jj].w);
                }
            } else {
#pragma unroll
                for (int tg = 0; tg < 2; tg++)
#pragma unroll
                    for (int jj = 0; jj < DV; jj++) vv[tg][jj] = vin[tg][jj];
            }
            if (nvalid < kSub) {
                // tokens past the end carry weight 0 and V may hold anything
                // (NaN included): zero their V
#pragma unroll
                for (int tg = 0; tg < 2; tg++) {
                    const int nv = nvalid - 8 * tg;
#pragma unroll
                    for (int jj = 0; jj < DV; jj++) {
                        vv[tg][jj].x = mask_pair(vv[tg][jj].x, 0, nv);
                        vv[tg][jj].y = mask_pair(vv[tg][jj].y, 2, nv);
                        vv[tg][jj].z = mask_pair(vv[tg][jj].z, 4, nv);
                        vv[tg][jj].w = mask_pair(vv[tg][jj].w, 6, nv);
                    }
                }
            }
#pragma unroll
            for (int h = 0; h < G; h += 2)
                pv_2h<D>(acc[h], acc[h + 1], ph[h], pl[h], ph[h + 1], pl[h + 1], vv);
            dpp_result_fence<G * DV>(&acc[0][0]);
        };

        // two buffers: sub-block k + 1 is requested before k is computed
        uint4 kA[CQ], vA[2][DV], kB[CQ], vB[2][DV];
        load_kv(0, kA, vA);
        for (int k = 0; k < nmine; k += 2) {
            load_kv(k + 1, kB, vB);
            compute_sub(k, kA, vA);
            load_kv(k + 2, kA, vA);
            compute_sub(k + 1, kB, vB);
        }
    }
    if constexpr (FP8) {  // V codes were summed unscaled
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int jj = 0; jj < DV; jj++) acc[h][jj] *= p.v_scale;
    }
}

// Merge of the 4 waves' states (accumulators as in merge_waves, maxima and
// weight sums per row head) in LDS, then emit(h, d, o, L) per (head, 4 dims)
// as merge_waves does.
template <int D, int G, int NWV, typename Emit>
__device__ __forceinline__ void merge_waves_rh(WaveMergeLDS<D, G, NWV> &sm, int Ga,
                                               const float (&m)[G / 4], const float (&lsum)[G / 4],
                                               const float (&acc)[G][D / 64], Emit emit) {
    constexpr int DV = D / 64, NR = G / 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, row = lane >> 4, col = lane & 15;
#pragma unroll
    for (int i = 0; i < NR; i++) {
        const float l = row_sum16(lsum[i]);
        if (col == 0) {
            sm.m[wave][4 * i + row] = m[i];
            sm.l[wave][4 * i + row] = l;
        }
    }
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int jj = 0; jj < DV; jj++) sm.acc[wave][h][lane + 64 * jj] = acc[h][jj];
    __syncthreads();
    for (int idx = threadIdx.x; idx < Ga * (D / 4); idx += NWV * 64) {
        const int h = idx / (D / 4), d = 4 * (idx % (D / 4));
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < NWV; w++) M = fmax_nc(M, sm.m[w][h]);
        const float Mr = M == kNegInf ? 0.f : M;
        float o[4] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; w++) {
            const float wt = fast_exp2(sm.m[w][h] - Mr);
            const float4 a = *reinterpret_cast<const float4 *>(&sm.acc[w][h][d]);
            o[0] += wt * a.x;
            o[1] += wt * a.y;
            o[2] += wt * a.z;
            o[3] += wt * a.w;
            den += wt * sm.l[w][h];
        }
        const float inv = den > 0.f ? 1.f / den : 0.f;
        const float L = den > 0.f ? (M + fast_log2(den)) * kLn2 : kNegInf;
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] *= inv;
        emit(h, d, o, L);
    }
}

// The gathered-weight formulation serves 4, 8 or 16 query heads per kv head
// over every cache (FP8 codes widened to bf16 after the load); smaller
// groups use attend_range.
template <int LAY, int G>
constexpr bool uses_rh() { return G >= 4; }

template <int D, int G, int LAY, int NWV = kWaves>
using MergeLDS = WaveMergeLDS<D, G, NWV>;

// Attention of this workgroup's waves over tokens [tb, te) of unit (s, g),
// then the merge of the waves' states; emit(h, d, o, L) as in merge_waves.
template <int D, int B, int G, int SUBS, int LAY, int NWV, typename Emit>
__device__ __forceinline__ void attend_merge(const DecodeParams &p, int s, int g, int tb, int te,
                                             int bt_first, const uint32_t (&qreg)[G],
                                             MergeLDS<D, G, LAY, NWV> &sm, int Ga, Emit emit) {
    if constexpr (uses_rh<LAY, G>()) {
        constexpr int NR = G / 4, DV = D / 64;
        float m[NR], lsum[NR], acc[G][DV];
#pragma unroll
        for (int i = 0; i < NR; i++) {
            m[i] = kNegInf;
            lsum[i] = 0.f;
        }
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int jj = 0; jj < DV; jj++) acc[h][jj] = 0.f;
        attend_range_rh<D, B, G, SUBS, true, LAY, NWV>(p, s, g, tb, te, bt_first, qreg, m, lsum, acc);
        merge_waves_rh<D, G, NWV>(sm, Ga, m, lsum, acc, emit);
    } else {
        constexpr int DV = D / 64;
        float m[G], lsum[G], acc[G][DV];
        reset_state<G, DV>(m, lsum, acc);
        attend_range<D, B, G, SUBS, true, LAY, 2, NWV>(p, s, g, tb, te, bt_first, qreg, m, lsum, acc);
        merge_waves<D, G, NWV>(sm, Ga, m, lsum, acc, emit);
    }
}

// bf16 x 4 output store
__device__ __forceinline__ void store_out4(uint16_t *dst, const float (&o)[4]) {
    uint2 v;
    v.x = pack_bf16x2(o[0], o[1]);
    v.y = pack_bf16x2(o[2], o[3]);
    *reinterpret_cast<uint2 *>(dst) = v;
}

// Counts one finished piece of a split unit; true in the one workgroup that
// finished last (which then merges).  Each thread first waits for its
// partial stores to complete (they are device-coherent, so no cache-wide
// fence is needed).  The last workgroup leaves the counter zero.
__device__ __forceinline__ bool count_finished(int *counter, int nparts) {
    __shared__ int sm_last;
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        const int prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm_last = prev == nparts - 1;
        if (prev == nparts - 1) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return sm_last;
}

// Fused cache write (reshape_and_cache for one decode token, "ROCm
// attention backends" blog, decode path: the new token is written into the
// preshuffled cache before attention reads it): sequence s's key and value
// for kv head g go to slot slot_mapping[s] = block * B + o, the key vector of
// dims 8c..8c+7 to k_cache[block][g][c][o][0..8) and dim d of the value to
// v_cache[block][g][o / 8][d][o % 8].  Threads 0..D/8-1 write the key,
// D/8..2D/8-1 the value; the stores are complete and the workgroup has met at
// a barrier before any wave reads the cache.  Called by every thread.
template <int D, int B, int LAY>
__device__ __forceinline__ void write_new_token(const DecodeParams &p, int s, int g) {
    constexpr int C = D / 8;
    constexpr bool STD = LAY == kLayStd;
    const int64_t slot = as_const<int64_t>(p.slot_mapping)[s];
    if constexpr (LAY == kLayFp8) {
        // thread t < D / 16: K codes of dims 16 t .. 16 t + 15 (one vector);
        // D / 16 <= t < D / 8: V codes of the same dims (16 single bytes)
        constexpr int C16 = D / kFp8X;
        if (slot >= 0 && slot < p.num_blocks * B && (int)threadIdx.x < 2 * C16) {
            const int t = threadIdx.x, j = t % C16;
            const int64_t blk = slot / B;
            const int o = (int)(slot - blk * B);
            const uint4 *src =
                reinterpret_cast<const uint4 *>(t < C16 ? p.new_key : p.new_value) +
                ((size_t)s * p.Hkv + g) * C + 2 * j;
            if (t < C16) {
                uint4 *kc = reinterpret_cast<uint4 *>(const_cast<void *>(p.k_cache));
                kc[(((size_t)blk * p.Hkv + g) * C16 + j) * B + o] = quantize16(src[0], src[1], p.k_inv);
            } else {
                const uint4 vq = quantize16(src[0], src[1], p.v_inv);
                const uint32_t w[4] = {vq.x, vq.y, vq.z, vq.w};
                uint8_t *vc = reinterpret_cast<uint8_t *>(const_cast<void *>(p.v_cache)) +
                              ((((size_t)blk * p.Hkv + g) * (B / kFp8X) + o / kFp8X) * D +
                               j * kFp8X) * kFp8X + o % kFp8X;
#pragma unroll
                for (int e = 0; e < 16; e++) vc[e * kFp8X] = (uint8_t)(w[e / 4] >> ((e % 4) * 8));
            }
            wait_stores();
        }
        __syncthreads();
        return;
    }
    if (slot >= 0 && slot < p.num_blocks * B && (int)threadIdx.x < 2 * C) {
        const int t = threadIdx.x, c = t % C;
        const int64_t blk = slot / B;
        const int o = (int)(slot - blk * B);
        const size_t row = ((size_t)s * p.Hkv + g) * C + c;
        if (STD) {  // both rows are copied whole: ((blk * B + o) * Hkv + g) * C + c
            const void *src = t < C ? p.new_key : p.new_value;
            void *dst = const_cast<void *>(t < C ? p.k_cache : p.v_cache);
            reinterpret_cast<uint4 *>(dst)[((size_t)slot * p.Hkv + g) * C + c] =
                reinterpret_cast<const uint4 *>(src)[row];
        } else if (t < C) {
            const uint4 kv = reinterpret_cast<const uint4 *>(p.new_key)[row];
            uint4 *kc = reinterpret_cast<uint4 *>(const_cast<void *>(p.k_cache));
            kc[(((size_t)blk * p.Hkv + g) * C + c) * B + o] = kv;
        } else {
            const uint4 vv = reinterpret_cast<const uint4 *>(p.new_value)[row];
            uint16_t *vc = reinterpret_cast<uint16_t *>(const_cast<void *>(p.v_cache)) +
                           ((((size_t)blk * p.Hkv + g) * (B / 8) + o / 8) * D + 8 * c) * 8 + o % 8;
            const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
            for (int e = 0; e < 8; e++) vc[e * 8] = (uint16_t)(w[e / 2] >> ((e & 1) * 16));
        }
        wait_stores();
    }
    __syncthreads();
}

__device__ __forceinline__ void write_empty(const DecodeParams &p, int s, int g, int Ga, int D) {
    uint16_t *out = reinterpret_cast<uint16_t *>(p.out);
    for (int idx = threadIdx.x; idx < Ga * D; idx += blockDim.x) {
        const int hq = g * Ga + idx / D;
        out[((size_t)s * p.Hq + hq) * D + idx % D] = 0;
        if (idx % D == 0 && p.lse) p.lse[(size_t)s * p.Hq + hq] = kNegInf;
    }
}

// Explicit partitions: one workgroup per (partition, kv head, sequence),
// partition-major grid; partials in [S, Hq, max_parts, D].
template <int D, int B, int G, int SUBS, int LAY>
__global__ __launch_bounds__(256, 2) void paged_decode_kernel(DecodeParams p) {
    constexpr int DV = D / 64;
    const int units = p.S * p.Hkv;
    const int part = blockIdx.x / units;
    const int rem = blockIdx.x - part * units;
    const int s = rem / p.Hkv, g = rem - s * p.Hkv;
    const int Ga = p.Hq / p.Hkv;
    const int P = p.partition;
    const int start = part * P;
    uint16_t *out = reinterpret_cast<uint16_t *>(p.out);

    // issued together, before anything waits: the context length, the
    // block-table entries of the partition's first piece and the queries
    const int ctx_raw = as_const<int32_t>(p.context_lens)[s];
    const int bt_first = bt_entry<B, SUBS, true>(p, s, start);
    uint32_t qreg[G];
    load_queries<D, G>(p, s, g, Ga, qreg);
    const int ctx = clamp_ctx<B>(p, ctx_raw);
    if (start >= ctx) {
        if (ctx == 0 && part == 0) {
            if (p.slot_mapping) write_new_token<D, B, LAY>(p, s, g);
            write_empty(p, s, g, Ga, D);
        }
        return;
    }
    const int end = min(start + P, ctx);
    const int nparts = (ctx + P - 1) / P;
    // the partition holding the last token writes the new token first
    if (p.slot_mapping && end == ctx) write_new_token<D, B, LAY>(p, s, g);
    __shared__ MergeLDS<D, G, LAY, kWaves> sm;
    const size_t row0 = (size_t)s * p.Hq + (size_t)g * Ga;
    // partials of this unit's rows, addressed from its first row (32-bit offsets)
    const auto prs = coherent_rsrc(p.part_out + row0 * p.max_parts * D,
                                   (uint32_t)Ga * p.max_parts * D * 4);
    attend_merge<D, B, G, SUBS, LAY, kWaves>(p, s, g, start, end, bt_first, qreg, sm, Ga,
                                     [&](int h, int d, const float (&o)[4], float L) {
        const size_t orow = row0 + h;
        if (nparts == 1) {
            store_out4(out + orow * D + d, o);
            if (d == 0 && p.lse) p.lse[orow] = L;
        } else {
            store_coherent4(prs, (uint32_t)(((h * p.max_parts + part) * D + d) * 4), o[0], o[1],
                            o[2], o[3]);
            if (d == 0) store_coherent(&p.part_lse[orow * p.max_parts + part], L);
        }
    });
    if (nparts == 1) return;
    if (!count_finished(p.counters + (size_t)s * p.Hkv + g, nparts)) return;
    // up to 8 partitions (the automatic split's usual count) in one batch of
    // 8: the same sums as a batch of 16, whose extra entries add exact zeros
    if (nparts <= 8)
        merge_partition_rows<D, 4, 8, kWaves * 64>(p.part_out, p.part_lse, p.max_parts, out, p.lse,
                                                    row0, Ga, nparts);
    else
        merge_partition_rows<D, 4, 16, kWaves * 64>(p.part_out, p.part_lse, p.max_parts, out,
                                                     p.lse, row0, Ga, nparts);
}

// Balanced split.  The grid has NW workgroups (as many as are resident at
// once).  Every non-empty (sequence, kv head) unit u, of nsb_u 16-token
// sub-blocks, is cut into n_u contiguous pieces of near-equal size, one per
// workgroup: with U non-empty units and SB sub-blocks in all,
//   n_u = min(nsb_u, 1 + floor(nsb_u (NW - U) / SB))   if U <= NW,
// so that sum n_u <= NW and every piece holds about SB / NW sub-blocks
// whatever the length mix; with more units than workgroups every unit is
// one piece and the workgroups take several.  Pieces are numbered
// unit-major (unit u = s Hkv + g); workgroup w takes piece w (+ NW, ...),
// and its 4 waves take the piece's sub-blocks in turn.  A unit cut into
// pieces P_u .. P_u + n_u - 1 leaves their partials in slots P_u ..
// P_u + n_u - 1 of [NW, Ga, D] and [NW, Ga]; the last to finish merges them
// in piece order.

// Inclusive prefix sum over the wave's lanes: Hillis-Steele inside each
// 16-lane row (DPP row shifts, zero shifted in), then row 1 and 3 add the
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

// Merge of a unit's piece partials (slots P_u .. P_u + nparts - 1, in that
// order) into rows row0 .. row0 + Ga - 1: thread -> (head, 4 dims), 16
// partials per round trip.
template <int D, int NT>
__device__ __forceinline__ void merge_unit_partials(const DecodeParams &p, size_t row0, int Ga,
                                                    int P_u, int nparts, int NW) {
    constexpr int kBatch = 16;
    const auto rs = coherent_rsrc(p.part_out, (uint32_t)NW * Ga * D * 4);
    for (int it = threadIdx.x; it < Ga * (D / 4); it += NT) {
        const int h = it / (D / 4), d0 = (it % (D / 4)) * 4;
        float M = kNegInf, den = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
        for (int b = 0; b < nparts; b += kBatch) {
            float L[kBatch];
            float4 x[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; u++) {
                const int slot = P_u + (b + u < nparts ? b + u : b);
                L[u] = load_coherent(&p.part_lse[(size_t)slot * Ga + h]);
                x[u] = load_coherent4(rs, (uint32_t)(((size_t)slot * Ga + h) * D + d0) * 4);
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
            for (int e = 0; e < 4; e++) o[e] *= r;
#pragma unroll
            for (int u = 0; u < kBatch; u++) {
                const float wt = fast_exp2((L[u] - Mr) * kLog2e);
                den += wt;
                o[0] += wt * x[u].x;
                o[1] += wt * x[u].y;
                o[2] += wt * x[u].z;
                o[3] += wt * x[u].w;
            }
            M = Mb;
        }
        const float inv = den > 0.f ? 1.f / den : 0.f;
        const size_t orow = row0 + h;
        uint2 v;
        v.x = pack_bf16x2(o[0] * inv, o[1] * inv);
        v.y = pack_bf16x2(o[2] * inv, o[3] * inv);
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.out) + orow * D + d0) = v;
        if (d0 == 0 && p.lse) p.lse[orow] = den > 0.f ? M + fast_log2(den) * kLn2 : kNegInf;
    }
}

template <int D, int B, int G, int LAY, int NWV>
__global__ __launch_bounds__(NWV * 64, 8 / NWV) void paged_decode_balanced_kernel(DecodeParams p) {
    constexpr int DV = D / 64;
    const int NW = gridDim.x, w = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int Ga = p.Hq / p.Hkv, Hkv = p.Hkv;
    // clamped context length of sequence s (lane-wise; 0 past the end); the
    // first 64 are kept in a register
    auto ctx_of = [&](int s) { return s < p.S ? clamp_ctx<B>(p, p.context_lens[min(s, p.S - 1)]) : 0; };
    const int ctx_w0 = ctx_of(lane);
    auto ctx_in = [&](int c0) { return c0 == 0 ? ctx_w0 : ctx_of(c0 + lane); };

    // empty sequences: workgroup s % NW writes out = 0, lse = -inf
    for (int s = w; s < p.S; s += NW)
        if (readlane_i32(ctx_in(s & ~63), s & 63) == 0)
            for (int g = 0; g < Hkv; g++) {
                if (p.slot_mapping) write_new_token<D, B, LAY>(p, s, g);
                write_empty(p, s, g, Ga, D);
            }

    // pass 1 (every wave): sub-blocks and non-empty sequences
    int64_t SBs = 0;
    int Ns = 0;
    for (int c0 = 0; c0 < p.S; c0 += 64) {
        const int nsb = (ctx_in(c0) + kSub - 1) / kSub;
        SBs += readlane_i32(wave_prefix_sum_i(nsb), 63);
        Ns += __popcll(__ballot(nsb > 0));
    }
    if (Ns == 0) return;
    const int64_t SB = SBs * Hkv;
    const int64_t U = (int64_t)Ns * Hkv;
    const bool split = U <= NW;
    // pieces per unit of a sequence; when split, SB <= NW * 2^16 and the
    // arithmetic fits 32 bits
    const uint32_t spare = split ? (uint32_t)(NW - U) : 0u, SB32 = split ? (uint32_t)SB : 1u;
    auto pieces_of = [&](int nsb) -> int {
        if (nsb == 0) return 0;
        if (!split) return 1;
        const uint32_t n = 1u + (uint32_t)nsb * spare / SB32;
        return n < (uint32_t)nsb ? (int)n : nsb;
    };

    __shared__ MergeLDS<D, G, LAY, NWV> sm;
    for (int64_t v = w; ; v += NW) {
        // find piece v (every wave computes the same)
        int s = -1, g = 0, k = 0, n = 1, a = 0, b = 0, ctx = 0, P_u = 0;
        int64_t base = 0;  // pieces of the sequences before window c0
        for (int c0 = 0; c0 < p.S; c0 += 64) {
            const int ctx_l = ctx_in(c0);
            const int nsb_l = (ctx_l + kSub - 1) / kSub;
            const int np_l = pieces_of(nsb_l) * Hkv;
            const int incl = wave_prefix_sum_i(np_l);
            const uint64_t past = __ballot(base + incl > v);
            if (past) {
                const int i = __builtin_ctzll(past);
                const int np = readlane_i32(np_l, i);
                const int nsb = readlane_i32(nsb_l, i);
                n = np / Hkv;
                const int64_t first = base + readlane_i32(incl, i) - np;  // sequence's first piece
                const int r = (int)(v - first);
                s = c0 + i;
                g = r / n;
                k = r - g * n;
                a = (int)((uint32_t)k * (uint32_t)nsb / (uint32_t)n);
                b = (int)((uint32_t)(k + 1) * (uint32_t)nsb / (uint32_t)n);
                P_u = (int)(first + (int64_t)g * n);  // < NW when split
                ctx = readlane_i32(ctx_l, i);
                if (s >= p.S || n < 1 || g >= Hkv || (split && (int64_t)P_u + n > NW)) s = -1;
                break;
            }
            base += readlane_i32(incl, 63);
        }
        if (s < 0) break;  // no piece left for this workgroup
        if (v != w) __syncthreads();  // the LDS of the previous piece has been read

        const int tb = a * kSub, te = min(b * kSub, ctx);
        // the piece holding the last token writes the new token first
        if (p.slot_mapping && te == ctx) write_new_token<D, B, LAY>(p, s, g);
        const int bt_first = bt_entry<B, 1, true, NWV>(p, s, tb);
        uint32_t qreg[G];
        load_queries<D, G>(p, s, g, Ga, qreg);
        const size_t row0 = (size_t)s * p.Hq + (size_t)g * Ga;
        const auto prs = coherent_rsrc(p.part_out + (size_t)v * Ga * D, (uint32_t)Ga * D * 4);
        attend_merge<D, B, G, 1, LAY, NWV>(p, s, g, tb, te, bt_first, qreg, sm, Ga,
                                      [&](int h, int d, const float (&o)[4], float L) {
            if (n == 1) {
                store_out4(reinterpret_cast<uint16_t *>(p.out) + (row0 + h) * D + d, o);
                if (d == 0 && p.lse) p.lse[row0 + h] = L;
            } else {
                store_coherent4(prs, (uint32_t)((h * D + d) * 4), o[0], o[1], o[2], o[3]);
                if (d == 0) store_coherent(&p.part_lse[(size_t)v * Ga + h], L);
            }
        });
        if (n > 1 && count_finished(p.counters + (size_t)s * Hkv + g, n))
            merge_unit_partials<D, NWV * 64>(p, row0, Ga, P_u, n, NW);
        if (split) break;  // one piece per workgroup
    }
}

template <int D, int B, int G, int LAY>
hipError_t launch_partition(const DecodeParams &p, hipStream_t stream) {
    constexpr int kSubs = 1;  // waves take single sub-blocks in turn
    if (p.balanced_workgroups > 0) {
        // one wave of workgroups: as many as are resident together, counted
        // for the shuffled-layout instance and used for every layout, so the
        // split (and the rounding) does not depend on the layout
        static const int per_cu = [] {
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &n,
                    reinterpret_cast<const void *>(
                        &paged_decode_balanced_kernel<D, B, G, kLayShuffled, kWaves>),
                    kWaves * 64, 0) != hipSuccess || n < 1)
                n = 1;
            return n;
        }();
        const int nw = min(p.balanced_workgroups, per_cu * p.num_cus);
        hipLaunchKernelGGL((paged_decode_balanced_kernel<D, B, G, LAY, kWaves>),
                           dim3((unsigned)nw), dim3(kWaves * 64), 0, stream, p);
        return hipGetLastError();
    }
    const int64_t units = (int64_t)p.max_parts * p.S * p.Hkv;
    if (units > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((paged_decode_kernel<D, B, G, kSubs, LAY>), dim3((unsigned)units), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

template <int D, int B, int LAY>
hipError_t dispatch_group(const DecodeParams &p, hipStream_t stream) {
    const int Ga = p.Hq / p.Hkv;
    if (Ga <= 1) return launch_partition<D, B, 1, LAY>(p, stream);
    if (Ga <= 2) return launch_partition<D, B, 2, LAY>(p, stream);
    if (Ga <= 4) return launch_partition<D, B, 4, LAY>(p, stream);
    if (Ga <= 8) return launch_partition<D, B, 8, LAY>(p, stream);
    return launch_partition<D, B, 16, LAY>(p, stream);
}

template <int LAY>
hipError_t dispatch_layout(const DecodeParams &p, hipStream_t stream) {
    if (p.D == 128)
        return p.B == 16 ? dispatch_group<128, 16, LAY>(p, stream)
                         : dispatch_group<128, 32, LAY>(p, stream);
    return p.B == 16 ? dispatch_group<64, 16, LAY>(p, stream) : dispatch_group<64, 32, LAY>(p, stream);
}

}  // namespace

hipError_t launch_paged_decode(const DecodeParams &p, hipStream_t stream) {
    if (p.layout == kLayStd) return dispatch_layout<kLayStd>(p, stream);
    if (p.layout == kLayFp8) return dispatch_layout<kLayFp8>(p, stream);
    return dispatch_layout<kLayShuffled>(p, stream);
}

}  // namespace pa
