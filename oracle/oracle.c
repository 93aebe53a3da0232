/*
 * oracle.c -- plain fp64 CPU reference for paged attention over a
 * block-table KV cache in the preshuffled layout.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code,
 * header, table or helper with the GPU library; it is written from the
 * pages' statement of what is computed, not from any kernel.
 *
 * What it computes (all floating point in double precision):
 *   - the cache write into the preshuffled layout of the "ROCm attention
 *     backends" blog (ROCM_AITER_FA section, item 4, "hardware-optimised
 *     KV cache layout"):
 *         k_cache [num_blocks, kv_heads, head_dim / x, block_size, x]
 *         v_cache [num_blocks, kv_heads, block_size / x, head_dim, x]
 *     and the MLA latent cache [num_blocks, block_size, 576] (MLA section:
 *     the cache holds one 576-wide latent per token);
 *   - the gather of a token range from that layout back to the standard
 *     [tokens, heads, head_dim] layout (extend path: the fetch operator
 *     that converts context K/V to the standard layout);
 *   - exact softmax attention softmax(scale * q . K^T) V over tokens found
 *     through the block table, returning the output and the natural-log
 *     log-sum-exp of the scaled scores;
 *   - the log-sum-exp merge of partial results (extend path: each chunk
 *     yields an output and an LSE, merged stably);
 *   - extend attention by its definition: new token i of a request sees
 *     every cached token and the new tokens 0..i.
 *
 * Readings where the pages are silent (listed with the design notes):
 *   x = 8 for bf16 (one 16-byte vector); "num_heads" in the cache shapes is
 *   the number of KV heads; slot = physical_block * block_size + offset,
 *   negative or out-of-pool slots are skipped; query head h uses KV head
 *   h / (Hq / Hkv); an empty token range gives out = 0, lse = -inf.
 *
 * bf16 values arrive as raw uint16 bit patterns; bf16 -> double is exact.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---- shuffled-layout element offsets (straight from the two shapes) ---- */

/* k_cache[p][g][d / x][o][d % x] */
static int64_t k_off(int64_t p, int64_t g, int64_t d, int64_t o, int Hkv, int D, int B, int x)
{
    return ((((p * Hkv + g) * (D / x) + d / x) * B + o) * x) + d % x;
}

/* v_cache[p][g][o / x][d][o % x] */
static int64_t v_off(int64_t p, int64_t g, int64_t d, int64_t o, int Hkv, int D, int B, int x)
{
    return ((((p * Hkv + g) * (B / x) + o / x) * D + d) * x) + o % x;
}

/* ---- cache write ---- */

/* Scatter new tokens into the shuffled cache.  key/value: [T, Hkv, D]. */
void oracle_cache_write_shuffled(const uint16_t *key, const uint16_t *value,
                                 const int64_t *slot_mapping, int64_t T, int Hkv, int D,
                                 int B, int x, int64_t num_blocks,
                                 uint16_t *k_cache, uint16_t *v_cache)
{
    for (int64_t i = 0; i < T; i++) {
        int64_t slot = slot_mapping[i];
        if (slot < 0 || slot >= num_blocks * B)
            continue;
        int64_t p = slot / B, o = slot % B;
        for (int g = 0; g < Hkv; g++)
            for (int d = 0; d < D; d++) {
                int64_t src = (i * Hkv + g) * D + d;
                k_cache[k_off(p, g, d, o, Hkv, D, B, x)] = key[src];
                v_cache[v_off(p, g, d, o, Hkv, D, B, x)] = value[src];
            }
    }
}

/* Scatter new latents into the MLA cache [num_blocks, B, Dl].  latent: [T, Dl]. */
void oracle_cache_write_latent(const uint16_t *latent, const int64_t *slot_mapping, int64_t T,
                               int Dl, int B, int64_t num_blocks, uint16_t *kv_cache)
{
    for (int64_t i = 0; i < T; i++) {
        int64_t slot = slot_mapping[i];
        if (slot < 0 || slot >= num_blocks * B)
            continue;
        int64_t p = slot / B, o = slot % B;
        for (int c = 0; c < Dl; c++)
            kv_cache[(p * B + o) * Dl + c] = latent[i * Dl + c];
    }
}

/* ---- gather back to the standard layout ---- */

/* For each sequence s, copy tokens [tok_begin[s], tok_end[s]) out of the
 * shuffled cache into rows out_start[s] ... of k_out/v_out [rows, Hkv, D]. */
void oracle_gather_shuffled(const uint16_t *k_cache, const uint16_t *v_cache,
                            const int32_t *block_table, int max_blocks, int S,
                            const int32_t *tok_begin, const int32_t *tok_end,
                            const int64_t *out_start, int Hkv, int D, int B, int x,
                            uint16_t *k_out, uint16_t *v_out)
{
    for (int s = 0; s < S; s++)
        for (int64_t t = tok_begin[s]; t < tok_end[s]; t++) {
            int64_t p = block_table[(int64_t)s * max_blocks + t / B], o = t % B;
            int64_t row = out_start[s] + (t - tok_begin[s]);
            for (int g = 0; g < Hkv; g++)
                for (int d = 0; d < D; d++) {
                    k_out[(row * Hkv + g) * D + d] = k_cache[k_off(p, g, d, o, Hkv, D, B, x)];
                    v_out[(row * Hkv + g) * D + d] = v_cache[v_off(p, g, d, o, Hkv, D, B, x)];
                }
        }
}

/* ---- softmax attention of one query row over n gathered keys ----
 * z[t] holds the scaled scores and V[t * Dv ...] the gathered value rows.
 * Writes out[0..Dv) and *lse.  n == 0 gives out = 0, lse = -inf. */
static void softmax_apply(const double *z, int64_t n, const double *V, int Dv,
                          double *out, double *lse)
{
    for (int d = 0; d < Dv; d++)
        out[d] = 0.0;
    if (n == 0) {
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int64_t t = 0; t < n; t++)
        if (z[t] > m)
            m = z[t];
    double l = 0.0;
    for (int64_t t = 0; t < n; t++) {
        double e = exp(z[t] - m);
        l += e;
        for (int d = 0; d < Dv; d++)
            out[d] += e * V[t * Dv + d];
    }
    for (int d = 0; d < Dv; d++)
        out[d] /= l;
    *lse = m + log(l);
}

/* ---- GQA / MHA paged attention over a token range ----
 * q: [S, Hq, D]; out: [S, Hq, D]; lse: [S, Hq].  Sequence s attends to its
 * tokens [tok_begin[s], tok_end[s]) found through block_table.  row_mask
 * (nullable, [S, Hq]) limits the work to the selected (s, h) rows. */
void oracle_paged_attn_gqa(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                           const int32_t *block_table, int max_blocks,
                           const int32_t *tok_begin, const int32_t *tok_end, int S, int Hq,
                           int Hkv, int D, int B, int x, double scale, const uint8_t *row_mask,
                           double *out, double *lse)
{
    int group = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int s = 0; s < S; s++)
        for (int h = 0; h < Hq; h++) {
            if (row_mask && !row_mask[(int64_t)s * Hq + h])
                continue;
            int g = h / group;
            int64_t b = tok_begin[s], n = tok_end[s] - tok_begin[s];
            if (n < 0)
                n = 0;
            double *z = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
            double *V = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
            const uint16_t *qr = q + ((int64_t)s * Hq + h) * D;
            for (int64_t t = 0; t < n; t++) {
                int64_t pos = b + t;
                int64_t p = block_table[(int64_t)s * max_blocks + pos / B], o = pos % B;
                double acc = 0.0;
                for (int d = 0; d < D; d++) {
                    acc += bf(qr[d]) * bf(k_cache[k_off(p, g, d, o, Hkv, D, B, x)]);
                    V[t * D + d] = bf(v_cache[v_off(p, g, d, o, Hkv, D, B, x)]);
                }
                z[t] = scale * acc;
            }
            softmax_apply(z, n, V, D, out + ((int64_t)s * Hq + h) * D, lse + (int64_t)s * Hq + h);
            free(z);
            free(V);
        }
}

/* ---- absorbed MLA paged attention over a token range ----
 * q: [S, Hq, Dl]; kv_cache [num_blocks, B, Dl]; keys are whole latent rows,
 * values their first Dv entries.  out: [S, Hq, Dv]; lse: [S, Hq]. */
void oracle_paged_attn_mla(const uint16_t *q, const uint16_t *kv_cache,
                           const int32_t *block_table, int max_blocks,
                           const int32_t *tok_begin, const int32_t *tok_end, int S, int Hq,
                           int Dl, int Dv, int B, double scale, const uint8_t *row_mask,
                           double *out, double *lse)
{
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int s = 0; s < S; s++)
        for (int h = 0; h < Hq; h++) {
            if (row_mask && !row_mask[(int64_t)s * Hq + h])
                continue;
            int64_t b = tok_begin[s], n = tok_end[s] - tok_begin[s];
            if (n < 0)
                n = 0;
            double *z = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
            double *V = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * Dv);
            const uint16_t *qr = q + ((int64_t)s * Hq + h) * Dl;
            for (int64_t t = 0; t < n; t++) {
                int64_t pos = b + t;
                int64_t p = block_table[(int64_t)s * max_blocks + pos / B], o = pos % B;
                const uint16_t *row = kv_cache + (p * B + o) * Dl;
                double acc = 0.0;
                for (int c = 0; c < Dl; c++)
                    acc += bf(qr[c]) * bf(row[c]);
                for (int c = 0; c < Dv; c++)
                    V[t * Dv + c] = bf(row[c]);
                z[t] = scale * acc;
            }
            softmax_apply(z, n, V, Dv, out + ((int64_t)s * Hq + h) * Dv, lse + (int64_t)s * Hq + h);
            free(z);
            free(V);
        }
}

/* ---- log-sum-exp merge of n partial results ----
 * outs: [n][R][D], lses: [n][R].  L = log sum_i exp(L_i);
 * O = sum_i exp(L_i - L) O_i.  Parts with L_i = -inf carry no weight; if
 * every part is empty the result is out = 0, lse = -inf. */
void oracle_merge(int n, const double *outs, const double *lses, int64_t R, int D,
                  double *out, double *lse)
{
    for (int64_t r = 0; r < R; r++) {
        double m = -INFINITY;
        for (int i = 0; i < n; i++)
            if (lses[(int64_t)i * R + r] > m)
                m = lses[(int64_t)i * R + r];
        for (int d = 0; d < D; d++)
            out[r * D + d] = 0.0;
        if (m == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double sum = 0.0;
        for (int i = 0; i < n; i++) {
            double li = lses[(int64_t)i * R + r];
            if (li == -INFINITY)
                continue;
            sum += exp(li - m);
        }
        double L = m + log(sum);
        for (int i = 0; i < n; i++) {
            double li = lses[(int64_t)i * R + r];
            if (li == -INFINITY)
                continue;
            double w = exp(li - L);
            for (int d = 0; d < D; d++)
                out[r * D + d] += w * outs[((int64_t)i * R + r) * D + d];
        }
        lse[r] = L;
    }
}

/* ---- dense varlen attention in the standard layout ----
 * q: [Tq, Hq, D] with request r's queries at rows cu_q[r] .. cu_q[r+1];
 * k, v: [Tk, Hkv, D] with request r's keys at rows cu_k[r] .. cu_k[r+1].
 * causal != 0: bottom-right aligned mask, query i of nq sees keys
 * j <= i + (nk - nq).  out: [Tq, Hq, D]; lse: [Tq, Hq]. */
void oracle_dense_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       const int64_t *cu_q, const int64_t *cu_k, int S, int Hq, int Hkv, int D,
                       double scale, int causal, double *out, double *lse)
{
    int group = Hq / Hkv;
    for (int r = 0; r < S; r++) {
        int64_t nq = cu_q[r + 1] - cu_q[r], nk = cu_k[r + 1] - cu_k[r];
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
        for (int64_t i = 0; i < nq; i++)
            for (int h = 0; h < Hq; h++) {
                int g = h / group;
                int64_t qi = cu_q[r] + i;
                int64_t nvis = causal ? i + (nk - nq) + 1 : nk;
                if (nvis < 0)
                    nvis = 0;
                if (nvis > nk)
                    nvis = nk;
                double *z = (double *)malloc(sizeof(double) * (size_t)(nvis > 0 ? nvis : 1));
                double *V = (double *)malloc(sizeof(double) * (size_t)(nvis > 0 ? nvis : 1) * D);
                const uint16_t *qr = q + (qi * Hq + h) * D;
                for (int64_t j = 0; j < nvis; j++) {
                    int64_t kj = cu_k[r] + j;
                    double acc = 0.0;
                    for (int d = 0; d < D; d++) {
                        acc += bf(qr[d]) * bf(k[(kj * Hkv + g) * D + d]);
                        V[j * D + d] = bf(v[(kj * Hkv + g) * D + d]);
                    }
                    z[j] = scale * acc;
                }
                softmax_apply(z, nvis, V, D, out + (qi * Hq + h) * D, lse + qi * Hq + h);
                free(z);
                free(V);
            }
    }
}

/* ---- extend attention by its definition ----
 * Request r has ctx_lens[r] cached tokens (read through block_table from
 * the shuffled cache) and new tokens at query rows qsl[r] .. qsl[r+1]
 * whose K/V are k_new/v_new at the same rows.  New token i sees every
 * cached token and the new tokens 0..i.  row_mask [Tn, Hq] (nullable)
 * selects the (row, head) outputs to compute; the others are left as they
 * are. */
void oracle_extend(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                   const int32_t *qsl, const uint16_t *k_cache, const uint16_t *v_cache,
                   const int32_t *block_table, int max_blocks, const int32_t *ctx_lens, int S,
                   int Hq, int Hkv, int D, int B, int x, double scale, const uint8_t *row_mask,
                   double *out, double *lse)
{
    int group = Hq / Hkv;
    for (int r = 0; r < S; r++) {
        int64_t c = ctx_lens[r], nq = qsl[r + 1] - qsl[r];
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
        for (int64_t i = 0; i < nq; i++)
            for (int h = 0; h < Hq; h++) {
                int g = h / group;
                int64_t qi = qsl[r] + i;
                if (row_mask && !row_mask[qi * Hq + h])
                    continue;
                int64_t n = c + i + 1;
                double *z = (double *)malloc(sizeof(double) * (size_t)n);
                double *V = (double *)malloc(sizeof(double) * (size_t)n * D);
                const uint16_t *qr = q + (qi * Hq + h) * D;
                for (int64_t t = 0; t < n; t++) {
                    double acc = 0.0;
                    if (t < c) {
                        int64_t p = block_table[(int64_t)r * max_blocks + t / B], o = t % B;
                        for (int d = 0; d < D; d++) {
                            acc += bf(qr[d]) * bf(k_cache[k_off(p, g, d, o, Hkv, D, B, x)]);
                            V[t * D + d] = bf(v_cache[v_off(p, g, d, o, Hkv, D, B, x)]);
                        }
                    } else {
                        int64_t row = qsl[r] + (t - c);
                        for (int d = 0; d < D; d++) {
                            acc += bf(qr[d]) * bf(k_new[(row * Hkv + g) * D + d]);
                            V[t * D + d] = bf(v_new[(row * Hkv + g) * D + d]);
                        }
                    }
                    z[t] = scale * acc;
                }
                softmax_apply(z, n, V, D, out + (qi * Hq + h) * D, lse + qi * Hq + h);
                free(z);
                free(V);
            }
    }
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the oracle's parallel loops use from now on (for timing it on one
 * core); no effect on its results, which do not depend on the split. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n < 1 ? 1 : n);
#else
    (void)n;
#endif
}
