/*
 * dsa_oracle.c -- plain CPU definition of the DeepSeek Sparse Attention
 * decode hot path (lightning-indexer scores, top-k selection, absorbed-MLA
 * attention over the selection, and the pooled "k-pool" NoPE variant).
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the oracle that the HIP path is
 * checked against.  Only the test-suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.  It
 * shares no code, header, table or helper with the HIP library: it is built
 * by gcc from this one file.
 *
 * Precision: every floating-point sum is formed in double from the bf16
 * inputs and rounded to float once, when stored.  With integer-valued
 * indexer inputs (as in every workload here) the scores are exact.
 *
 * Sources (pages on GLM-5.x and DeepSeek Sparse Attention):
 *  [TS]  TensorSharp2 docs, "GLM-5.x (glm-dsa, glm5next)": table "The block";
 *        section "The sparse-attention path"; section "GLM-5.3-Flash
 *        (glm5next)" and its table.
 *  [PC]  "GLM 5.2 in pure C" (Medium): sections "Attention: Multi head Latent
 *        Attention With a Tiny KV Cache" and "The Lightning Indexer: Sparse
 *        Attention When It Helps".
 *  [WA]  "GLM-5.3-Flash on WASTE" (sqliteai/warp docs/GLM.md): section
 *        "DeepSeek Sparse Attention, k-pool flavour".
 *  [ST]  Strata PR "Add GLM-5.3-Flash (glm5-next) support": "What a glm5-next
 *        block has that nothing else in the engine does"; "Known gaps".
 *
 * Readings taken where the pages are silent or disagree (each is listed in
 * the design notes as well):
 *  - the score carries no 1/sqrt(128) or 1/sqrt(32) factor: the problem
 *    statement's score is sum_h w_h * relu(q_h . k); positive constants do
 *    not change the ranking and a caller may fold them into w;
 *  - top-k keeps exactly min(k, n) rows: everything ranked at or above the
 *    k-th under the total order (score descending, index ascending), so
 *    equal scores go to the lower index;
 *  - the selection is reported in ascending token order, padded with -1;
 *  - k-pool: dense (every visible token) while the complete pools number at
 *    most top_k/kpool; otherwise the best top_k/kpool pools, expanded to
 *    their tokens, plus the unpooled tail [kpool*n_pools, n_vis) always;
 *  - the softmax scale multiplies the whole 576-wide (or 512-wide) dot; V is
 *    the first d_latent columns of the selected rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the upper half of an IEEE float: widen it exactly. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double f16_value(uint16_t bits)
{
    const int e = (bits >> 10) & 31;
    const int f = bits & 1023;
    double v;
    if (e == 0) v = ldexp((double)f, -24);                 /* zero and subnormals */
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), e - 25);
    return (bits & 0x8000u) ? -v : v;
}

/* An indexer element: bf16 bits, or IEEE f16 bits when f16 is set. */
static double idx_value(uint16_t bits, int32_t f16)
{
    return f16 ? f16_value(bits) : bf16_value(bits);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the parallel loops that follow (timing only: results do
 * not depend on it). */
void oracle_set_threads(int32_t n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Indexer score of every visible row ([PC] "The Lightning Indexer": a
 * rectified dot product per indexer head, then a weighted sum across heads;
 * [TS] "The block": 32 indexer heads of width 128 score every cached token).
 *
 *   s[q][r] = sum_{h < n_idx_heads} w[q][h] * max(0, sum_{d < d_idx} qi[q][h][d] * K[seq(q)][r][d])
 *
 * for r < rows(q) = q_nvis[q] / kpool.  Rows are tokens (kpool = 1) or
 * complete pools of kpool tokens ([WA] "k-pool flavour": one compressed
 * 128-wide key per pool).  Entries of s at r >= rows(q) are left untouched.
 * qi and K hold bf16, or IEEE f16 when idx_f16 is set ([TS] "The
 * sparse-attention path": the indexer key cache is F16).
 */
int oracle_index_scores(int32_t n_q, const int32_t *q_seq, const int32_t *q_nvis,
                        int32_t kpool, int32_t n_idx_heads, int32_t d_idx,
                        const uint16_t *idx_q, const float *idx_w,
                        const uint16_t *idx_k, int64_t key_seq_stride,
                        float *scores, int64_t score_ld, int32_t idx_f16)
{
    for (int32_t q = 0; q < n_q; q++) {
        const int64_t rows = q_nvis[q] / kpool;
        const int64_t seq = q_seq ? q_seq[q] : q;
        const uint16_t *qi = idx_q + (int64_t)q * n_idx_heads * d_idx;
        const float *w = idx_w + (int64_t)q * n_idx_heads;
        const uint16_t *K = idx_k + seq * key_seq_stride * d_idx;
        #pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; r++) {
            const uint16_t *k = K + r * d_idx;
            double acc = 0.0;
            for (int32_t h = 0; h < n_idx_heads; h++) {
                double dot = 0.0;
                for (int32_t d = 0; d < d_idx; d++)
                    dot += idx_value(qi[h * d_idx + d], idx_f16) * idx_value(k[d], idx_f16);
                if (dot > 0.0)
                    acc += (double)w[h] * dot;
            }
            scores[(int64_t)q * score_ld + r] = (float)acc;
        }
    }
    return 0;
}

typedef struct {
    float s;
    int64_t r;
} scored_row;

/* Total order of the selection: higher score first, equal scores by lower
 * index ([WA] "k-pool flavour": ties are ordered by index upstream).  The
 * float comparison treats -0 and +0 as equal. */
static int by_score_then_index(const void *pa, const void *pb)
{
    const scored_row *a = (const scored_row *)pa, *b = (const scored_row *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->r > b->r) - (a->r < b->r);
}

static int by_index(const void *pa, const void *pb)
{
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    return (a > b) - (a < b);
}

/*
 * Top-k selection ([PC] "The Lightning Indexer": keep the best index_topk
 * positions, and with fewer visible keys than that keep them all -- the dense
 * case of [TS] "The sparse-attention path"; [WA] "k-pool flavour": keep the
 * best index_topk/index_kpool pools, attend their tokens plus the tail that
 * has not filled a pool; [ST] "Known gaps": the tail is appended).
 *
 * Output per query: sel[q][0..count) in ascending token order, the rest of
 * the sel_ld slots set to -1; sel_count[q] = count.
 * Returns 0, or -1 if sel_ld cannot hold a selection.
 */
int oracle_topk(int32_t n_q, const int32_t *q_nvis, int32_t kpool, int32_t top_k,
                const float *scores, int64_t score_ld,
                int32_t *sel, int32_t sel_ld, int32_t *sel_count)
{
    const int64_t keep = top_k / kpool;
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int32_t q = 0; q < n_q; q++) {
        const int64_t n_vis = q_nvis[q];
        const int64_t rows = n_vis / kpool;
        int32_t *dst = sel + (int64_t)q * sel_ld;
        int64_t count = 0;
        if (rows <= keep) {
            /* nothing to remove: every visible token */
            if (n_vis > sel_ld) { bad = 1; continue; }
            for (int64_t t = 0; t < n_vis; t++)
                dst[count++] = (int32_t)t;
        } else {
            scored_row *all = (scored_row *)malloc((size_t)rows * sizeof *all);
            int64_t *pick = (int64_t *)malloc((size_t)keep * sizeof *pick);
            for (int64_t r = 0; r < rows; r++) {
                all[r].s = scores[(int64_t)q * score_ld + r];
                all[r].r = r;
            }
            qsort(all, (size_t)rows, sizeof *all, by_score_then_index);
            for (int64_t i = 0; i < keep; i++)
                pick[i] = all[i].r;
            qsort(pick, (size_t)keep, sizeof *pick, by_index);
            const int64_t tail = n_vis - rows * kpool;
            if (keep * kpool + tail > sel_ld) {
                bad = 1;
            } else {
                for (int64_t i = 0; i < keep; i++)
                    for (int64_t j = 0; j < kpool; j++)
                        dst[count++] = (int32_t)(pick[i] * kpool + j);
                for (int64_t t = rows * kpool; t < n_vis; t++)
                    dst[count++] = (int32_t)t;
            }
            free(all);
            free(pick);
        }
        sel_count[q] = (int32_t)count;
        for (int64_t i = count; i < sel_ld; i++)
            dst[i] = -1;
    }
    return bad ? -1 : 0;
}

/*
 * Absorbed-MLA attention over the selected rows ([PC] "Attention: Multi head
 * Latent Attention With a Tiny KV Cache": the absorbed query is dotted with
 * the latent and the rotary part of each cached row, scaled, softmaxed, and
 * the latents are pooled with those weights; [TS] "The block": one 576-wide
 * row per token, 64 query heads and one key head, softmax scale 1/16;
 * [TS] "GLM-5.3-Flash" and [ST]: NoPE rows are the 512-wide latent alone).
 *
 * For query q, head h, and each selected token t:
 *   z_t = scale * sum_{d < D} qt[q][h][d] * C[seq(q)][t][d],  D = d_latent + d_rope
 *   out[q][h][j] = sum_t exp(z_t - m) * C[t][j] / sum_t exp(z_t - m),  j < d_latent
 *   lse[q][h]   = m + log(sum_t exp(z_t - m)),  m = max_t z_t
 */
int oracle_mla_attend(int32_t n_q, const int32_t *q_seq, int32_t n_heads,
                      int32_t d_latent, int32_t d_rope, float scale,
                      const uint16_t *q, const uint16_t *cache, int64_t cache_seq_stride,
                      const int32_t *sel, int32_t sel_ld, const int32_t *sel_count,
                      float *out, float *lse)
{
    const int32_t D = d_latent + d_rope;
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int32_t qq = 0; qq < n_q; qq++) {
        for (int32_t h = 0; h < n_heads; h++) {
            const int64_t seq = q_seq ? q_seq[qq] : qq;
            const int32_t n = sel_count[qq];
            const int32_t *rows = sel + (int64_t)qq * sel_ld;
            const uint16_t *qh = q + ((int64_t)qq * n_heads + h) * D;
            const uint16_t *C = cache + seq * cache_seq_stride * D;
            double *z = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof *z);
            double *o = (double *)calloc((size_t)d_latent, sizeof *o);
            double m = -INFINITY;
            for (int32_t i = 0; i < n; i++) {
                const uint16_t *c = C + (int64_t)rows[i] * D;
                double dot = 0.0;
                for (int32_t d = 0; d < D; d++)
                    dot += bf16_value(qh[d]) * bf16_value(c[d]);
                z[i] = (double)scale * dot;
                if (z[i] > m) m = z[i];
            }
            double l = 0.0;
            for (int32_t i = 0; i < n; i++) {
                const double p = exp(z[i] - m);
                const uint16_t *c = C + (int64_t)rows[i] * D;
                l += p;
                for (int32_t j = 0; j < d_latent; j++)
                    o[j] += p * bf16_value(c[j]);
            }
            float *dst = out + ((int64_t)qq * n_heads + h) * d_latent;
            for (int32_t j = 0; j < d_latent; j++)
                dst[j] = (float)(o[j] / l);
            if (lse)
                lse[(int64_t)qq * n_heads + h] = (float)(m + log(l));
            free(z);
            free(o);
        }
    }
    return 0;
}

/*
 * One decode (or prefill-chunk) step: scores, then top-k, then attention,
 * for every query of the batch ([TS] "The sparse-attention path": below
 * top_k cached tokens the scoring is skipped and attention is dense, which
 * the top-k definition above already yields).  Scores live in a scratch
 * buffer owned by this call.  sel/sel_count are outputs (caller-sized).
 */
int oracle_decode_step(int32_t n_q, const int32_t *q_seq, const int32_t *q_nvis,
                       int32_t kpool, int32_t top_k, int32_t n_heads,
                       int32_t d_latent, int32_t d_rope, float scale,
                       int32_t n_idx_heads, int32_t d_idx,
                       const uint16_t *idx_q, const float *idx_w,
                       const uint16_t *idx_k, int64_t key_seq_stride,
                       const uint16_t *q, const uint16_t *cache, int64_t cache_seq_stride,
                       int32_t *sel, int32_t sel_ld, int32_t *sel_count,
                       float *out, float *lse, int32_t idx_f16)
{
    int64_t max_rows = 1;
    for (int32_t i = 0; i < n_q; i++)
        if (q_nvis[i] / kpool > max_rows) max_rows = q_nvis[i] / kpool;
    float *scores = (float *)malloc((size_t)n_q * (size_t)max_rows * sizeof *scores);
    if (!scores) return -2;
    int rc = oracle_index_scores(n_q, q_seq, q_nvis, kpool, n_idx_heads, d_idx,
                                 idx_q, idx_w, idx_k, key_seq_stride, scores, max_rows, idx_f16);
    if (rc == 0)
        rc = oracle_topk(n_q, q_nvis, kpool, top_k, scores, max_rows, sel, sel_ld, sel_count);
    if (rc == 0)
        rc = oracle_mla_attend(n_q, q_seq, n_heads, d_latent, d_rope, scale, q, cache,
                               cache_seq_stride, sel, sel_ld, sel_count, out, lse);
    free(scores);
    return rc;
}

/*
 * k-pool key producer.
 *
 * [WA] "DeepSeek Sparse Attention, k-pool flavour": a pool's compressed key
 * is one 128-wide vector per four adjacent tokens, computed once, when the
 * pool's last token arrives; the per-step state is a rolling buffer of the
 * (key, gate) pairs of the pool being filled plus an append-only array of
 * finished pool keys.  [TS] "GLM-5.3-Flash (glm5next)" table: [key|gate] is
 * cached per cell and a softmax over the gates, plus a per-slot position
 * embedding, compresses each pool.
 *
 * Readings: the softmax runs over the four slots separately for every key
 * dimension d ([ST]'s verification notes list "one softmax over the whole
 * pool block instead of per key-dim" as a rival that must disagree), and the
 * position embedding E[j][d] is added to the gate logit:
 *     K[d] = sum_j exp(a_j) key_j[d] / sum_j exp(a_j),   a_j = gate_j[d] + E[j][d].
 * A cell is key (d_idx bf16) followed by gate (d_idx bf16).  The pool key is
 * stored as bf16, rounded to nearest (ties to even) from the double value.
 */

/* Nearest bf16 (ties to even) of a double in the normal range. */
static uint16_t bf16_from_double(double v)
{
    if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
    int e;
    const double m = frexp(fabs(v), &e);         /* |v| = m * 2^e, m in [0.5, 1) */
    const double r = rint(ldexp(m, 8));          /* 8 significant bits, ties to even */
    float f = (float)ldexp(r, e - 8);            /* exact */
    if (v < 0) f = -f;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* Compresses the four cells c[j] (each 2 * d_idx bf16) into out[d_idx]. */
static void pool_compress(const uint16_t *const c[4], int32_t d_idx, const float *pos_emb, uint16_t *out)
{
    for (int32_t d = 0; d < d_idx; d++) {
        double a[4], m = -INFINITY;
        for (int j = 0; j < 4; j++) {
            a[j] = bf16_value(c[j][d_idx + d]) + (double)pos_emb[j * d_idx + d];
            if (a[j] > m) m = a[j];
        }
        double num = 0.0, den = 0.0;
        for (int j = 0; j < 4; j++) {
            const double e = exp(a[j] - m);
            num += e * bf16_value(c[j][d]);
            den += e;
        }
        out[d] = bf16_from_double(num / den);
    }
}

/*
 * Appends n_new[s] tokens to sequence s, which holds n_tok[s] tokens: token
 * t = n_tok[s] + i takes its cell from new_kg[s][i] into rolling slot t mod 4;
 * when that slot is 3, pool t / 4 is complete and its key is written to
 * pool_keys[s][t / 4].  Token by token, in order.
 *   new_kg    [n_seq][new_stride][2 d_idx]  bf16
 *   rolling   [n_seq][4][2 d_idx]           bf16 (read and updated)
 *   pool_keys [n_seq][pool_stride][d_idx]   bf16
 *   pos_emb   [4][d_idx]                    float
 */
int oracle_pool_append(int32_t n_seq, const int32_t *n_tok, const int32_t *n_new,
                       const uint16_t *new_kg, int64_t new_stride, int32_t d_idx,
                       uint16_t *rolling, uint16_t *pool_keys, int64_t pool_stride,
                       const float *pos_emb)
{
    const int64_t cell = 2 * (int64_t)d_idx;
    for (int32_t s = 0; s < n_seq; s++) {
        uint16_t *roll = rolling + (int64_t)s * 4 * cell;
        for (int32_t i = 0; i < n_new[s]; i++) {
            const int64_t t = (int64_t)n_tok[s] + i;
            const int slot = (int)(t % 4);
            memcpy(roll + slot * cell, new_kg + ((int64_t)s * new_stride + i) * cell,
                   (size_t)cell * sizeof *roll);
            if (slot == 3) {
                const uint16_t *c[4] = {roll, roll + cell, roll + 2 * cell, roll + 3 * cell};
                pool_compress(c, d_idx, pos_emb, pool_keys + ((int64_t)s * pool_stride + t / 4) * d_idx);
            }
        }
    }
    return 0;
}

/*
 * Absorption of the per-head key and value up-projections ("GLM 5.2 in pure
 * C", section "Attention: Multi head Latent Attention With a Tiny KV Cache":
 * by linearity q . k_nope = (W_K^T q) . L, so the query absorbs the key
 * up-projection once, scores are dots against the latent, and the pooled
 * latent is projected back out per head at the end; TensorSharp2 table "The
 * block": the K/V decompression is folded into the query and the output).
 *
 *   q_abs[m][h][n]        = sum_{k < d_nope} q_nope[m][h][k] * w_uk[h][k][n]   (n < d_latent)
 *   q_abs[m][h][d_latent + r] = q_rope[m][h][r]                               (r < d_rope)
 *   ctx[m][h][i]          = sum_{j < d_latent} o[m][h][j] * w_uv[h][i][j]      (i < d_v)
 *
 * q_abs is stored as bf16 (nearest, ties to even, from the double sum); ctx
 * as float.  Weight layouts follow the model's up-projection rows: w_uk
 * [H][d_nope][d_latent] (row k of head h), w_uv [H][d_v][d_latent].
 */
int oracle_absorb_query(int32_t n_q, int32_t n_heads, int32_t d_nope, int32_t d_latent, int32_t d_rope,
                        const uint16_t *q_nope, const uint16_t *q_rope, const uint16_t *w_uk,
                        uint16_t *q_abs)
{
    const int64_t D = d_latent + d_rope;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int32_t m = 0; m < n_q; m++) {
        for (int32_t h = 0; h < n_heads; h++) {
            const uint16_t *qn = q_nope + ((int64_t)m * n_heads + h) * d_nope;
            const uint16_t *W = w_uk + (int64_t)h * d_nope * d_latent;
            uint16_t *dst = q_abs + ((int64_t)m * n_heads + h) * D;
            for (int32_t n = 0; n < d_latent; n++) {
                double acc = 0.0;
                for (int32_t k = 0; k < d_nope; k++)
                    acc += bf16_value(qn[k]) * bf16_value(W[(int64_t)k * d_latent + n]);
                dst[n] = bf16_from_double(acc);
            }
            for (int32_t r = 0; r < d_rope; r++)
                dst[d_latent + r] = q_rope[((int64_t)m * n_heads + h) * d_rope + r];
        }
    }
    return 0;
}

int oracle_project_output(int32_t n_q, int32_t n_heads, int32_t d_latent, int32_t d_v,
                          const float *o, const uint16_t *w_uv, float *ctx)
{
    #pragma omp parallel for collapse(2) schedule(static)
    for (int32_t m = 0; m < n_q; m++) {
        for (int32_t h = 0; h < n_heads; h++) {
            const float *oh = o + ((int64_t)m * n_heads + h) * d_latent;
            const uint16_t *W = w_uv + (int64_t)h * d_v * d_latent;
            float *dst = ctx + ((int64_t)m * n_heads + h) * d_v;
            for (int32_t i = 0; i < d_v; i++) {
                double acc = 0.0;
                for (int32_t j = 0; j < d_latent; j++)
                    acc += (double)oh[j] * bf16_value(W[(int64_t)i * d_latent + j]);
                dst[i] = (float)acc;
            }
        }
    }
    return 0;
}

/*
 * Indexer input preparation ([TS] "The sparse-attention path": once the
 * context passes top_k the indexer applies rope and then a Walsh-Hadamard
 * rotation to its queries and keys before scoring; the rotation is
 * orthonormal and its own inverse, so it cancels in exact arithmetic, but the
 * indexer key cache is F16 and rotating before the rounding spreads the
 * rounding error evenly over the 128 dimensions.  [TS] "The block": RoPE
 * NORM, base 8e6, no YaRN, on a 64-wide rope slice).
 *
 * For one d_idx-wide vector x at position p, in double:
 *   rope:     for j < d_rope / 2 the pair (x[o + 2j], x[o + 2j + 1]),
 *             o = d_idx - d_rope, turns by the angle p * base^(-2j / d_rope):
 *                 (a, b) -> (a cos t - b sin t, a sin t + b cos t)
 *   rotation: y[i] = d_idx^(-1/2) * sum_j (-1)^popcount(i & j) * x[j]
 * Readings: the rope slice is the tail of the head, as in the attention
 * query and cache row where the rope part follows the NoPE part; NORM turns
 * adjacent pairs in place; the rotation is the Sylvester-ordered Hadamard
 * matrix, scaled to be orthonormal.  d_idx is a power of two.
 */
void oracle_index_rotate(int32_t d_idx, int32_t d_rope, double base, int64_t pos,
                         const double *x, double *y)
{
    double r[1024];
    memcpy(r, x, (size_t)d_idx * sizeof *r);
    const int32_t o = d_idx - d_rope;
    for (int32_t j = 0; j < d_rope / 2; j++) {
        const double t = (double)pos * pow(base, -2.0 * j / d_rope);
        const double a = x[o + 2 * j], b = x[o + 2 * j + 1];
        r[o + 2 * j] = a * cos(t) - b * sin(t);
        r[o + 2 * j + 1] = a * sin(t) + b * cos(t);
    }
    const double norm = 1.0 / sqrt((double)d_idx);
    for (int32_t i = 0; i < d_idx; i++) {
        double acc = 0.0;
        for (int32_t j = 0; j < d_idx; j++)
            acc += (__builtin_popcount((unsigned)(i & j)) & 1) ? -r[j] : r[j];
        y[i] = acc * norm;
    }
}

/* Nearest IEEE f16 (ties to even) of a double, subnormals and overflow to
 * infinity included. */
static uint16_t f16_from_double(double v)
{
    const uint16_t sign = signbit(v) ? 0x8000u : 0u;
    const double a = fabs(v);
    if (isnan(a)) return 0x7e00u;
    if (a < ldexp(1.0, -14))                      /* quantum 2^-24; may round up to 2^-14 */
        return sign | (uint16_t)rint(ldexp(a, 24));
    int e;
    double m = frexp(a, &e);                      /* a = m * 2^e, m in [0.5, 1) */
    double r = rint(ldexp(m, 11));                /* 11 significant bits, ties to even */
    if (r == 2048.0) { r = 1024.0; e += 1; }
    const int E = e - 1 + 15;
    if (E >= 31) return sign | 0x7c00u;
    return sign | (uint16_t)(E << 10) | (uint16_t)((int)r - 1024);
}

/* Rounds n doubles to bf16 or (f16 set) IEEE f16 bits. */
void oracle_round16(int64_t n, const double *v, uint16_t *out, int32_t f16)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = f16 ? f16_from_double(v[i]) : bf16_from_double(v[i]);
}

/*
 * Prepares a step's indexer inputs from their float projections:
 *  - query head h of query q sits at position q_nvis[q] - 1 (the query's own
 *    token is the last one it sees) and goes to q_out[q][h];
 *  - new key i sits at position k_pos[i] of sequence k_seq[i] (i when k_seq
 *    is NULL) and is appended at that row of the key cache,
 *    k_cache[seq][pos]; a key whose sequence or position lies outside
 *    [0, n_seq) x [0, key_seq_stride) is not written.
 * Each vector is rotated as above and rounded to bf16, or f16 when idx_f16.
 *   q_in [n_q][n_idx_heads][d_idx], k_in [n_new][d_idx] float.
 */
int oracle_index_prepare(int32_t n_q, int32_t n_idx_heads, int32_t d_idx, int32_t d_rope, double base,
                         const int32_t *q_nvis, const float *q_in, uint16_t *q_out,
                         int32_t n_new, int32_t n_seq, const int32_t *k_seq, const int32_t *k_pos,
                         const float *k_in, uint16_t *k_cache, int64_t key_seq_stride, int32_t idx_f16)
{
    if (d_idx > 1024 || (d_idx & (d_idx - 1)) || d_rope < 0 || d_rope > d_idx || (d_rope & 1)) return -1;
    const int64_t n_vec = (int64_t)n_q * n_idx_heads;
    #pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < n_vec + n_new; v++) {
        double x[1024], y[1024];
        const float *src;
        uint16_t *dst;
        int64_t pos;
        if (v < n_vec) {
            pos = (int64_t)q_nvis[v / n_idx_heads] - 1;
            src = q_in + v * d_idx;
            dst = q_out + v * d_idx;
        } else {
            const int64_t i = v - n_vec;
            const int64_t seq = k_seq ? k_seq[i] : i;
            pos = k_pos[i];
            if (seq < 0 || seq >= n_seq || pos < 0 || pos >= key_seq_stride) continue;
            src = k_in + i * d_idx;
            dst = k_cache + (seq * key_seq_stride + pos) * d_idx;
        }
        for (int32_t d = 0; d < d_idx; d++) x[d] = (double)src[d];
        oracle_index_rotate(d_idx, d_rope, base, pos, x, y);
        oracle_round16(d_idx, y, dst, idx_f16);
    }
    return 0;
}
