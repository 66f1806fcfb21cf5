/*
 * dsa.h -- C ABI of the DeepSeek Sparse Attention decode hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes, for a batch of queries against per-sequence caches:
 *   1. lightning-indexer scores of every visible cached row
 *      ("GLM 5.2 in pure C", section "The Lightning Indexer: Sparse Attention
 *      When It Helps": a rectified dot product per indexer head, weighted and
 *      summed across heads; TensorSharp2 GLM-5.x docs, table "The block":
 *      32 indexer heads of width 128, top-k 2048);
 *   2. the top-k selection that follows (same sections; ties go to the lower
 *      index as in "GLM-5.3-Flash on WASTE", section "DeepSeek Sparse
 *      Attention, k-pool flavour"; nothing is removed when no more than k rows
 *      are visible, TensorSharp2 section "The sparse-attention path");
 *   3. absorbed-MLA attention over the selected latent rows ("GLM 5.2 in pure
 *      C", section "Attention: Multi head Latent Attention With a Tiny KV
 *      Cache"; TensorSharp2 table "The block": 64 query heads, one 576-wide
 *      latent row per token, softmax scale 1/16);
 *   4. the pooled NoPE variant (WASTE "k-pool flavour"; TensorSharp2 section
 *      "GLM-5.3-Flash (glm5next)": pools of 4 tokens, keep top_k/4 pools plus
 *      the unpooled tail, 512-wide rows, K = V = latent).
 *
 * Conventions shared by every entry point
 *  - Pointers are DEVICE pointers unless stated otherwise; the geometry and
 *    batch structs are HOST structs.  bf16 tensors are raw 16-bit patterns.
 *  - Arrays are row-major with contiguous rows; strides count rows.  Every
 *    device base pointer must be 16-byte aligned.
 *  - The caller owns and allocates every buffer, including the workspace
 *    (size from dsa_workspace_bytes).  The library keeps no pointer after the
 *    work it enqueued has finished, and allocates no device memory.
 *  - Workspace contract: a workspace must be zero-filled once before its
 *    first use (dsa_workspace_init, or any zero fill).  Its first sixteenth
 *    (rounded down to whole 20 KiB blocks) holds per-query histograms of the
 *    top-k, block q for the call's query q: the 16 KiB first-digit
 *    histogram, which each call accumulates and clears again before its
 *    work completes, so that it is zero between calls, then a 4 KiB
 *    second-digit histogram, which each call clears before it uses it.
 *    Everything else follows that region.  So one workspace serves any
 *    sequence of calls,
 *    with any query counts and visible bounds, with no clearing in between
 *    (a serving loop whose batch size changes step to step keeps one
 *    workspace), provided that
 *      (a) every call passes the same ws_bytes (normally the buffer's
 *          size: the region's extent follows from it), and
 *      (b) ws_bytes >= dsa_workspace_bytes(geom, n_q, max_nvis) of the call
 *          (calls that do not fit return DSA_ERR_WORKSPACE).
 *    After a DSA_ERR_LAUNCH, or after a call that passed another ws_bytes,
 *    zero-fill it again.
 *    Calls on different streams must use different workspaces.
 *  - Errors: every entry point validates its arguments before enqueuing
 *    anything and returns a status.  On DSA_ERR_ARG, DSA_ERR_UNSUPPORTED,
 *    DSA_ERR_WORKSPACE and DSA_ERR_DEVICE nothing was enqueued and no output
 *    was written; dsa_last_error() gives a thread-local description.
 *    DSA_ERR_LAUNCH means a kernel launch was refused: outputs are then
 *    unspecified.  Faults after enqueue surface asynchronously, as for any
 *    HIP call.  No entry point throws, aborts or exits.
 *  - Per-query values that live in device memory (sequence ids, visible
 *    counts, selection indices) cannot be checked on the host.  Kernels treat
 *    a query whose sequence id is outside [0, n_seq) or whose visible count is
 *    outside [1, max_nvis] as invalid: it gets sel_count 0, no selection, and
 *    NaN output and lse.  Selection entries outside [0, cache_seq_stride)
 *    are skipped by the attention; a sel_count outside
 *    [0, top_k + kpool - 1] makes the attention of that query NaN, and a
 *    query left with no row gets NaN too.  No such value causes an
 *    out-of-bounds access.
 *  - Selection dump (a debugging aid for comparing selections line by line
 *    with another implementation, as the WASTE page does with its DSA dump,
 *    section "What is checked"): with the environment variable DSA_DUMP_SEL
 *    set to a file path, dsa_topk, dsa_decode_step and
 *    dsa_decode_step_noalloc open that file for appending before they
 *    enqueue anything (DSA_ERR_ARG if it cannot be opened), then wait for
 *    their stream and append one line per query:
 *        q=<query> nvis=<visible count> count=<selection count>: <tokens>
 *    with the selected token indices in ascending order, separated by
 *    spaces.  The fused steps report their selection even when the caller
 *    passes no selection buffer.  The wait makes such calls synchronous and
 *    unusable under graph capture (DSA_ERR_LAUNCH there).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t dsa_bf16;

enum {
    DSA_OK = 0,
    DSA_ERR_ARG = -1,          /* null pointer, bad size, misalignment, stride too small */
    DSA_ERR_UNSUPPORTED = -2,  /* a geometry this library does not implement             */
    DSA_ERR_WORKSPACE = -3,    /* workspace absent or smaller than dsa_workspace_bytes   */
    DSA_ERR_DEVICE = -4,       /* the current HIP device is not a gfx950                 */
    DSA_ERR_LAUNCH = -5        /* a kernel launch was refused                            */
};

/* Shape of one DSA attention layer.  Supported values: n_heads 64,
 * d_latent 512, d_rope 64 (token-level rows of 576) or 0 (NoPE rows of 512),
 * n_idx_heads 32, d_idx 128, kpool 1 (rows are tokens) or 4 (rows are pools),
 * 1 <= top_k <= 4096 with top_k a multiple of kpool, softmax_scale finite
 * and > 0 (the pages' value is 1/16), idx_f16 0 or 1 (1 only with kpool 1).
 * Anything else returns DSA_ERR_UNSUPPORTED rather than being approximated.
 * Zero-initialise the struct so that fields added later read as 0. */
typedef struct {
    int32_t n_heads;        /* query heads (64)                                   */
    int32_t d_latent;       /* latent width = V width = output width (512)        */
    int32_t d_rope;         /* RoPE tail of a cache row and of a query (64 or 0)  */
    int32_t n_idx_heads;    /* indexer heads (32)                                 */
    int32_t d_idx;          /* indexer head width (128)                           */
    int32_t top_k;          /* tokens kept per query (2048)                       */
    int32_t kpool;          /* tokens per indexer row: 1, or 4 for k-pool         */
    float softmax_scale;    /* multiplies the full (d_latent + d_rope) dot (1/16) */
    int32_t idx_f16;        /* 16-bit format of the indexer queries and keys:
                               0 bf16, 1 IEEE f16 (TensorSharp2 "The
                               sparse-attention path": the indexer key cache
                               is F16).  Every other 16-bit tensor is bf16.   */
} dsa_geometry;

/* The queries of one call.  A decode batch has one query per sequence with
 * n_vis = that sequence's cached length; a chunked prefill has consecutive
 * positions p of one sequence with n_vis = p + 1 (a query sees its own
 * token).  "rows(q)" below is q_nvis[q] / kpool. */
typedef struct {
    int32_t n_q;                 /* number of queries, 1..65535 (DSA_ERR_UNSUPPORTED
                                    above)                                            */
    int32_t n_seq;               /* number of sequences in the cache arrays (>= 1)    */
    const int32_t *q_seq;        /* device [n_q] sequence of each query; NULL: query i
                                    reads sequence i (then n_q <= n_seq)              */
    const int32_t *q_nvis;       /* device [n_q] visible cached tokens, 1..max_nvis   */
    int64_t max_nvis;            /* host upper bound of q_nvis, sizes grids/workspace */
    int32_t q_per_seq_hint;      /* > 1: queries come in consecutive runs of this many
                                    that share one sequence (prefill); runs that do
                                    not are still handled correctly, only slower      */
} dsa_batch;

/* Bytes of workspace that dsa_topk, dsa_mla_attend and dsa_decode_step need
 * for this geometry, query count and visible bound (the maximum of the three;
 * one workspace serves all of them): at least 16 x n_q x 20 KiB, so that the
 * histogram region (the first sixteenth) holds n_q blocks, and large enough
 * that the rest fits after that region.  Returns 0 for an unsupported geometry
 * or sizes out of range (n_q outside 1..65535, max_nvis outside 1..2^31 - 1). */
size_t dsa_workspace_bytes(const dsa_geometry *geom, int32_t n_q, int64_t max_nvis);

/* Zero-fills ws_bytes of a workspace on the stream (a fill kernel, no
 * memset node).  DSA_OK, DSA_ERR_ARG, DSA_ERR_DEVICE or DSA_ERR_LAUNCH. */
int dsa_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream);

/* 1. Indexer scores.
 *   scores[q][r] = sum_h idx_w[q][h] * max(0, sum_d idx_q[q][h][d] * idx_k[seq(q)][r][d])
 * for r < rows(q); other entries of the row are not written.
 *   idx_q  [n_q][n_idx_heads][d_idx] 16-bit    idx_w [n_q][n_idx_heads] fp32
 *   idx_k  [n_seq][key_seq_stride][d_idx] 16-bit (tokens, or pool keys for
 *          kpool 4; key_seq_stride >= max_nvis / kpool).  Any row below
 *          max_nvis / kpool of a query's sequence may be read, whatever the
 *          query's own length; only rows below rows(q) affect the result.
 *   scores [n_q][score_ld] fp32, score_ld >= max_nvis / kpool.
 * idx_q and idx_k are bf16, or IEEE f16 when geom->idx_f16 (the same holds
 * for dsa_decode_step).  Accumulation is fp32 over exact products; with
 * integer-valued inputs whose partial sums stay below 2^24 the result is
 * exact. */
int dsa_index_scores(const dsa_geometry *geom, const dsa_batch *batch,
                     const dsa_bf16 *idx_q, const float *idx_w,
                     const dsa_bf16 *idx_k, int64_t key_seq_stride,
                     float *scores, int64_t score_ld, hipStream_t stream);

/* 2. Top-k selection from scores.
 * kpool 1: if n_vis <= top_k every visible token is selected; otherwise the
 * first top_k tokens under (score descending, index ascending).
 * kpool 4: if rows(q) <= top_k/4 every visible token is selected; otherwise
 * the best top_k/4 pools under (score descending, pool ascending), expanded
 * to their 4 tokens, followed by the unpooled tail tokens [4 rows(q), n_vis).
 * -0.0 ranks equal to +0.0.  NaN scores are not supported.
 *   sel [n_q][sel_ld] int32, sel_ld >= top_k + kpool - 1: token indices in
 *   ascending order, unused slots set to -1.   sel_count [n_q] int32. */
int dsa_topk(const dsa_geometry *geom, const dsa_batch *batch,
             const float *scores, int64_t score_ld,
             int32_t *sel, int32_t sel_ld, int32_t *sel_count,
             void *ws, size_t ws_bytes, hipStream_t stream);

/* 3. Absorbed-MLA attention over selected cache rows.  For each query q and
 * head h, with D = d_latent + d_rope and t over sel[q][0..sel_count[q]):
 *   z_t = softmax_scale * sum_{d<D} q[q][h][d] * cache[seq(q)][t][d]
 *   out[q][h][j] = sum_t exp(z_t - m) cache[seq(q)][t][j] / sum_t exp(z_t - m),  j < d_latent
 *   lse[q][h] = m + ln(sum_t exp(z_t - m)),  m = max_t z_t
 *   q     [n_q][n_heads][D] bf16 (absorbed queries)
 *   cache [n_seq][cache_seq_stride][D] bf16, cache_seq_stride >= max_nvis
 *   out   [n_q][n_heads][d_latent] fp32;  lse [n_q][n_heads] fp32 or NULL.
 * bf16 products, fp32 accumulation and exponentials; the result is within
 * 2e-3 of the exact value relative to the largest |out| of the row. */
int dsa_mla_attend(const dsa_geometry *geom, const dsa_batch *batch,
                   const dsa_bf16 *q, const dsa_bf16 *cache, int64_t cache_seq_stride,
                   const int32_t *sel, int32_t sel_ld, const int32_t *sel_count,
                   float *out, float *lse,
                   void *ws, size_t ws_bytes, hipStream_t stream);

/* 4. One fused step: scores -> top-k -> attention for every query, with the
 * scoring skipped for queries that keep every visible token.  Arguments as
 * above; sel and sel_count may be NULL (then the selection stays in the
 * workspace), lse may be NULL. */
int dsa_decode_step(const dsa_geometry *geom, const dsa_batch *batch,
                    const dsa_bf16 *idx_q, const float *idx_w,
                    const dsa_bf16 *idx_k, int64_t key_seq_stride,
                    const dsa_bf16 *q, const dsa_bf16 *cache, int64_t cache_seq_stride,
                    int32_t *sel, int32_t sel_ld, int32_t *sel_count,
                    float *out, float *lse,
                    void *ws, size_t ws_bytes, hipStream_t stream);

/* The fused step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, results and errors as dsa_decode_step, without the
 * workspace: the call uses the library's own device scratch of
 * DSA_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, a static array that each GPU
 * holds from the library's load until the process ends.  A call whose
 * workspace would not fit in it (dsa_workspace_bytes above that size; the
 * 8 x 131,072-token decode needs about 16 MB) returns DSA_ERR_WORKSPACE
 * before enqueuing anything.  The call itself allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); the first call on a
 * device looks up that device's copy of the array and clears its histogram
 * region with a fill kernel on the stream.  Every call on one GPU shares
 * that GPU's scratch: calls that overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller. */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int dsa_decode_step_noalloc(const dsa_geometry *geom, const dsa_batch *batch,
                            const dsa_bf16 *idx_q, const float *idx_w,
                            const dsa_bf16 *idx_k, int64_t key_seq_stride,
                            const dsa_bf16 *q, const dsa_bf16 *cache, int64_t cache_seq_stride,
                            int32_t *sel, int32_t sel_ld, int32_t *sel_count,
                            float *out, float *lse, hipStream_t stream);

/* 5. k-pool key producer ("GLM-5.3-Flash on WASTE", "DeepSeek Sparse
 * Attention, k-pool flavour"; TensorSharp2 "GLM-5.3-Flash (glm5next)").
 * A cell is a token's indexer key followed by its gate, 2 x 128 bf16.
 * For each sequence s, which holds n_tok[s] tokens, appends n_new[s] tokens
 * whose cells are new_kg[s][0 .. n_new[s]).  Token t goes to rolling slot
 * t mod 4, and every pool that the call completes (pool p = tokens
 * 4p .. 4p+3) gets its key, per dimension d:
 *   pool_keys[s][p][d] = bf16( sum_j softmax_j(gate_j[d] + pos_emb[j][d]) * key_j[d] )
 * computed in fp32 and rounded to nearest even.  Cells of a pool that began
 * before the call are read from the rolling buffer; afterwards slots
 * 0 .. (end mod 4) - 1 hold the cells of each sequence's incomplete pool
 * (end = n_tok + n_new), and the other slots are unspecified.
 *   n_tok, n_new  device int32 [n_seq]; a sequence with n_tok < 0, n_new < 0
 *                 or n_new > max_new is left untouched
 *   max_new       host bound of n_new (sizes the grid); new_stride >= max_new
 *   new_kg        device bf16 [n_seq][new_stride][256]
 *   rolling       device bf16 [n_seq][4][256], read and written; its cells
 *                 of tokens < n_tok must be those of the current pool
 *   pool_keys     device bf16 [n_seq][pool_stride][128]; pools at or past
 *                 pool_stride are not written
 *   pos_emb       device fp32 [4][128]
 * All pointers 16-byte aligned.  No workspace.  Errors as for the calls
 * above. */
int dsa_pool_append(int32_t n_seq, const int32_t *n_tok, const int32_t *n_new, int32_t max_new,
                    const dsa_bf16 *new_kg, int64_t new_stride,
                    dsa_bf16 *rolling, dsa_bf16 *pool_keys, int64_t pool_stride,
                    const float *pos_emb, hipStream_t stream);

/* 6. Absorption GEMMs on either side of the attention ("GLM 5.2 in pure C",
 * "Attention: Multi head Latent Attention With a Tiny KV Cache";
 * TensorSharp2 table "The block": the per-head K/V decompression folded
 * into the query and the output).  64 heads.
 *   q_abs[m][h][n] = bf16( sum_{k<256} q_nope[m][h][k] * w_uk[h][k][n] )   n < 512
 *   q_abs[m][h][512 + r] = q_rope[m][h][r]                                 r < d_rope
 * fp32 accumulation, rounded to nearest even; the result is the absorbed
 * query that dsa_mla_attend and dsa_decode_step take.
 *   q_nope [n_q][64][256] bf16, q_rope [n_q][64][d_rope] bf16 (NULL if
 *   d_rope is 0), w_uk [64][256][512] bf16 (the model's key up-projection
 *   rows), q_abs [n_q][64][512 + d_rope] bf16.  d_rope is 0 or 64.
 * 1 <= n_q <= 2^20 (DSA_ERR_ARG below 1, DSA_ERR_UNSUPPORTED above). */
int dsa_absorb_query(int32_t n_q, int32_t d_rope, const dsa_bf16 *q_nope, const dsa_bf16 *q_rope,
                     const dsa_bf16 *w_uk, dsa_bf16 *q_abs, hipStream_t stream);

/*   ctx[m][h][i] = sum_{j<512} o[m][h][j] * w_uv[h][i][j]                  i < 256
 * o [n_q][64][512] fp32 (the attention output), w_uv [64][256][512] bf16
 * (the model's value up-projection rows), ctx [n_q][64][256] fp32.  o
 * enters the bf16 MFMA as two halves (truncated value + rounded
 * remainder); |error| <= 2^-14 * sum_j |o_j w_ij|.  1 <= n_q <= 2^20, as
 * for dsa_absorb_query. */
int dsa_project_output(int32_t n_q, const float *o, const dsa_bf16 *w_uv, float *ctx, hipStream_t stream);

/* 7. Indexer input preparation (TensorSharp2 "The sparse-attention path":
 * past top_k the indexer turns its queries and keys by rope and then by a
 * Walsh-Hadamard rotation before scoring, and caches its keys as F16;
 * table "The block": RoPE NORM, base 8e6, no YaRN, 64 rope dimensions).
 * Every 128-wide vector x at position p becomes, in fp32,
 *   rope (geom->d_rope = 64): for j < 32 the pair (x[64+2j], x[65+2j]) turns
 *     by t = p * rope_base^(-j/32):  (a, b) -> (a cos t - b sin t, a sin t + b cos t)
 *   rotation: y[i] = 128^(-1/2) * sum_k (-1)^popcount(i & k) * x[k]
 * and is rounded to nearest even in the indexer format (geom->idx_f16).
 * The angle is reduced modulo pi/2 in double before its sine and cosine.
 *   queries  query q (batch->n_q of them) sits at position q_nvis[q] - 1:
 *            q_in [n_q][32][128] fp32 -> q_out [n_q][32][128] 16-bit.  Both
 *            NULL: no queries are prepared.
 *   keys     key i < n_new sits at position k_pos[i] of sequence k_seq[i]
 *            (i when k_seq is NULL; then n_new <= batch->n_seq) and is
 *            written to row idx_k[seq][pos]: k_in [n_new][128] fp32 ->
 *            idx_k [batch->n_seq][key_seq_stride][128] 16-bit.  A key whose
 *            sequence is outside [0, n_seq) or position outside
 *            [0, key_seq_stride) is not written; no other row is touched.
 * Only kpool 1 is supported (DSA_ERR_UNSUPPORTED otherwise): the pages do
 * not say that the pooled variant's keys are rotated.  rope_base must be
 * finite and > 1.  Inputs and outputs must not overlap.  batch->max_nvis and
 * q_per_seq_hint are not used.  No workspace.  Errors as for the calls
 * above.  Each output is within half a unit in the last place of the 16-bit
 * format, plus 2^-20 * sum_k |x_k| / sqrt(128), of the exact transform.  Two
 * keys aimed at one row leave either of them there. */
int dsa_index_prepare(const dsa_geometry *geom, const dsa_batch *batch, double rope_base,
                      const float *q_in, dsa_bf16 *q_out,
                      int32_t n_new, const int32_t *k_seq, const int32_t *k_pos, const float *k_in,
                      dsa_bf16 *idx_k, int64_t key_seq_stride, hipStream_t stream);

/* Instrumentation for benchmarks.  With events set (n_events > 0), each
 * dsa_decode_step call on this thread launches its i-th kernel with
 * events[2 i] and events[2 i + 1] as the kernel's own start and stop marks
 * (hipExtLaunchKernel: the marks come from the dispatch, so
 * elapsed(events[2 i], events[2 i + 1]) is the kernel's execution time, as a
 * kernel trace reports it), as many as fit.  Kernel order: score, filter,
 * select, attend, split merge (ten events in all).  A kernel the call does
 * not run (the filter of a one-kernel top-k, the merge of an unsplit
 * attention) leaves its two events unrecorded; dsa_timing_ran tells which
 * ran.  Pass NULL/0 to stop.  Returns DSA_OK. */
int dsa_set_timing_events(hipEvent_t *events, int32_t n_events);

/* Bit i set: the last successful dsa_decode_step on this thread ran kernel i
 * of the order above (score 1, filter 2, select 4, attend 8, merge 16).
 * Host only; 0 before the first such call. */
int32_t dsa_timing_ran(void);

/* Bandwidth probe for benchmarks: reads bytes (a multiple of 16) from the
 * 16-byte aligned device buffer buf with non-temporal 16-byte loads in a
 * grid-stride loop, the plainest streaming read of HBM, so that a benchmark
 * can report the read bandwidth the device sustains beside its published
 * peak.  *sink (device) is written only if the loaded words xor to an
 * impossible pattern, which keeps the loads alive.  DSA_ERR_ARG for a NULL,
 * misaligned or empty buffer. */
int dsa_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Static description of a status code. */
const char *dsa_status_str(int status);

/* Thread-local description of the last non-OK status returned on this
 * thread (empty string if none). */
const char *dsa_last_error(void);

/* Checks that the current HIP device is a gfx950: DSA_OK or DSA_ERR_DEVICE. */
int dsa_device_check(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
