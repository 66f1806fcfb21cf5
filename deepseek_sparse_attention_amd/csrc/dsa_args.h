// dsa_args.h -- argument block passed by value to every DSA kernel.
#pragma once

#include <stdint.h>

#include "dsa_plan.h"

namespace dsa {

struct Args {
    // batch
    int32_t n_q, n_seq;
    const int32_t *q_seq, *q_nvis;
    int64_t max_nvis;
    // geometry
    int32_t kpool, top_k, keep, D;
    float scale_log2;     // softmax_scale * log2(e)
    // tensors
    const uint16_t *idx_q;
    const float *idx_w;
    const uint16_t *idx_k;
    int64_t key_stride;
    const uint16_t *q, *cache;
    int64_t cache_stride;
    const float *scores_in;
    float *scores;
    int64_t score_ld;
    int32_t *sel;
    int32_t sel_ld;
    int32_t *sel_count;
    float *out, *lse;
    // workspace
    uint32_t *hist;
    uint32_t *thr;        // per query: first digit of the threshold, rows above its bucket
    uint32_t *chunk_cnt;  // per (query, chunk): candidates found by k_filter
    uint64_t *cand;
    float *pacc, *pml;
    // plan
    int32_t chunk, n_chunks, cand_cap, split_rows, n_split, score_tile;
    int32_t score_ilv;   // k_score: a query's work-groups take interleaved steps of all their waves
    int32_t score_waves; // k_score: waves per work-group (4 or 8)
    int32_t fused;        // 1: dense queries are not scored, histogram accumulated
    int32_t prefill;      // 1: queries come in runs of pf_run that share a sequence
    int32_t pf_run;       // queries per run (>= 2 when prefill)
    int32_t idx_f16;      // indexer queries and keys are IEEE f16 (else bf16)
    int32_t attn_hs;      // attention kernel: 0 k_attend, 1 k_attend_hs, 2 k_attend_wv
    int32_t select_scan;  // k_select gathers its candidates itself (no k_filter)
    int32_t attn_sel;     // fused step: the top-k runs inside the attention (k_attend_sel)
    int32_t hist_on;      // the scorer accumulates the first-digit histograms
    int32_t sel_export;   // k_attend_sel writes the selection and its count to sel / sel_count
    int32_t score_valu;   // decode scorer on the vector ALU (k_score_valu), for measurement
};

// Arguments of the k-pool key producer.
struct PoolArgs {
    int32_t n_seq;
    const int32_t *n_tok, *n_new;  // per sequence: tokens held, tokens appended now
    int64_t max_new;               // host bound of n_new
    const uint16_t *new_kg;        // [n_seq][new_stride][2 * 128] key|gate cells
    int64_t new_stride;
    uint16_t *rolling;             // [n_seq][4][2 * 128]
    uint16_t *pool_keys;           // [n_seq][pool_stride][128]
    int64_t pool_stride;
    const float *pos_emb;          // [4][128]
};

// Arguments of the absorption GEMMs.
struct AbsorbArgs {
    int32_t n_q, d_rope;
    const uint16_t *q_nope;  // [n_q][64][256]
    const uint16_t *q_rope;  // [n_q][64][d_rope]
    const uint16_t *w_uk;    // [64][256][512]
    uint16_t *q_abs;         // [n_q][64][512 + d_rope]
    const float *o;          // [n_q][64][512]
    const uint16_t *w_uv;    // [64][256][512]
    float *ctx;              // [n_q][64][256]
};

// Arguments of the indexer input preparation.
struct PrepArgs {
    int32_t n_q, n_new, n_seq;
    int32_t rope;              // 1: rope on the tail 64 dimensions of every vector
    int32_t f16;               // output format: 1 IEEE f16, 0 bf16
    double inv_freq[8];        // base^(-4i/32): frequency of rope pair 4i
    double freq_ratio;         // base^(-1/32): from pair j to pair j + 1
    const int32_t *q_nvis;     // [n_q]; a query sits at position q_nvis - 1
    const float *q_in;         // [n_q][32][128], or NULL with n_q = 0
    uint16_t *q_out;           // [n_q][32][128]
    const int32_t *k_seq;      // [n_new] or NULL: key i goes to sequence i
    const int32_t *k_pos;      // [n_new] position = cache row
    const float *k_in;         // [n_new][128]
    uint16_t *k_cache;         // [n_seq][key_stride][128]
    int64_t key_stride;
};

}  // namespace dsa
