// dsa_plan.h -- launch plan and workspace layout shared by the host
// dispatch and the kernels of the DSA library (gfx950).
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

namespace dsa {

constexpr int kHeads = 64;        // query heads
constexpr int kLatent = 512;      // latent / V / output width
constexpr int kIdxHeads = 32;     // indexer heads
constexpr int kIdxDim = 128;      // indexer head width
constexpr int kHistBins = 4096;   // first radix digit: order-key bits 31..20
constexpr int kHistH2 = kHistBins;               // the second-digit bins of the threshold bucket follow
constexpr int kHistStride = kHistH2 + 1024;      // words per query
constexpr int kMaxTopK = 4096;
constexpr int kMaxChunks = 1024;  // top-k chunks per query (one per k_select thread)
constexpr int kAttnRows = 32;     // latent rows per attention step (one MFMA K block)
constexpr int kMaxSplitRows = 4096;  // selected rows per attention work-group
constexpr int kWvMaxRows = 2048;     // the same for k_attend_wv
constexpr size_t kScratchBytes = (size_t)32 << 20;  // workspace of the allocation-free fused step
                                                    // (DSA_NOALLOC_SCRATCH_BYTES)

// Everything a launch needs that depends on (geometry, n_q, max_nvis).
struct Plan {
    int32_t n_q;
    int64_t max_nvis;
    int32_t kpool, top_k, keep;   // keep = top_k / kpool rows
    int32_t d_rope, D;            // D = kLatent + d_rope
    int64_t max_rows;             // max_nvis / kpool
    int64_t score_ld;             // row stride of the workspace score matrix
    int32_t chunk;                // rows per top-k chunk
    int32_t n_chunks;             // chunks per query
    int32_t cand_cap;             // candidate slots per chunk
    int32_t sel_max;              // top_k + kpool - 1
    int32_t split_rows;           // selected rows per attention work-group
    int32_t n_split;              // attention splits per query
    int32_t attn_hs;              // attention kernel: 0 k_attend, 1 k_attend_hs, 2 k_attend_wv
    int32_t attn_sel;             // fused decode step: top-k inside the attention (k_attend_sel)
    int32_t select_scan;          // 1: top-k in one kernel that scans the scores
    int32_t score_tile;           // key rows per score work-group
    int32_t score_ilv;            // score work-groups take interleaved 256-row steps
    int32_t score_waves;          // waves per score work-group
    int32_t score_valu;           // decode scorer on the vector ALU instead of MFMA

    // workspace byte offsets (absolute once place_workspace has run): the
    // histograms lead, the rest (the body) follows the histogram region
    size_t off_hist;
    size_t off_thr, off_chunk, off_cand, off_scores, off_sel, off_cnt;
    size_t off_pacc, off_pml;
    size_t body;                  // bytes after the histogram region
    size_t hist_region;           // bytes of the histogram region (0 until placed)
};

constexpr size_t kHistQueryBytes = (size_t)kHistStride * 4;   // one query's histograms

// The histogram region of a workspace of ws_bytes: its first sixteenth,
// rounded down to whole blocks of kHistStride words (a query's first-digit
// histogram and the second-digit histogram of its threshold bucket).  It depends on the workspace
// size only, never on the call's shape, so calls of different query counts
// and context lengths on one workspace all find their histograms inside
// the same region -- which only histogram accumulation (and the clearing
// after it) ever touches, so it is all zero between calls -- and put
// everything else after it.
inline size_t hist_region_bytes(size_t ws_bytes) { return (ws_bytes / 16) / kHistQueryBytes * kHistQueryBytes; }

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline Plan make_plan(int32_t kpool, int32_t top_k, int32_t d_rope, int32_t n_q, int64_t max_nvis) {
    Plan p{};
    p.n_q = n_q;
    p.max_nvis = max_nvis;
    p.kpool = kpool;
    p.top_k = top_k;
    p.keep = top_k / kpool;
    p.d_rope = d_rope;
    p.D = kLatent + d_rope;
    p.max_rows = max_nvis / kpool;
    if (p.max_rows < 1) p.max_rows = 1;
    p.score_ld = (p.max_rows + 63) & ~(int64_t)63;
    p.sel_max = top_k + kpool - 1;

    // top-k chunks: aim at ~512 work-groups over the batch, 1024..8192 rows
    // each.  Longer chunks make each k_filter work-group a longer chain of
    // dependent block loads, and k_select gathers fewer chunks at once
    // (filter + select, us: the 512-position prefill chunk at 128K 79.6 with
    // 8192 rows vs 93.7 with 65536; 128 queries at 128K 28.3 vs 34.8 with
    // 32768; 64 queries 21.5 vs 24.8 with 16384)
    int64_t want = (p.max_rows * (int64_t)n_q) / 512;
    int64_t ch = 1024;
    while (ch < want && ch < 8192) ch <<= 1;
    if (const char *e = getenv("DSA_TOPK_CHUNK")) {   // tuning override: a power of two, 1024 .. 65536
        const int t = atoi(e);
        if (t >= 1024 && t <= 65536 && (t & (t - 1)) == 0) ch = t;
    }
    while ((p.max_rows + ch - 1) / ch > kMaxChunks) ch <<= 1;
    p.chunk = (int32_t)ch;
    p.n_chunks = (int32_t)((p.max_rows + ch - 1) / ch);
    p.cand_cap = p.chunk / 4;     // a chunk's candidates beyond this are found again by k_select

    // attention kernels, by batch (decode at 8 x 128K: 17.5 vs 20.4 us for
    // k_attend_wv vs k_attend_hs; at 64 queries 62 vs 94 us; at 1-2 queries
    // k_attend_hs is ~1.3 us faster; beyond 64 queries, and for a prefill
    // chunk, k_attend is as fast or faster):
    //   1..3 queries  k_attend_hs (attn_hs 1): head group x query x split,
    //                 8 waves sharing each 32-row step;
    //   4..64         k_attend_wv (attn_hs 2): the same grid, 4 waves with
    //                 private rows, merged once at the end;
    //   more          k_attend (attn_hs 0): all 64 heads per work-group.
    // The head-group kernels aim at ~64 (query, split) pairs = 256
    // work-groups, k_attend at up to 256 work-groups.  Whole 32-row steps,
    // 64..kMaxSplitRows rows per split (kWvMaxRows for k_attend_wv).  Tuning
    // overrides from the environment: DSA_ATTN_HS (0, 1 or 2) picks the
    // kernel, DSA_ATTN_PAIRS the (query, split) target.
    p.attn_hs = n_q < 4 ? 1 : n_q <= 64 ? 2 : 0;
    if (const char *e = getenv("DSA_ATTN_HS")) p.attn_hs = atoi(e) == 2 ? 2 : atoi(e) ? 1 : 0;
    // The fused decode step of up to 8 queries (not a prefill chunk) runs
    // its top-k inside the wave-private attention, k_attend_sel: no
    // k_select launch and no selection round trip through memory.  Every
    // work-group repeats its query's selection, which beyond 8 queries
    // costs as much as the launch it saves or more (128K, us per step: 9,
    // 12 and 16 queries the same either way, 87.7, 106 and 131; 64 queries,
    // attention with top-k 82.8 vs 71.7 for k_select + k_attend_wv).
    // DSA_ATTN_SEL=0 keeps k_select + the attention kernel above instead;
    // DSA_ATTN_SEL=2 takes the fused kernel up to 64 queries.
    p.attn_sel = n_q <= 8 ? 1 : 0;
    if (const char *e = getenv("DSA_ATTN_SEL"))
        p.attn_sel = atoi(e) == 2 ? (n_q <= 64 ? 1 : 0) : p.attn_sel && atoi(e) != 0;
    // k_attend_sel takes the candidates of up to 64 chunks per query straight
    // into registers (16 chunks per wave): larger chunks when a query has more
    if (p.attn_sel) {
        int64_t ch2 = p.chunk;
        while ((p.max_rows + ch2 - 1) / ch2 > 64) ch2 <<= 1;
        p.chunk = (int32_t)ch2;
        p.n_chunks = (int32_t)((p.max_rows + ch2 - 1) / ch2);
        p.cand_cap = p.chunk / 4;
    }
    // k_attend runs one work-group per CU (143 KiB of LDS): as many splits as
    // keep the grid within one round of 256 work-groups (8 x 128K at 128
    // queries: 2 splits, 100 us for attention + merge against 144 us with 1)
    // (one or two queries aim at 16 pairs per query instead: 16 splits of
    // 128 rows, merged in one round trip; measured 0.5-1.2 us faster per
    // step at C0, C4 and 2 x 128K, equal at 1 x 128K)
    const int64_t pair_target = n_q <= 2 ? 16 * (int64_t)n_q : 64;
    int64_t ns = p.attn_hs ? (pair_target + n_q - 1) / n_q : (n_q < 256 ? 256 / n_q : 1);
    const char *pairs_env = getenv("DSA_ATTN_PAIRS");
    if (pairs_env) ns = (atoi(pairs_env) + n_q - 1) / n_q;
    int64_t sr = (p.sel_max + ns - 1) / ns;
    sr = (sr + 31) / 32 * 32;
    if (p.attn_hs == 2 || p.attn_sel) {
        // the wave-private kernels deal 16-row steps to their 4 waves in
        // turn: splits of a multiple of 64 rows give every wave as many
        // steps.  The kept rows (top_k) are split evenly, and an unpooled
        // tail (up to kpool - 1 rows) goes to a split of its own (k-pool,
        // 2,048 + 3 rows, one query: 17 splits of 128 rows, step 37.7 us,
        // against 13 of 160, 38.3 us)
        sr = (p.top_k + ns - 1) / ns;
        sr = (sr + 63) / 64 * 64;
        if (sr < 64) sr = 64;
        // and at most 64 (query, split) pairs, so that the 4 head groups'
        // work-groups (one per CU) run in one round of 256: with 3, 5 or 7
        // queries the pairs had rounded up past 64, and a second round of
        // work-groups doubled the attention (3 queries at 128K: attention
        // with top-k 27.5 us with 22 splits of 96 rows, 16.6 with 16 of 128;
        // 7 queries 33.1 vs 18.6 us)
        while (!pairs_env && sr < kWvMaxRows && (int64_t)n_q * ((p.sel_max + sr - 1) / sr) > 64) sr += 64;
    }
    if (sr < 64) sr = 64;
    if (sr > kMaxSplitRows) sr = kMaxSplitRows;
    if ((p.attn_hs == 2 || p.attn_sel) && sr > kWvMaxRows) sr = kWvMaxRows;
    p.split_rows = (int32_t)sr;
    p.n_split = (int32_t)((p.sel_max + sr - 1) / sr);

    // top-k: when a query's rows fit one 16,384-row tile, one work-group per
    // query scans its scores (no k_filter); beyond that the scan is bound by
    // one CU's load rate and the chunked k_filter + k_select pair is faster
    // (8 x 64K rows: 64.1 vs 71.1 us per step).  DSA_SELECT_SCAN=0/1 forces
    // either path.
    p.select_scan = p.max_rows <= 16384 ? 1 : 0;
    if (const char *e = getenv("DSA_SELECT_SCAN")) p.select_scan = atoi(e) ? 1 : 0;

    // score tiles: 1024 rows per work-group (4 waves x 4 steps of 64 rows).
    // Only a batch of under 128 such tiles (a short context) halves the tile,
    // down to 256 rows (one step per wave), until it has 128: smaller tiles
    // pay the histogram's per-work-group setup and flush more often (one
    // query over 128K rows: 13.2 us with 1024-row tiles, 14.9 with 256;
    // one over 4,096 rows: 12.3 us with 1024, 7.4 with 256)
    int64_t tile = 1024;
    while (tile > 256 && (int64_t)n_q * ((p.max_rows + tile - 1) / tile) < 128) tile >>= 1;
    // Between one and two work-groups per CU of 1,024-row tiles, some CUs
    // would take two and the rest one; 2,048-row tiles (with 8 waves, see
    // below) give every busy CU one (3 queries at 128K: 42.6 vs 43.7 us).
    // Between two and four, the second round of work-groups would be partly
    // empty; 4,096-row tiles with 8 waves run in one round (128K, us per
    // step: 5 queries 55.8-56.0 vs 56.7, 6 queries 60.9 vs 61.3, 7 queries
    // 67.0-67.2 vs 68.1-68.2; 8 queries, 1,024 tiles, gain nothing)
    {
        const int64_t n1024 = (int64_t)n_q * ((p.max_rows + 1023) / 1024);
        if (tile == 1024 && n1024 > 256 && n1024 < 512) tile = 2048;
        if (tile == 1024 && n1024 > 512 && n1024 < 1024) tile = 4096;
    }
    if (const char *e = getenv("DSA_SCORE_TILE")) {   // tuning override: a power of two, 256 .. 8192
        const int t = atoi(e);
        if (t >= 256 && t <= 8192 && (t & (t - 1)) == 0) tile = t;
    }
    p.score_tile = (int32_t)tile;
    // With whole 1024-row tiles a query's work-groups take interleaved
    // 256-row steps (work-group x: rows 256 x + 256 G i, G work-groups per
    // query), so that at any time they read one window of the query's keys
    // together (8 x 128K: 44.4 vs 45.6 us); DSA_SCORE_ILV=0/1 forces either.
    p.score_ilv = tile >= 1024 ? 1 : 0;
    if (const char *e = getenv("DSA_SCORE_ILV")) p.score_ilv = atoi(e) != 0;
    // A batch of at most 256 whole 1,024-row tiles (one or two queries at
    // 128K, the k-pool query) has one work-group per CU either way: 8 waves
    // per work-group then keep twice the key steps in flight per CU (C4 38.4
    // vs 38.8 us per step, one query at 128K 34.0 vs 34.3, two 37.3 vs 37.9);
    // larger batches keep 4 waves and two work-groups per CU (8 x 128K with
    // 8 waves: 77.9 vs 73.3 us).  DSA_SCORE_WAVES=4/8 forces either.
    const int64_t n_tiles = (int64_t)n_q * ((p.max_rows + tile - 1) / tile);
    p.score_waves = tile >= 1024 && n_tiles <= 256 ? 8 : 4;
    if (const char *e = getenv("DSA_SCORE_WAVES")) p.score_waves = atoi(e) == 8 ? 8 : 4;
    // DSA_SCORE_VALU=1: the decode scorer on v_dot2_f32_bf16 instead of MFMA
    // (k_score_valu; bf16 inputs), kept to measure the choice
    p.score_valu = 0;
    if (const char *e = getenv("DSA_SCORE_VALU")) p.score_valu = atoi(e) != 0;

    size_t o = 0;
    p.off_hist = 0;
    p.off_thr = o;    o += align256((size_t)n_q * 8);
    p.off_chunk = o;  o += align256((size_t)n_q * p.n_chunks * 4);
    p.off_cand = o;   o += align256((size_t)n_q * p.n_chunks * p.cand_cap * 8);
    p.off_scores = o; o += align256((size_t)n_q * p.score_ld * 4);
    p.off_sel = o;    o += align256((size_t)n_q * p.sel_max * 4);
    p.off_cnt = o;    o += align256((size_t)n_q * 4);
    p.off_pacc = o;   o += align256((size_t)n_q * p.n_split * kHeads * kLatent * 4);
    p.off_pml = o;    o += align256((size_t)n_q * p.n_split * kHeads * 2 * 4);
    p.body = o;
    p.hist_region = 0;
    return p;
}

// Smallest workspace for the plan: with k = the histogram blocks its first
// sixteenth holds (k = ws / (16 blocks), rounded down), k >= n_q and
// k blocks + body <= ws.  Growing ws for the body can raise k, which the
// loop follows until both hold.
inline size_t workspace_bytes(const Plan &p) {
    size_t k = (size_t)p.n_q;
    for (;;) {
        const size_t h = k * kHistQueryBytes * 16, b = k * kHistQueryBytes + p.body;
        const size_t w = align256(h > b ? h : b);
        const size_t kk = w / (kHistQueryBytes * 16);
        if (kk <= k) return w;
        k = kk;
    }
}

// Lays the plan out in a workspace of ws_bytes; false if it does not fit.
inline bool place_workspace(Plan &p, size_t ws_bytes) {
    const size_t h = hist_region_bytes(ws_bytes);
    if ((size_t)p.n_q * kHistQueryBytes > h || h + p.body > ws_bytes) return false;
    p.hist_region = h;
    p.off_thr += h;
    p.off_chunk += h;
    p.off_cand += h;
    p.off_scores += h;
    p.off_sel += h;
    p.off_cnt += h;
    p.off_pacc += h;
    p.off_pml += h;
    return true;
}

}  // namespace dsa
