// dsa_api.cpp -- host side of the C ABI declared in include/dsa.h:
// argument validation, workspace plan, path choice and kernel enqueue on
// the caller's stream.  Nothing here allocates device memory or waits for
// the device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dsa.h"
#include "dsa_plan.h"

#include "dsa_args.h"

namespace dsa {
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st);
hipError_t launch_score(const Args &a, int64_t max_rows, hipStream_t st, hipEvent_t ev0 = nullptr,
                        hipEvent_t ev1 = nullptr);
hipError_t launch_hist(const Args &a, hipStream_t st);
hipError_t launch_filter(const Args &a, hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_select(const Args &a, hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_attend(const Args &a, hipStream_t st, const hipEvent_t *ev = nullptr);
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st);
hipError_t launch_pool_append(const PoolArgs &a, hipStream_t st);
hipError_t launch_absorb(const AbsorbArgs &a, hipStream_t st);
hipError_t launch_project(const AbsorbArgs &a, hipStream_t st);
hipError_t launch_index_prep(const PrepArgs &a, hipStream_t st);
hipError_t scratch_acquire(hipStream_t st, void **ptr);
void scratch_mark_dirty();
}  // namespace dsa

static_assert(DSA_NOALLOC_SCRATCH_BYTES == dsa::kScratchBytes, "scratch size in the header and the library agree");

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t *g_events = nullptr;
thread_local int32_t g_n_events = 0;
thread_local int32_t g_ran = 0;   // kernels the last dsa_decode_step on this thread ran (bit i: kernel i)

// Queries per call of the attention path: its kernels take one grid row
// (gridDim.y) per query.
constexpr int32_t kMaxQueries = 65535;

// Queries per absorption call: keeps the 1-D grid (512 work-groups of 256
// threads per 64 queries) under 2^32 work-items.
constexpr int32_t kMaxAbsorbQueries = 1 << 20;

// Timing event i of this call, or NULL when instrumentation is off.
hipEvent_t timing_event(int32_t i) { return g_events && i < g_n_events ? g_events[i] : nullptr; }

int fail(int status, const std::string &msg) {
    g_last_error = msg;
    return status;
}

// Per-device result of the architecture check (0 unknown, 1 gfx950, 2 other).
std::atomic<int> g_dev_ok[64];

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return fail(DSA_ERR_DEVICE, "no current HIP device");
    if (dev < 64) {
        int s = g_dev_ok[dev].load(std::memory_order_acquire);
        if (s == 1) return DSA_OK;
        if (s == 2) return fail(DSA_ERR_DEVICE, "current device is not a gfx950");
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return fail(DSA_ERR_DEVICE, "hipGetDeviceProperties failed");
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_release);
    if (!ok) return fail(DSA_ERR_DEVICE, std::string("current device is ") + prop.gcnArchName + ", not gfx950");
    return DSA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_geometry(const dsa_geometry *g) {
    if (!g) return fail(DSA_ERR_ARG, "geometry is NULL");
    if (g->n_heads != dsa::kHeads || g->d_latent != dsa::kLatent || g->n_idx_heads != dsa::kIdxHeads ||
        g->d_idx != dsa::kIdxDim)
        return fail(DSA_ERR_UNSUPPORTED, "only n_heads 64, d_latent 512, n_idx_heads 32, d_idx 128 are implemented");
    if (g->d_rope != 64 && g->d_rope != 0) return fail(DSA_ERR_UNSUPPORTED, "d_rope must be 64 or 0");
    if (g->kpool != 1 && g->kpool != 4) return fail(DSA_ERR_UNSUPPORTED, "kpool must be 1 or 4");
    if (g->top_k < 1 || g->top_k > dsa::kMaxTopK || g->top_k % g->kpool != 0)
        return fail(DSA_ERR_UNSUPPORTED, "top_k must be in [1, 4096] and a multiple of kpool");
    if (!(std::isfinite(g->softmax_scale) && g->softmax_scale > 0.f))
        return fail(DSA_ERR_UNSUPPORTED, "softmax_scale must be finite and positive");
    if (g->idx_f16 != 0 && g->idx_f16 != 1) return fail(DSA_ERR_UNSUPPORTED, "idx_f16 must be 0 or 1");
    if (g->idx_f16 && g->kpool != 1) return fail(DSA_ERR_UNSUPPORTED, "f16 indexer inputs need kpool 1");
    return DSA_OK;
}

int check_batch(const dsa_batch *b) {
    if (!b) return fail(DSA_ERR_ARG, "batch is NULL");
    if (b->n_q < 1) return fail(DSA_ERR_ARG, "n_q must be >= 1");
    if (b->n_q > kMaxQueries) return fail(DSA_ERR_UNSUPPORTED, "n_q must be <= 65535 (one grid row per query)");
    if (b->n_seq < 1) return fail(DSA_ERR_ARG, "n_seq must be >= 1");
    if (!b->q_nvis) return fail(DSA_ERR_ARG, "q_nvis is NULL");
    if (!b->q_seq && b->n_q > b->n_seq) return fail(DSA_ERR_ARG, "q_seq NULL needs n_q <= n_seq");
    if (b->max_nvis < 1 || b->max_nvis > (int64_t)INT32_MAX) return fail(DSA_ERR_ARG, "max_nvis must be in [1, 2^31)");
    if (!aligned16(b->q_nvis) || (b->q_seq && !aligned16(b->q_seq)))
        return fail(DSA_ERR_ARG, "q_seq / q_nvis must be 16-byte aligned");
    return DSA_OK;
}

#define DSA_TRY(expr)                         \
    do {                                      \
        int _s = (expr);                      \
        if (_s != DSA_OK) return _s;          \
    } while (0)

bool test_fail_launch() {
    const char *e = std::getenv("DSA_TEST_FAIL_LAUNCH");
    return e && e[0] == '1';
}

// DSA_DUMP_SEL=<path>: every call that selects appends its queries'
// selections to <path>, one line per query (format in dsa.h).  The file is
// opened before anything is enqueued and written once the work is done.
struct SelDump {
    FILE *f = nullptr;
    ~SelDump() {
        if (f) std::fclose(f);
    }
    int open() {
        const char *path = std::getenv("DSA_DUMP_SEL");
        if (!path || !*path) return DSA_OK;
        f = std::fopen(path, "a");
        return f ? (int)DSA_OK : fail(DSA_ERR_ARG, std::string("DSA_DUMP_SEL: cannot open ") + path);
    }
    int write(const dsa_batch *b, const int32_t *sel, int32_t sel_ld, const int32_t *cnt, hipStream_t st) {
        if (!f) return DSA_OK;
        const size_t n = (size_t)b->n_q;
        std::vector<int32_t> hs(n * sel_ld), hc(n), hv(n);
        if (hipStreamSynchronize(st) != hipSuccess ||
            hipMemcpy(hs.data(), sel, hs.size() * 4, hipMemcpyDeviceToHost) != hipSuccess ||
            hipMemcpy(hc.data(), cnt, n * 4, hipMemcpyDeviceToHost) != hipSuccess ||
            hipMemcpy(hv.data(), b->q_nvis, n * 4, hipMemcpyDeviceToHost) != hipSuccess)
            return fail(DSA_ERR_LAUNCH, "DSA_DUMP_SEL: reading the selection back failed");
        for (size_t q = 0; q < n; q++) {
            std::fprintf(f, "q=%zu nvis=%d count=%d:", q, hv[q], hc[q]);
            const int32_t c = hc[q] < 0 ? 0 : (hc[q] > sel_ld ? sel_ld : hc[q]);
            for (int32_t i = 0; i < c; i++) std::fprintf(f, " %d", hs[q * sel_ld + i]);
            std::fputc('\n', f);
        }
        std::fflush(f);
        return DSA_OK;
    }
};

dsa::Args base_args(const dsa_geometry *g, const dsa_batch *b, const dsa::Plan &p) {
    dsa::Args a;
    std::memset(&a, 0, sizeof a);
    a.n_q = b->n_q;
    a.n_seq = b->n_seq;
    a.q_seq = b->q_seq;
    a.q_nvis = b->q_nvis;
    a.max_nvis = b->max_nvis;
    a.kpool = g->kpool;
    a.top_k = g->top_k;
    a.keep = p.keep;
    a.D = p.D;
    a.scale_log2 = g->softmax_scale * 1.4426950408889634f;
    a.chunk = p.chunk;
    a.n_chunks = p.n_chunks;
    a.cand_cap = p.cand_cap;
    a.split_rows = p.split_rows;
    a.n_split = p.n_split;
    a.attn_hs = p.attn_hs;
    a.select_scan = p.select_scan;
    a.score_tile = p.score_tile;
    a.score_ilv = p.score_ilv;
    a.score_waves = p.score_waves;
    a.score_valu = p.score_valu;
    a.prefill = b->q_per_seq_hint >= 2 ? 1 : 0;
    a.pf_run = b->q_per_seq_hint;
    a.idx_f16 = g->idx_f16;
    return a;
}

void bind_workspace(dsa::Args &a, const dsa::Plan &p, void *ws) {
    uint8_t *w = static_cast<uint8_t *>(ws);
    a.hist = reinterpret_cast<uint32_t *>(w + p.off_hist);
    a.thr = reinterpret_cast<uint32_t *>(w + p.off_thr);
    a.chunk_cnt = reinterpret_cast<uint32_t *>(w + p.off_chunk);
    a.cand = reinterpret_cast<uint64_t *>(w + p.off_cand);
    a.pacc = reinterpret_cast<float *>(w + p.off_pacc);
    a.pml = reinterpret_cast<float *>(w + p.off_pml);
}

int launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(DSA_ERR_LAUNCH, std::string(what) + ": " + hipGetErrorString(e));
    return DSA_OK;
}

// Lays the plan out in the caller's workspace (the histogram region's size
// follows from ws_bytes alone); refuses a workspace it does not fit.
int check_ws(dsa::Plan &p, const void *ws, size_t ws_bytes) {
    if (!ws) return fail(DSA_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned16(ws)) return fail(DSA_ERR_ARG, "workspace must be 16-byte aligned");
    if (!dsa::place_workspace(p, ws_bytes))
        return fail(DSA_ERR_WORKSPACE, "workspace has " + std::to_string(ws_bytes) + " bytes, needs " +
                                           std::to_string(dsa::workspace_bytes(p)));
    return DSA_OK;
}

template <class F>
int guarded(F &&f) {
    try {
        g_last_error.clear();
        return f();
    } catch (...) {
        return fail(DSA_ERR_ARG, "unexpected host exception");
    }
}

}  // namespace

extern "C" {

const char *dsa_status_str(int s) {
    switch (s) {
        case DSA_OK: return "ok";
        case DSA_ERR_ARG: return "invalid argument";
        case DSA_ERR_UNSUPPORTED: return "unsupported geometry";
        case DSA_ERR_WORKSPACE: return "workspace missing or too small";
        case DSA_ERR_DEVICE: return "current device is not a gfx950";
        case DSA_ERR_LAUNCH: return "kernel launch refused";
        default: return "unknown status";
    }
}

const char *dsa_last_error(void) { return g_last_error.c_str(); }

int32_t dsa_timing_ran(void) { return g_ran; }

int dsa_set_timing_events(hipEvent_t *events, int32_t n_events) {
    g_events = (events && n_events > 0) ? events : nullptr;
    g_n_events = g_events ? n_events : 0;
    return DSA_OK;
}

int dsa_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
    return guarded([&] {
        DSA_TRY(check_device());
        if (!buf || !aligned16(buf) || bytes == 0 || bytes % 16 != 0 || !sink)
            return fail(DSA_ERR_ARG, "stream_read: buffer NULL, misaligned or empty, or sink NULL");
        return launched(dsa::launch_stream_read(buf, bytes, sink, stream), "stream_read");
    });
}

int dsa_device_check(void) {
    return guarded([&] { return check_device(); });
}

size_t dsa_workspace_bytes(const dsa_geometry *g, int32_t n_q, int64_t max_nvis) {
    if (check_geometry(g) != DSA_OK || n_q < 1 || n_q > kMaxQueries || max_nvis < 1 || max_nvis > (int64_t)INT32_MAX)
        return 0;
    return dsa::workspace_bytes(dsa::make_plan(g->kpool, g->top_k, g->d_rope, n_q, max_nvis));
}

int dsa_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream) {
    return guarded([&] {
        DSA_TRY(check_device());
        if (!ws || !aligned16(ws)) return fail(DSA_ERR_ARG, "workspace NULL or misaligned");
        if (test_fail_launch()) return fail(DSA_ERR_LAUNCH, "injected launch failure (DSA_TEST_FAIL_LAUNCH)");
        return launched(dsa::launch_fill_zero(ws, ws_bytes, stream), "fill");
    });
}

int dsa_index_scores(const dsa_geometry *g, const dsa_batch *b, const dsa_bf16 *idx_q, const float *idx_w,
                     const dsa_bf16 *idx_k, int64_t key_seq_stride, float *scores, int64_t score_ld,
                     hipStream_t stream) {
    return guarded([&] {
        DSA_TRY(check_device());
        DSA_TRY(check_geometry(g));
        DSA_TRY(check_batch(b));
        if (!idx_q || !idx_w || !idx_k || !scores) return fail(DSA_ERR_ARG, "NULL tensor pointer");
        if (!aligned16(idx_q) || !aligned16(idx_w) || !aligned16(idx_k) || !aligned16(scores))
            return fail(DSA_ERR_ARG, "tensor pointers must be 16-byte aligned");
        dsa::Plan p = dsa::make_plan(g->kpool, g->top_k, g->d_rope, b->n_q, b->max_nvis);
        if (key_seq_stride < p.max_rows) return fail(DSA_ERR_ARG, "key_seq_stride < max_nvis / kpool");
        if (score_ld < p.max_rows) return fail(DSA_ERR_ARG, "score_ld < max_nvis / kpool");
        if (test_fail_launch()) return fail(DSA_ERR_LAUNCH, "injected launch failure (DSA_TEST_FAIL_LAUNCH)");
        dsa::Args a = base_args(g, b, p);
        a.idx_q = idx_q;
        a.idx_w = idx_w;
        a.idx_k = idx_k;
        a.key_stride = key_seq_stride;
        a.scores = scores;
        a.score_ld = score_ld;
        a.fused = 0;
        return launched(dsa::launch_score(a, p.max_rows, stream), "score");
    });
}

int dsa_topk(const dsa_geometry *g, const dsa_batch *b, const float *scores, int64_t score_ld, int32_t *sel,
             int32_t sel_ld, int32_t *sel_count, void *ws, size_t ws_bytes, hipStream_t stream) {
    return guarded([&] {
        DSA_TRY(check_device());
        DSA_TRY(check_geometry(g));
        DSA_TRY(check_batch(b));
        if (!scores || !sel || !sel_count) return fail(DSA_ERR_ARG, "NULL tensor pointer");
        if (!aligned16(scores) || !aligned16(sel) || !aligned16(sel_count))
            return fail(DSA_ERR_ARG, "tensor pointers must be 16-byte aligned");
        dsa::Plan p = dsa::make_plan(g->kpool, g->top_k, g->d_rope, b->n_q, b->max_nvis);
        if (score_ld < p.max_rows) return fail(DSA_ERR_ARG, "score_ld < max_nvis / kpool");
        if (sel_ld < p.sel_max) return fail(DSA_ERR_ARG, "sel_ld < top_k + kpool - 1");
        DSA_TRY(check_ws(p, ws, ws_bytes));
        if (test_fail_launch()) return fail(DSA_ERR_LAUNCH, "injected launch failure (DSA_TEST_FAIL_LAUNCH)");
        SelDump dump;
        DSA_TRY(dump.open());
        dsa::Args a = base_args(g, b, p);
        bind_workspace(a, p, ws);
        a.scores_in = scores;
        a.score_ld = score_ld;
        a.sel = sel;
        a.sel_ld = sel_ld;
        a.sel_count = sel_count;
        DSA_TRY(launched(dsa::launch_hist(a, stream), "hist"));
        if (!a.select_scan) DSA_TRY(launched(dsa::launch_filter(a, stream), "filter"));
        DSA_TRY(launched(dsa::launch_select(a, stream), "select"));
        return dump.write(b, sel, sel_ld, sel_count, stream);
    });
}

int dsa_mla_attend(const dsa_geometry *g, const dsa_batch *b, const dsa_bf16 *q, const dsa_bf16 *cache,
                   int64_t cache_seq_stride, const int32_t *sel, int32_t sel_ld, const int32_t *sel_count,
                   float *out, float *lse, void *ws, size_t ws_bytes, hipStream_t stream) {
    return guarded([&] {
        DSA_TRY(check_device());
        DSA_TRY(check_geometry(g));
        DSA_TRY(check_batch(b));
        if (!q || !cache || !sel || !sel_count || !out) return fail(DSA_ERR_ARG, "NULL tensor pointer");
        if (!aligned16(q) || !aligned16(cache) || !aligned16(sel) || !aligned16(sel_count) || !aligned16(out) ||
            (lse && !aligned16(lse)))
            return fail(DSA_ERR_ARG, "tensor pointers must be 16-byte aligned");
        dsa::Plan p = dsa::make_plan(g->kpool, g->top_k, g->d_rope, b->n_q, b->max_nvis);
        if (cache_seq_stride < b->max_nvis) return fail(DSA_ERR_ARG, "cache_seq_stride < max_nvis");
        if (sel_ld < p.sel_max) return fail(DSA_ERR_ARG, "sel_ld < top_k + kpool - 1");
        DSA_TRY(check_ws(p, ws, ws_bytes));
        if (test_fail_launch()) return fail(DSA_ERR_LAUNCH, "injected launch failure (DSA_TEST_FAIL_LAUNCH)");
        dsa::Args a = base_args(g, b, p);
        bind_workspace(a, p, ws);
        a.q = q;
        a.cache = cache;
        a.cache_stride = cache_seq_stride;
        a.sel = const_cast<int32_t *>(sel);
        a.sel_ld = sel_ld;
        a.sel_count = const_cast<int32_t *>(sel_count);
        a.out = out;
        a.lse = lse;
        return launched(dsa::launch_attend(a, stream), "attend");
    });
}

}  // extern "C"

namespace {

// Argument checks of the fused step that do not concern the workspace; the
// plan is made here.
int check_step(const dsa_geometry *g, const dsa_batch *b, const dsa_bf16 *idx_q, const float *idx_w,
               const dsa_bf16 *idx_k, int64_t key_seq_stride, const dsa_bf16 *q, const dsa_bf16 *cache,
               int64_t cache_seq_stride, const int32_t *sel, int32_t sel_ld, const int32_t *sel_count,
               const float *out, const float *lse, dsa::Plan &p) {
    DSA_TRY(check_geometry(g));
    DSA_TRY(check_batch(b));
    if (!idx_q || !idx_w || !idx_k || !q || !cache || !out) return fail(DSA_ERR_ARG, "NULL tensor pointer");
    if (!aligned16(idx_q) || !aligned16(idx_w) || !aligned16(idx_k) || !aligned16(q) || !aligned16(cache) ||
        !aligned16(out) || (lse && !aligned16(lse)) || (sel && !aligned16(sel)) ||
        (sel_count && !aligned16(sel_count)))
        return fail(DSA_ERR_ARG, "tensor pointers must be 16-byte aligned");
    if ((sel == nullptr) != (sel_count == nullptr)) return fail(DSA_ERR_ARG, "sel and sel_count go together");
    p = dsa::make_plan(g->kpool, g->top_k, g->d_rope, b->n_q, b->max_nvis);
    if (key_seq_stride < p.max_rows) return fail(DSA_ERR_ARG, "key_seq_stride < max_nvis / kpool");
    if (cache_seq_stride < b->max_nvis) return fail(DSA_ERR_ARG, "cache_seq_stride < max_nvis");
    if (sel && sel_ld < p.sel_max) return fail(DSA_ERR_ARG, "sel_ld < top_k + kpool - 1");
    return DSA_OK;
}

// Enqueues the fused step on a plan already placed in the workspace ws.
int enqueue_step(const dsa_geometry *g, const dsa_batch *b, const dsa::Plan &p, const dsa_bf16 *idx_q,
                 const float *idx_w, const dsa_bf16 *idx_k, int64_t key_seq_stride, const dsa_bf16 *q,
                 const dsa_bf16 *cache, int64_t cache_seq_stride, int32_t *sel, int32_t sel_ld, int32_t *sel_count,
                 float *out, float *lse, void *ws, hipStream_t stream) {
    SelDump dump;
    DSA_TRY(dump.open());
    dsa::Args a = base_args(g, b, p);
    bind_workspace(a, p, ws);
    uint8_t *w = static_cast<uint8_t *>(ws);
    a.idx_q = idx_q;
    a.idx_w = idx_w;
    a.idx_k = idx_k;
    a.key_stride = key_seq_stride;
    a.scores = reinterpret_cast<float *>(w + p.off_scores);
    a.scores_in = a.scores;
    a.score_ld = p.score_ld;
    a.q = q;
    a.cache = cache;
    a.cache_stride = cache_seq_stride;
    if (sel) {
        a.sel = sel;
        a.sel_ld = sel_ld;
        a.sel_count = sel_count;
    } else {
        a.sel = reinterpret_cast<int32_t *>(w + p.off_sel);
        a.sel_ld = p.sel_max;
        a.sel_count = reinterpret_cast<int32_t *>(w + p.off_cnt);
    }
    a.out = out;
    a.lse = lse;
    a.fused = 1;
    // decode batches select inside the attention (k_attend_sel); a prefill
    // chunk keeps k_select
    a.attn_sel = p.attn_sel && !a.prefill ? 1 : 0;
    a.sel_export = sel || dump.f ? 1 : 0;
    // the scorer's histograms feed k_filter, k_select's own scan, or the
    // in-attention scan, which k_reduce then clears; an unsplit in-attention
    // scan (no k_reduce) builds its own
    a.hist_on = (a.attn_sel && a.select_scan && a.n_split <= 1) ? 0 : 1;
    hipEvent_t ev[10];
    for (int32_t i = 0; i < 10; i++) ev[i] = timing_event(i);
    g_ran = 0;
    DSA_TRY(launched(dsa::launch_score(a, p.max_rows, stream, ev[0], ev[1]), "score"));
    if (!a.select_scan) DSA_TRY(launched(dsa::launch_filter(a, stream, ev[2], ev[3]), "filter"));
    if (!a.attn_sel) DSA_TRY(launched(dsa::launch_select(a, stream, ev[4], ev[5]), "select"));
    DSA_TRY(launched(dsa::launch_attend(a, stream, g_events ? ev + 6 : nullptr), "attend"));
    g_ran = 1 | (a.select_scan ? 0 : 2) | (a.attn_sel ? 0 : 4) | 8 | (a.n_split > 1 ? 16 : 0);
    return dump.write(b, a.sel, a.sel_ld, a.sel_count, stream);
}

}  // namespace

extern "C" {

int dsa_decode_step(const dsa_geometry *g, const dsa_batch *b, const dsa_bf16 *idx_q, const float *idx_w,
                    const dsa_bf16 *idx_k, int64_t key_seq_stride, const dsa_bf16 *q, const dsa_bf16 *cache,
                    int64_t cache_seq_stride, int32_t *sel, int32_t sel_ld, int32_t *sel_count, float *out,
                    float *lse, void *ws, size_t ws_bytes, hipStream_t stream) {
    return guarded([&] {
        DSA_TRY(check_device());
        dsa::Plan p;
        DSA_TRY(check_step(g, b, idx_q, idx_w, idx_k, key_seq_stride, q, cache, cache_seq_stride, sel, sel_ld,
                           sel_count, out, lse, p));
        DSA_TRY(check_ws(p, ws, ws_bytes));
        if (test_fail_launch()) return fail(DSA_ERR_LAUNCH, "injected launch failure (DSA_TEST_FAIL_LAUNCH)");
        return enqueue_step(g, b, p, idx_q, idx_w, idx_k, key_seq_stride, q, cache, cache_seq_stride, sel, sel_ld,
                            sel_count, out, lse, ws, stream);
    });
}

int dsa_decode_step_noalloc(const dsa_geometry *g, const dsa_batch *b, const dsa_bf16 *idx_q, const float *idx_w,
                            const dsa_bf16 *idx_k, int64_t key_seq_stride, const dsa_bf16 *q, const dsa_bf16 *cache,
                            int64_t cache_seq_stride, int32_t *sel, int32_t sel_ld, int32_t *sel_count, float *out,
                            float *lse, hipStream_t stream) {
    return guarded([&] {
        DSA_TRY(check_device());
        dsa::Plan p;
        DSA_TRY(check_step(g, b, idx_q, idx_w, idx_k, key_seq_stride, q, cache, cache_seq_stride, sel, sel_ld,
                           sel_count, out, lse, p));
        if (!dsa::place_workspace(p, dsa::kScratchBytes))
            return fail(DSA_ERR_WORKSPACE, "the call needs a workspace of " + std::to_string(dsa::workspace_bytes(p)) +
                                               " bytes; the allocation-free entry point's scratch holds " +
                                               std::to_string(dsa::kScratchBytes));
        if (test_fail_launch()) return fail(DSA_ERR_LAUNCH, "injected launch failure (DSA_TEST_FAIL_LAUNCH)");
        void *ws = nullptr;
        DSA_TRY(launched(dsa::scratch_acquire(stream, &ws), "scratch"));
        const int s = enqueue_step(g, b, p, idx_q, idx_w, idx_k, key_seq_stride, q, cache, cache_seq_stride, sel,
                                   sel_ld, sel_count, out, lse, ws, stream);
        if (s != DSA_OK) dsa::scratch_mark_dirty();
        return s;
    });
}

int dsa_pool_append(int32_t n_seq, const int32_t *n_tok, const int32_t *n_new, int32_t max_new,
                    const dsa_bf16 *new_kg, int64_t new_stride, dsa_bf16 *rolling, dsa_bf16 *pool_keys,
                    int64_t pool_stride, const float *pos_emb, hipStream_t stream) {
    return guarded([&] {
        DSA_TRY(check_device());
        if (n_seq < 1) return fail(DSA_ERR_ARG, "n_seq < 1");
        if (max_new < 0) return fail(DSA_ERR_ARG, "max_new < 0");
        if (new_stride < (max_new > 0 ? max_new : 1)) return fail(DSA_ERR_ARG, "new_stride < max_new");
        if (pool_stride < 1) return fail(DSA_ERR_ARG, "pool_stride < 1");
        if (!n_tok || !n_new || !new_kg || !rolling || !pool_keys || !pos_emb)
            return fail(DSA_ERR_ARG, "NULL pointer");
        if (!aligned16(n_tok) || !aligned16(n_new) || !aligned16(new_kg) || !aligned16(rolling) ||
            !aligned16(pool_keys) || !aligned16(pos_emb))
            return fail(DSA_ERR_ARG, "pointers must be 16-byte aligned");
        if (test_fail_launch()) return fail(DSA_ERR_LAUNCH, "injected launch failure (DSA_TEST_FAIL_LAUNCH)");
        dsa::PoolArgs a;
        a.n_seq = n_seq;
        a.n_tok = n_tok;
        a.n_new = n_new;
        a.max_new = max_new;
        a.new_kg = new_kg;
        a.new_stride = new_stride;
        a.rolling = rolling;
        a.pool_keys = pool_keys;
        a.pool_stride = pool_stride;
        a.pos_emb = pos_emb;
        return launched(dsa::launch_pool_append(a, stream), "pool_append");
    });
}

int dsa_absorb_query(int32_t n_q, int32_t d_rope, const dsa_bf16 *q_nope, const dsa_bf16 *q_rope,
                     const dsa_bf16 *w_uk, dsa_bf16 *q_abs, hipStream_t stream) {
    return guarded([&] {
        DSA_TRY(check_device());
        if (n_q < 1) return fail(DSA_ERR_ARG, "n_q < 1");
        if (n_q > kMaxAbsorbQueries) return fail(DSA_ERR_UNSUPPORTED, "n_q > 2^20");
        if (d_rope != 0 && d_rope != 64) return fail(DSA_ERR_UNSUPPORTED, "d_rope must be 0 or 64");
        if (!q_nope || !w_uk || !q_abs || (d_rope && !q_rope)) return fail(DSA_ERR_ARG, "NULL pointer");
        if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_abs) || (d_rope && !aligned16(q_rope)))
            return fail(DSA_ERR_ARG, "pointers must be 16-byte aligned");
        if (test_fail_launch()) return fail(DSA_ERR_LAUNCH, "injected launch failure (DSA_TEST_FAIL_LAUNCH)");
        dsa::AbsorbArgs a{};
        a.n_q = n_q;
        a.d_rope = d_rope;
        a.q_nope = q_nope;
        a.q_rope = q_rope;
        a.w_uk = w_uk;
        a.q_abs = q_abs;
        return launched(dsa::launch_absorb(a, stream), "absorb");
    });
}

int dsa_project_output(int32_t n_q, const float *o, const dsa_bf16 *w_uv, float *ctx, hipStream_t stream) {
    return guarded([&] {
        DSA_TRY(check_device());
        if (n_q < 1) return fail(DSA_ERR_ARG, "n_q < 1");
        if (n_q > kMaxAbsorbQueries) return fail(DSA_ERR_UNSUPPORTED, "n_q > 2^20");
        if (!o || !w_uv || !ctx) return fail(DSA_ERR_ARG, "NULL pointer");
        if (!aligned16(o) || !aligned16(w_uv) || !aligned16(ctx))
            return fail(DSA_ERR_ARG, "pointers must be 16-byte aligned");
        if (test_fail_launch()) return fail(DSA_ERR_LAUNCH, "injected launch failure (DSA_TEST_FAIL_LAUNCH)");
        dsa::AbsorbArgs a{};
        a.n_q = n_q;
        a.o = o;
        a.w_uv = w_uv;
        a.ctx = ctx;
        return launched(dsa::launch_project(a, stream), "project");
    });
}

int dsa_index_prepare(const dsa_geometry *g, const dsa_batch *b, double rope_base, const float *q_in,
                      dsa_bf16 *q_out, int32_t n_new, const int32_t *k_seq, const int32_t *k_pos, const float *k_in,
                      dsa_bf16 *idx_k, int64_t key_seq_stride, hipStream_t stream) {
    return guarded([&] {
        DSA_TRY(check_device());
        DSA_TRY(check_geometry(g));
        if (g->kpool != 1) return fail(DSA_ERR_UNSUPPORTED, "indexer preparation is for kpool 1 only");
        DSA_TRY(check_batch(b));
        if (!(std::isfinite(rope_base) && rope_base > 1.0)) return fail(DSA_ERR_ARG, "rope_base must be finite and > 1");
        if ((q_in == nullptr) != (q_out == nullptr)) return fail(DSA_ERR_ARG, "q_in and q_out go together");
        if (q_in && (!aligned16(q_in) || !aligned16(q_out)))
            return fail(DSA_ERR_ARG, "pointers must be 16-byte aligned");
        if (n_new < 0) return fail(DSA_ERR_ARG, "n_new < 0");
        if (n_new > 0) {
            if (!k_pos || !k_in || !idx_k) return fail(DSA_ERR_ARG, "NULL key pointer");
            if (!k_seq && n_new > b->n_seq) return fail(DSA_ERR_ARG, "k_seq NULL needs n_new <= n_seq");
            if (key_seq_stride < 1) return fail(DSA_ERR_ARG, "key_seq_stride < 1");
            if (!aligned16(k_pos) || !aligned16(k_in) || !aligned16(idx_k) || (k_seq && !aligned16(k_seq)))
                return fail(DSA_ERR_ARG, "pointers must be 16-byte aligned");
        }
        if (test_fail_launch()) return fail(DSA_ERR_LAUNCH, "injected launch failure (DSA_TEST_FAIL_LAUNCH)");
        dsa::PrepArgs a{};
        a.n_q = q_in ? b->n_q : 0;
        a.n_new = n_new;
        a.n_seq = b->n_seq;
        a.rope = g->d_rope == 64 ? 1 : 0;
        a.f16 = g->idx_f16;
        for (int i = 0; i < 8; i++) a.inv_freq[i] = std::pow(rope_base, -4.0 * i / 32.0);
        a.freq_ratio = std::pow(rope_base, -1.0 / 32.0);
        a.q_nvis = b->q_nvis;
        a.q_in = q_in;
        a.q_out = q_out;
        a.k_seq = k_seq;
        a.k_pos = k_pos;
        a.k_in = k_in;
        a.k_cache = idx_k;
        a.key_stride = key_seq_stride;
        return launched(dsa::launch_index_prep(a, stream), "index_prep");
    });
}

}  // extern "C"
