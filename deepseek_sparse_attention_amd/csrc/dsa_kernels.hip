// dsa_kernels.hip -- HIP kernels of the DeepSeek Sparse Attention decode hot
// path for CDNA4 (gfx950, wave64, MFMA 16x16x32 bf16, LDS transpose reads).
//
// Steps and the pages that define them:
//  * indexer scores: "GLM 5.2 in pure C", section "The Lightning Indexer:
//    Sparse Attention When It Helps" (per-head rectified dot product, then a
//    weighted sum over the 32 heads of TensorSharp2's table "The block");
//  * top-k: same section (keep the best index_topk rows; all of them when
//    fewer are visible, TensorSharp2 "The sparse-attention path"); ties go
//    to the lower index ("GLM-5.3-Flash on WASTE", "k-pool flavour");
//  * pools: WASTE "k-pool flavour" and TensorSharp2 "GLM-5.3-Flash
//    (glm5next)": keep top_k/4 pools, expand to tokens, add the unpooled tail;
//  * attention: "GLM 5.2 in pure C", section "Attention: Multi head Latent
//    Attention With a Tiny KV Cache" (absorbed query dotted with the latent
//    and rope parts, scaled, softmax, latents pooled); scale 1/16 from
//    TensorSharp2 "The block".
//
// Design (gfx950): the indexer is a [32 x 128] x [128 x rows] product per
// query on MFMA, key rows staged through LDS with coalesced loads (for a
// prefill chunk, eight consecutive queries share each key tile); its
// epilogue applies ReLU and the head weights and feeds a 4096-bin histogram
// of the scores' order keys.  Top-k is an exact radix select: the histogram
// fixes the threshold bucket, a pass over each chunk copies the rows at or
// above it, in row order, into the chunk's slots, and one work-group per
// query resolves the exact threshold from those candidates and writes the
// kept rows in ascending order.  Attention streams the selected rows into
// LDS by DMA, computes S^T = C Q^T on MFMA, keeps an online softmax in
// fp32, and computes O^T = V^T P^T on MFMA with V read through
// ds_read_b64_tr_b16 and P split into two bf16 halves (hi + lo) so that P
// carries ~16 mantissa bits; split partials are merged by an LSE reduction.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dsa_args.h"

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ---------------------------------------------------------------- helpers
// Order-preserving unsigned image of a float; -0 ranks as +0.
__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}


struct QInfo {
    int32_t seq, nvis, rows, mode;   // mode 0 dense, 1 sparse, 2 invalid
};

__device__ __forceinline__ QInfo query_info(const Args &a, int q) {
    QInfo r;
    r.seq = a.q_seq ? a.q_seq[q] : q;
    r.nvis = a.q_nvis[q];
    if (r.seq < 0 || r.seq >= a.n_seq || r.nvis < 1 || (int64_t)r.nvis > a.max_nvis) {
        r.mode = 2;
        r.rows = 0;
        return r;
    }
    r.rows = r.nvis / a.kpool;
    r.mode = (r.rows <= a.keep) ? 0 : 1;
    return r;
}

constexpr int kPfQ = 8;          // queries per prefill work-group

__device__ __forceinline__ int query_seq(const Args &a, int q) { return a.q_seq ? a.q_seq[q] : q; }

// Prefill blocks: every run of pf_run consecutive queries is covered by
// ceil(pf_run / kPfQ) blocks of up to kPfQ of its queries.  Block blk
// covers queries [first, last); pf_leader(q) is the first query of q's block.
__device__ __forceinline__ int pf_blocks_per_run(const Args &a) { return (a.pf_run + kPfQ - 1) / kPfQ; }
__device__ __forceinline__ int pf_block(const Args &a, int blk, int &last) {
    const int per = pf_blocks_per_run(a);
    const int run = blk / per, j = blk - run * per;
    const int first = run * a.pf_run + j * kPfQ;
    int e = first + kPfQ;
    const int run_end = (run + 1) * a.pf_run;
    e = e < run_end ? e : run_end;
    last = e < a.n_q ? e : a.n_q;
    return first;
}
__device__ __forceinline__ int pf_leader(const Args &a, int q) {
    const int run = q / a.pf_run, off = q - run * a.pf_run;
    return run * a.pf_run + (off / kPfQ) * kPfQ;
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over a wave with DPP: Hillis-Steele shifts inside
// each 16-lane row, then row_bcast:15 / row_bcast:31 carry the row totals.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Exclusive prefix sum over a 256-thread block; smem needs 4 words.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t *smem, uint32_t &total) {
    const uint32_t lane = lane_id(), w = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(v);
    if (lane == 63) smem[w] = x;
    __syncthreads();
    const uint32_t s0 = smem[0], s1 = smem[1], s2 = smem[2], s3 = smem[3];
    __syncthreads();
    total = s0 + s1 + s2 + s3;
    const uint32_t base = (w > 0 ? s0 : 0u) + (w > 1 ? s1 : 0u) + (w > 2 ? s2 : 0u);
    return base + x - v;
}

__device__ uint32_t block_sum(uint32_t v, uint32_t *smem) {
    uint32_t total;
    block_excl_scan(v, smem, total);
    return total;
}

// Radix step: with the counts of NB = 256 PER bins of the items still in
// play and `need` of them still to take from the top, find the bin b
// holding the need-th largest: suffix(b) >= need > suffix(b+1).  Returns b,
// sets above = suffix(b+1) (and *in_bin = the count of bin b).  256
// threads; thread t holds in c the counts of the PER bins just below
// NB - PER*t (c[i]: bin NB - PER t - 1 - i).
template <int PER>
__device__ uint32_t bucket_from_regs(const uint32_t (&c)[PER], uint32_t need, uint32_t *smem, uint32_t *res,
                                     uint32_t &above, uint32_t *in_bin = nullptr) {
    const int hi = 256 * PER - PER * (int)threadIdx.x;
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) s += c[i];
    uint32_t total;
    const uint32_t before = block_excl_scan(s, smem, total);   // items in higher bins
    if (before < need && before + s >= need) {
        uint32_t run = before, bin = 0, run_at = 0, cnt = 0;
        bool found = false;
#pragma unroll
        for (int i = 0; i < PER; i++) {
            if (!found && run + c[i] >= need) {
                found = true;
                bin = (uint32_t)(hi - 1 - i);
                run_at = run;
                cnt = c[i];
            }
            run += c[i];
        }
        res[0] = bin;
        res[1] = run_at;
        res[2] = cnt;
    }
    // fewer than `need` items in all (a histogram that does not match the
    // scores): bin 0, with every item above it counted
    if (threadIdx.x == 255 && before + s < need) {
        res[0] = 0;
        res[1] = before + s - c[PER - 1];
        res[2] = c[PER - 1];
    }
    __syncthreads();
    above = res[1];
    const uint32_t b = res[0];
    if (in_bin) *in_bin = res[2];
    __syncthreads();
    return b;
}

// The same over a histogram hist[0..NB) in memory.
template <int NB>
__device__ uint32_t find_bucket(const uint32_t *hist, uint32_t need, uint32_t *smem, uint32_t *res,
                                uint32_t &above) {
    constexpr int PER = NB / 256;
    const int hi = NB - PER * (int)threadIdx.x;
    uint32_t c[PER];
#pragma unroll
    for (int i = 0; i < PER; i++) c[i] = hist[hi - 1 - i];
    return bucket_from_regs<PER>(c, need, smem, res, above);
}

// Reductions over lanes l and l ^ 16 (l ^ 32) with v_permlane16_swap
// (v_permlane32_swap): with both operands x, the pair returned holds x at l
// and at the partner lane.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float xor16_max(float x) {
    const u32x2 p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
    const u32x2 p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
    const u32x2 p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
    const u32x2 p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// ---------------------------------------------------------------- workspace
__global__ void k_fill_zero(uint32_t *p, size_t n_words) {
    size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n_words; i += stride) p[i] = 0u;
}

// Streaming-read probe: non-temporal 16-byte loads over the whole buffer in
// a grid-stride loop (consecutive threads, consecutive 16 bytes).
__global__ __launch_bounds__(256) void k_stream_read(const u32x4 *p, size_t n, uint32_t *sink) {
    uint32_t x = 0;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const u32x4 t = __builtin_nontemporal_load(p + i);
        x ^= t[0] ^ t[1] ^ t[2] ^ t[3];
    }
    if (x == 0x9e3779b9u) *sink = x;
}

// ---------------------------------------------------------------- scores
// max(x, 0) in one integer max: a float with its sign bit set is a negative
// int32, so every negative x (and -0) becomes +0 and every positive x stays.
// fmaxf on an MFMA result costs a canonicalising max first.  Finite x only.
__device__ __forceinline__ float relu(float x) {
    const int32_t i = __float_as_int(x);
    return __int_as_float(i > 0 ? i : 0);
}

// One 16x16x32 MFMA step of the indexer on 16-bit operands: bf16, or IEEE
// f16 when F16 (the two formats of the indexer queries and key cache).
template <bool F16>
__device__ __forceinline__ f32x4 mfma_idx(bf16x8 a, bf16x8 b, f32x4 c) {
    if constexpr (F16) {
        typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                      c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
}

// grid (tiles, n_q), NW = 4 or 8 waves.  Wave w of a work-group takes
// 64-row steps t0 + 64 (w + NW i).  Keys are read with fully coalesced 16-byte loads
// (one wave instruction = 1 KiB = 4 rows), the next step's 16 KiB already in
// flight in registers while the current one is computed; each step is staged
// in the wave's own LDS tile with the 16-byte pieces of row r stored at
// slot (piece ^ (r & 15)), so that both the row-major store and the MFMA
// operand reads below are free of bank conflicts (the LDS has 64 banks:
// the 16 rows an MFMA operand read takes per 16-lane phase must land their
// pieces in 16 different 16-byte slots).  Per 16 rows:
// A = idx_q (heads x d, two 16-head blocks, from registers), B = keys^T
// (d x rows): lane (g = l/16, n = l%16) takes row n, d in [32 s + 8 g, +8)
// for k-step s.  D[head][row] lands as lane (g, n) holding heads 4g + r
// (+16) of row n; the epilogue applies ReLU and the head weights and sums
// the four lane groups.
template <bool STRIDE, bool F16, int NW>
__global__ __launch_bounds__(64 * NW) void k_score(Args a) {
    constexpr int kGroup = 64 * NW;   // rows of one step of all the work-group's waves
    __shared__ uint32_t lhist[kHistBins];
    __shared__ __attribute__((aligned(16))) uint8_t tiles[NW][64 * 256];
    const int q = blockIdx.y;
    const int lane = lane_id(), w = threadIdx.x >> 6, g = lane >> 4, n = lane & 15;
    u32x4 v[16];
    // With q_seq NULL (query q reads sequence q < n_seq) and one tile per
    // work-group, the wave's first step of keys is requested before the
    // query's fields return.  Rows are clamped below the batch's row bound
    // max_nvis / kpool (<= key_stride): every such row lies in the caller's
    // [n_seq][key_stride] buffer, and rows at or past the query's own are
    // neither scored nor counted.
    const int64_t rmax = a.max_nvis / a.kpool;
    const bool early = !STRIDE && a.q_seq == nullptr && rmax >= 1;
    if (early) {
        const uint8_t *K0 = reinterpret_cast<const uint8_t *>(a.idx_k + (size_t)q * a.key_stride * kIdxDim);
        const int64_t b0 = (a.score_ilv ? kGroup * (int64_t)blockIdx.x : (int64_t)blockIdx.x * a.score_tile) + 64 * w;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            int64_t r = b0 + 4 * i + (lane >> 4);
            r = r < rmax ? r : rmax - 1;
            v[i] = __builtin_nontemporal_load((const u32x4 *)(K0 + r * 256 + 16 * (lane & 15)));
        }
    }
    // a wave leaving without using them waits for its early loads first
    auto drain = [&] {
        if (early) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    const QInfo qi = query_info(a, q);
    if (qi.mode == 2 || (a.fused && qi.mode == 0) ||
        (a.prefill && qi.seq == query_seq(a, pf_leader(a, q)))) {   // the last: done by k_score_prefill
        drain();
        return;
    }
    const int64_t rows = qi.rows;
    const bool ilv = !STRIDE && a.score_ilv;
    if ((int64_t)blockIdx.x * (ilv ? kGroup : a.score_tile) >= rows) {
        drain();
        return;
    }
    const bool hist = a.hist_on != 0;
    if (hist) {
        for (int i = threadIdx.x; i < kHistBins; i += kGroup) lhist[i] = 0;
        __syncthreads();
    }
    // the in-attention top-k: k_filter accumulates the second-digit
    // histogram of the threshold bucket, which must start at zero; the
    // query's first work-group clears it (what the last call left there)
    if (!STRIDE && a.attn_sel && !a.select_scan && blockIdx.x == 0) {
        uint32_t *h2 = a.hist + (size_t)q * kHistStride + kHistH2;
        for (int i = threadIdx.x; i < 1024; i += kGroup) h2[i] = 0;
    }

    bf16x8 qa[2][4];
    float wt[2][4];
    const uint16_t *qip = a.idx_q + (size_t)q * kIdxHeads * kIdxDim;
#pragma unroll
    for (int mb = 0; mb < 2; mb++) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const u32x4 t = *(const u32x4 *)(qip + (16 * mb + n) * kIdxDim + 32 * s + 8 * g);
            qa[mb][s] = __builtin_bit_cast(bf16x8, t);
        }
#pragma unroll
        for (int r = 0; r < 4; r++) wt[mb][r] = a.idx_w[(size_t)q * kIdxHeads + 16 * mb + 4 * g + r];
    }
    const uint8_t *K = reinterpret_cast<const uint8_t *>(a.idx_k + (size_t)qi.seq * a.key_stride * kIdxDim);
    float *srow = a.scores + (size_t)q * a.score_ld;
    const int st_mine = 2 * (g & 1) + (g >> 1);
    uint8_t *tb = tiles[w];
    auto fetch = [&](u32x4 (&vv)[16], int64_t base) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            int64_t r = base + 4 * i + (lane >> 4);
            r = r < rows ? r : rows - 1;
            vv[i] = __builtin_nontemporal_load((const u32x4 *)(K + r * 256 + 16 * (lane & 15)));
        }
    };
    // A step's score is stored at the start of the next step, before that
    // step's key loads: the wait for those loads then leaves no store
    // younger than them outstanding (waits count completions in issue order,
    // so a store issued after them would have to complete too).
    int64_t pend_row = -1;
    float pend = 0.f;
    auto flush = [&] {
        if (pend_row >= 0) srow[pend_row] = pend;
    };
    // one 64-row step from the registers vv: staged in the LDS tile, vv
    // refilled with the wave's next step (row `ahead`), then scored
    auto step = [&](u32x4 (&vv)[16], int64_t base, int64_t ahead, int64_t end) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int r = 4 * i + (lane >> 4), pc = lane & 15;
            *(u32x4 *)(tb + r * 256 + 16 * (pc ^ (r & 15))) = vv[i];
        }
        flush();
        if (ahead < end) fetch(vv, ahead);
        __builtin_amdgcn_wave_barrier();
        float p[4];
#pragma unroll
        for (int st = 0; st < 4; st++) {
            const int r = 16 * st + n;
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; s++) {
                const bf16x8 b = __builtin_bit_cast(bf16x8, *(const u32x4 *)(tb + r * 256 + 16 * ((4 * s + g) ^ (r & 15))));
                acc0 = mfma_idx<F16>(qa[0][s], b, acc0);
                acc1 = mfma_idx<F16>(qa[1][s], b, acc1);
            }
            float x = 0.f;
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
                x += wt[0][rr] * relu(acc0[rr]);
                x += wt[1][rr] * relu(acc1[rr]);
            }
            p[st] = x;
        }
        __builtin_amdgcn_wave_barrier();
        // sum the four lane groups; each lane keeps one of the four 16-row steps
        const bool b0 = g & 1, b1 = (g >> 1) & 1;
        const float send0 = b0 ? p[0] : p[2], send1 = b0 ? p[1] : p[3];
        const float keep0 = b0 ? p[2] : p[0], keep1 = b0 ? p[3] : p[1];
        const float q0 = keep0 + __shfl_xor(send0, 16, 64);
        const float q1 = keep1 + __shfl_xor(send1, 16, 64);
        const float score = (b1 ? q1 : q0) + __shfl_xor(b1 ? q0 : q1, 32, 64);
        const int64_t row = base + 16 * st_mine + n;
        pend_row = row < end ? row : -1;
        pend = score;
        if (row < end && hist) atomicAdd(&lhist[order_key(score) >> 20], 1u);
    };
    // tiles t0 = blockIdx.x * tile, stepping by the grid (one pass in the
    // common case; the prefill fix-up grid has one work-group per query)
    const int64_t wstep = ilv ? kGroup * (int64_t)gridDim.x : kGroup;
    for (int64_t t0 = (int64_t)blockIdx.x * (ilv ? kGroup : a.score_tile); t0 < rows;
         t0 = STRIDE ? t0 + (int64_t)gridDim.x * a.score_tile : rows) {
    const int64_t end = !ilv && t0 + a.score_tile < rows ? t0 + a.score_tile : rows;
    int64_t base = t0 + 64 * w;
    if (early) {
        if (base >= end) drain();              // no step for this wave in a short last tile
    } else if (base < end) {
        fetch(v, base);
    }
    for (; base < end; base += wstep) step(v, base, base + wstep, end);
    }
    flush();
    if (hist) {
        __syncthreads();
        uint32_t *gh = a.hist + (size_t)q * kHistStride;
        for (int i = threadIdx.x; i < kHistBins; i += kGroup)
            if (lhist[i]) atomicAdd(&gh[i], lhist[i]);
    }
}

// The decode scorer on the vector ALU instead of MFMA, kept to measure the
// two against each other (DSA_SCORE_VALU=1): one key row per lane, its 128
// dimensions widened to fp32 in registers, the query's 32 heads of 128 in
// fp32 broadcast from LDS, one v_fma_f32 per product (exact here, as on
// MFMA: the products and their sums are integers below 2^24), then the same
// ReLU, weights, scores and first-digit histogram as k_score.  (The bf16
// pair dot product v_dot2_f32_bf16 does not keep such sums exact.)  bf16
// indexer inputs, decode batches only.  grid (tiles of 256 rows, n_q), 256
// threads.
__global__ __launch_bounds__(256) void k_score_valu(Args a) {
    __shared__ __attribute__((aligned(16))) f32x4 qs[kIdxHeads * kIdxDim / 4];
    __shared__ float wsh[kIdxHeads];
    __shared__ uint32_t lhist[kHistBins];
    const int q = blockIdx.y;
    const QInfo qi = query_info(a, q);
    if (qi.mode == 2 || (a.fused && qi.mode == 0)) return;
    const int64_t rows = qi.rows;
    if ((int64_t)blockIdx.x * 256 >= rows) return;
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool hist = a.hist_on != 0;
    const uint32_t *qg = reinterpret_cast<const uint32_t *>(a.idx_q + (size_t)q * kIdxHeads * kIdxDim);
    for (int i = threadIdx.x; i < kIdxHeads * kIdxDim / 4; i += 256) {
        const uint32_t x0 = qg[2 * i], x1 = qg[2 * i + 1];   // bf16 pairs -> fp32 (exact)
        qs[i] = f32x4{__uint_as_float(x0 << 16), __uint_as_float(x0 & 0xFFFF0000u), __uint_as_float(x1 << 16),
                      __uint_as_float(x1 & 0xFFFF0000u)};
    }
    if (threadIdx.x < kIdxHeads) wsh[threadIdx.x] = a.idx_w[(size_t)q * kIdxHeads + threadIdx.x];
    if (hist)
        for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0;
    if (a.attn_sel && !a.select_scan && blockIdx.x == 0) {
        uint32_t *h2 = a.hist + (size_t)q * kHistStride + kHistH2;
        for (int i = threadIdx.x; i < 1024; i += 256) h2[i] = 0;
    }
    u32x4 kv[16];
    const int64_t rr = r < rows ? r : rows - 1;
    const u32x4 *kg = reinterpret_cast<const u32x4 *>(a.idx_k + ((size_t)qi.seq * a.key_stride + rr) * kIdxDim);
#pragma unroll
    for (int j = 0; j < 16; j++) kv[j] = kg[j];
    float kf[kIdxDim];
#pragma unroll
    for (int j = 0; j < 16; j++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            kf[8 * j + 2 * e] = __uint_as_float(kv[j][e] << 16);
            kf[8 * j + 2 * e + 1] = __uint_as_float(kv[j][e] & 0xFFFF0000u);
        }
    __syncthreads();
    float score = 0.f;
#pragma unroll 1
    for (int h = 0; h < kIdxHeads; h++) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < kIdxDim / 4; j++) {
            const f32x4 qv = qs[h * (kIdxDim / 4) + j];
            acc = __builtin_fmaf(kf[4 * j], qv[0], acc);
            acc = __builtin_fmaf(kf[4 * j + 1], qv[1], acc);
            acc = __builtin_fmaf(kf[4 * j + 2], qv[2], acc);
            acc = __builtin_fmaf(kf[4 * j + 3], qv[3], acc);
        }
        score += wsh[h] * relu(acc);
    }
    if (r < rows) {
        a.scores[(size_t)q * a.score_ld + r] = score;
        if (hist) atomicAdd(&lhist[order_key(score) >> 20], 1u);
    }
    if (hist) {
        __syncthreads();
        uint32_t *gh = a.hist + (size_t)q * kHistStride;
        for (int i = threadIdx.x; i < kHistBins; i += 256)
            if (lhist[i]) atomicAdd(&gh[i], lhist[i]);
    }
}

// Chunked-prefill / verify-window indexer: a dense [queries x 32 heads] x
// [128 x keys] contraction per work-group.  grid (key ranges, blocks), 1024
// threads = 16 waves (4 per SIMD: the LDS of one work-group fills the CU, so
// latency is hidden inside it).  A block holds up to 8 consecutive queries of
// one run (pf_block); they are positions of one sequence (the leader's), and
// a query of another sequence is left to the fix-up pass of k_score.  Key
// tiles of 128 rows are loaded with coalesced 16-byte loads (1024 threads x
// 2 = 32 KiB), staged swizzled in LDS (double buffer) and shared by the
// block's queries.  With P = the block's query count rounded up to a power
// of two, wave w computes query w * P / 16 on 16-row blocks [NB s, NB s + NB)
// of each tile, NB = max(1, P / 2) and s = w % (16 / P): every wave has work
// however few queries the block holds, except half of them for a lone query.  Causality masks the scores and the histogram
// per query (a query scores rows < rows(q)).  Per-query first-digit
// histograms live in LDS as 16-bit counters, two to a word (bins i and
// i + 2048).
constexpr int kPfTile = 128;     // key rows per LDS tile
constexpr int kPfRange = 4096;   // key rows per work-group
constexpr int kPfWaves = 16;     // waves per work-group (two per query of a full block)

template <bool F16>
__global__ __launch_bounds__(kPfWaves * 64) void k_score_prefill(Args a) {
    __shared__ __attribute__((aligned(16))) uint8_t ktile[2][kPfTile * 256];
    __shared__ uint32_t lh[kPfQ][kHistBins / 2];
    __shared__ int32_t sh_rows[kPfQ];
    const int w = threadIdx.x >> 6, lane = lane_id(), g = lane >> 4, n = lane & 15;
    int q_end;
    const int q0 = pf_block(a, blockIdx.y, q_end);
    if (q0 >= q_end) return;                 // past the last query
    const int nq = q_end - q0;
    const int P = nq > 4 ? 8 : (nq > 2 ? 4 : nq);
    const int slot = w * P / kPfWaves;       // this wave's query within the block
    const int sl = w % (kPfWaves / P);       // and its share of each tile
    const int q = q0 + slot;
    const int lead = query_seq(a, q0);
    const bool hist = a.hist_on != 0;
    // does each query slot take part, and up to which row
    if (threadIdx.x < kPfQ) {
        int32_t rr = 0;
        const int qs = q0 + (int)threadIdx.x;
        if (qs < q_end) {
            const QInfo qi = query_info(a, qs);
            const bool part = qi.mode != 2 && !(a.fused && qi.mode == 0) && qi.seq == lead;
            rr = part ? qi.rows : 0;
        }
        sh_rows[threadIdx.x] = rr;
    }
    __syncthreads();
    int32_t kmax = 0;
#pragma unroll
    for (int i = 0; i < kPfQ; i++) kmax = sh_rows[i] > kmax ? sh_rows[i] : kmax;
    const int64_t k0 = (int64_t)blockIdx.x * kPfRange;
    if (k0 >= kmax) return;
    const int64_t k1 = k0 + kPfRange < kmax ? k0 + kPfRange : kmax;
    const int32_t my_rows = sh_rows[slot];
    if (hist)
        for (int i = threadIdx.x; i < kPfQ * kHistBins / 2; i += kPfWaves * 64) (&lh[0][0])[i] = 0;

    bf16x8 qa[2][4];
    float wt[2][4];
    const int qv = slot < nq ? q : q0;       // a valid query for the idle slots (no rows)
    {
        const uint16_t *qip = a.idx_q + (size_t)qv * kIdxHeads * kIdxDim;
#pragma unroll
        for (int mb = 0; mb < 2; mb++) {
#pragma unroll
            for (int s = 0; s < 4; s++)
                qa[mb][s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qip + (16 * mb + n) * kIdxDim + 32 * s + 8 * g));
#pragma unroll
            for (int r = 0; r < 4; r++) wt[mb][r] = a.idx_w[(size_t)qv * kIdxHeads + 16 * mb + 4 * g + r];
        }
    }
    const uint8_t *K = reinterpret_cast<const uint8_t *>(a.idx_k + (size_t)lead * a.key_stride * kIdxDim);
    float *srow = a.scores + (size_t)qv * a.score_ld;
    const int st_mine = 2 * (g & 1) + (g >> 1);

    constexpr int kPieces = kPfTile * 16 / (kPfWaves * 64);   // 16-byte pieces per thread
    u32x4 v[kPieces];
    auto fetch = [&](int64_t base) {
#pragma unroll
        for (int i = 0; i < kPieces; i++) {
            const int e = threadIdx.x + kPfWaves * 64 * i;   // 16-byte piece of the tile
            int64_t r = base + (e >> 4);
            r = r < kmax ? r : kmax - 1;
            v[i] = __builtin_nontemporal_load((const u32x4 *)(K + r * 256 + 16 * (e & 15)));
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kPieces; i++) {
            const int e = threadIdx.x + kPfWaves * 64 * i;
            const int r = e >> 4, pc = e & 15;
            *(u32x4 *)(&ktile[buf][r * 256 + 16 * (pc ^ (r & 15))]) = v[i];
        }
    };
    // partial score of 16-row block rb of the tile: lane (g, n) holds row n's
    // heads 4g..4g+3 and 16+4g..16+4g+3, weighted and rectified
    auto block_part = [&](const uint8_t *tb, int rb) -> float {
        const int r = 16 * rb + n;
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const bf16x8 bv = __builtin_bit_cast(bf16x8, *(const u32x4 *)(tb + r * 256 + 16 * ((4 * s + g) ^ (r & 15))));
            acc0 = mfma_idx<F16>(qa[0][s], bv, acc0);
            acc1 = mfma_idx<F16>(qa[1][s], bv, acc1);
        }
        float x = 0.f;
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
            x += wt[0][rr] * relu(acc0[rr]);
            x += wt[1][rr] * relu(acc1[rr]);
        }
        return x;
    };
    auto emit = [&](int64_t row, float score) {
        if (row < my_rows) {
            srow[row] = score;
            if (hist) {
                // word i holds bins i and i + 2048 (the order key's top bit:
                // negative and positive scores), so that neighbouring bins,
                // where a query's scores crowd, are different words and a
                // wave's adds to them do not serialise on one address
                const uint32_t bin = order_key(score) >> 20;
                atomicAdd(&lh[slot][bin & (kHistBins / 2 - 1)], 1u << (16 * (bin / (kHistBins / 2))));
            }
        }
    };
    auto tiles = [&](auto nb_tag) {
        constexpr int NB = decltype(nb_tag)::value;
        fetch(k0);
        int buf = 0;
        for (int64_t base = k0; base < k1; base += kPfTile, buf ^= 1) {
            stage(buf);
            if (base + kPfTile < k1) fetch(base + kPfTile);
            __syncthreads();
            const uint8_t *tb = ktile[buf];
            if (NB >= 4) {
                // groups of four blocks: the four lane groups end up holding
                // one block's full score each
#pragma unroll
                for (int j = 0; j < NB / 4; j++) {
                    const int rb0 = NB * sl + 4 * j;
                    float p[4];
#pragma unroll
                    for (int st = 0; st < 4; st++) p[st] = block_part(tb, rb0 + st);
                    const bool b0 = g & 1, b1 = (g >> 1) & 1;
                    const float send0 = b0 ? p[0] : p[2], send1 = b0 ? p[1] : p[3];
                    const float keep0 = b0 ? p[2] : p[0], keep1 = b0 ? p[3] : p[1];
                    const float q0s = keep0 + __shfl_xor(send0, 16, 64);
                    const float q1s = keep1 + __shfl_xor(send1, 16, 64);
                    const float score = (b1 ? q1s : q0s) + __shfl_xor(b1 ? q0s : q1s, 32, 64);
                    emit(base + 16 * (rb0 + st_mine) + n, score);
                }
            } else {
                // one or two blocks: full sum over the lane groups, written
                // by lane group 0 (a lone query leaves half the waves idle)
#pragma unroll
                for (int j = 0; j < NB; j++) {
                    const int rb = NB * sl + j;
                    if (rb >= kPfTile / 16) break;
                    const float score = xor32_sum(xor16_sum(block_part(tb, rb)));
                    if (g == 0) emit(base + 16 * rb + n, score);
                }
            }
            __syncthreads();                              // buffer free for the tile after next
        }
    };
    // 16-row blocks per wave: the tile's 8 blocks shared by each query's
    // kPfWaves / P waves
    if (P == 8)
        tiles(std::integral_constant<int, 4>());
    else if (P == 4)
        tiles(std::integral_constant<int, 2>());
    else
        tiles(std::integral_constant<int, 1>());
    if (hist) {
        __syncthreads();
        for (int i = threadIdx.x; i < kPfQ * kHistBins / 2; i += kPfWaves * 64) {
            const int qq = q0 + i / (kHistBins / 2);
            const uint32_t word = (&lh[0][0])[i];
            if (!word || qq >= q_end) continue;
            const int bin = i % (kHistBins / 2);
            uint32_t *gh = a.hist + (size_t)qq * kHistStride + bin;
            if (word & 0xFFFFu) atomicAdd(gh, word & 0xFFFFu);
            if (word >> 16) atomicAdd(gh + kHistBins / 2, word >> 16);
        }
    }
}

// Histogram of caller-provided scores (the standalone top-k entry point).
// grid (n_chunks, n_q), 256 threads.
__global__ __launch_bounds__(256) void k_hist(Args a) {
    __shared__ uint32_t lhist[kHistBins];
    const int q = blockIdx.y, c = blockIdx.x;
    const QInfo qi = query_info(a, q);
    if (qi.mode != 1) return;
    const int64_t r0 = (int64_t)c * a.chunk;
    if (r0 >= qi.rows) return;
    const int64_t r1 = r0 + a.chunk < qi.rows ? r0 + a.chunk : qi.rows;
    for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0;
    __syncthreads();
    const float *s = a.scores_in + (size_t)q * a.score_ld;
    for (int64_t r = r0 + threadIdx.x; r < r1; r += 256) atomicAdd(&lhist[order_key(s[r]) >> 20], 1u);
    __syncthreads();
    uint32_t *gh = a.hist + (size_t)q * kHistStride;
    for (int i = threadIdx.x; i < kHistBins; i += 256)
        if (lhist[i]) atomicAdd(&gh[i], lhist[i]);
}

// ---------------------------------------------------------------- top-k
// Exact radix select over 32-bit order keys, ranked by (key descending,
// row ascending), three digits: d1 = bits 31..20 (4096-bin histogram from
// the score kernel or k_hist), d2 = bits 19..10, d3 = bits 9..0.
//   k_filter (grid chunks x queries): from the first-digit histogram find
//     the bucket b1 holding the keep-th row; copy every row of the chunk
//     whose d1 is at least b1 as (key, row) into the chunk's own candidate
//     slots, in row order, and record how many there were.
//   k_select (one work-group per query): gathers the candidates of all
//     chunks into LDS in row order (re-reading the scores of a chunk whose
//     slots overflowed), resolves d2 and d3 of the threshold there, and
//     writes the kept rows in ascending order, expanded for pools, then the
//     unpooled tail and -1 padding.  If the candidates do not fit in LDS it
//     makes the same decisions from passes over the scores.  It also zeroes
//     the query's histogram, the only state that must be zero between calls.
// No global atomics: chunks own their candidate slots.

// n scores from s[r0..r0+n) (rows at or past r1 read as 0); 16-byte loads
// when the run is aligned and whole.
template <int N>
__device__ __forceinline__ void load_scores(const float *s, int64_t r0, int64_t r1, bool vec, float (&v)[N]) {
    if (vec && r0 + N <= r1) {
#pragma unroll
        for (int j = 0; j < N / 4; j++) {
            const f32x4 t = *(const f32x4 *)(s + r0 + 4 * j);
            v[4 * j] = t[0];
            v[4 * j + 1] = t[1];
            v[4 * j + 2] = t[2];
            v[4 * j + 3] = t[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; i++) v[i] = r0 + i < r1 ? s[r0 + i] : 0.f;
    }
}

// grid (n_chunks, n_q), 256 threads; thread t takes rows sb + PER t ..
// + PER - 1 of each 256 PER-row block, so the block-ordered compaction keeps
// row order.  PER = 16 for chunks of several such blocks (a prefill chunk:
// 60 vs 64 us), 8 for short ones (a 2,048-row chunk: 5.0 vs 6.0 us).
template <int kFiltPer>
__global__ __launch_bounds__(256) void k_filter(Args a) {
    constexpr int kFiltBlock = 256 * kFiltPer;
    __shared__ uint32_t scan[8];
    __shared__ uint32_t res[4];
    const int q = blockIdx.y, c = blockIdx.x;
    // The query's first-digit histogram (thread t: bins 4095 - 16 t - i,
    // four 16-byte loads) and the chunk's first block of scores are
    // requested before the query's fields return: one round trip, not two.
    // The block is read up to the score row's length (score_ld entries);
    // rows at or past the query's own are not used.
    const float *s = a.scores_in + (size_t)q * a.score_ld;
    const bool vec = (reinterpret_cast<uintptr_t>(s) & 15) == 0;
    const int64_t r0 = (int64_t)c * a.chunk;
    float sv[kFiltPer];
    load_scores<kFiltPer>(s, r0 + kFiltPer * threadIdx.x, r0 + a.chunk < a.score_ld ? r0 + a.chunk : a.score_ld, vec,
                          sv);
    u32x4 hv[4];
    {
        const uint32_t *gh = a.hist + (size_t)q * kHistStride + (kHistBins - 16 * (threadIdx.x + 1));
#pragma unroll
        for (int j = 0; j < 4; j++) hv[j] = *(const u32x4 *)(gh + 4 * j);
    }
    // a wave leaving without using them waits for those loads first
    auto drain = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
    const QInfo qi = query_info(a, q);
    if (qi.mode != 1) {
        drain();
        return;
    }
    const int64_t rows = qi.rows;
    const int nch = (int)((rows + a.chunk - 1) / a.chunk);
    if (c >= nch) {
        drain();
        return;
    }
    const int64_t r1 = r0 + a.chunk < rows ? r0 + a.chunk : rows;
    uint32_t hc[16];   // hc[i]: bin 4095 - 16 t - i
#pragma unroll
    for (int i = 0; i < 16; i++) hc[i] = hv[(15 - i) >> 2][(15 - i) & 3];
    uint32_t above1;
    const uint32_t b1 = bucket_from_regs<16>(hc, (uint32_t)a.keep, scan, res, above1);
    if (c == 0 && threadIdx.x == 0) {
        a.thr[2 * q] = b1;
        a.thr[2 * q + 1] = above1;
    }

    uint64_t *slots = a.cand + ((size_t)q * a.n_chunks + c) * a.cand_cap;
    uint32_t *h2 = a.attn_sel ? a.hist + (size_t)q * kHistStride + kHistH2 : nullptr;
    uint32_t n_cand = 0;
    for (int64_t sb = r0; sb < r1; sb += kFiltBlock) {
        const int64_t rb = sb + kFiltPer * threadIdx.x;
        // the next block's scores in flight while this one is filtered
        float sn[kFiltPer];
        if (sb + kFiltBlock < r1) {
            load_scores<kFiltPer>(s, rb + kFiltBlock, r1, vec, sn);
        } else {
#pragma unroll
            for (int i = 0; i < kFiltPer; i++) sn[i] = 0.f;
        }
        uint32_t keys[kFiltPer];
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < kFiltPer; i++) {
            keys[i] = order_key(sv[i]);
            if (rb + i < r1 && (keys[i] >> 20) >= b1) m |= 1u << i;
        }
        uint32_t tot;
        uint32_t pos = n_cand + block_excl_scan(__builtin_popcount(m), scan, tot);
        n_cand += tot;
#pragma unroll
        for (int i = 0; i < kFiltPer; i++) {
            if (!((m >> i) & 1)) continue;
            if (pos < (uint32_t)a.cand_cap) slots[pos] = ((uint64_t)keys[i] << 32) | (uint32_t)(rb + i);
            pos++;
            // the in-attention selection takes the second digit of the
            // threshold bucket's rows from this histogram
            if (h2 && (keys[i] >> 20) == b1) atomicAdd(&h2[(keys[i] >> 10) & 1023], 1u);
        }
#pragma unroll
        for (int i = 0; i < kFiltPer; i++) sv[i] = sn[i];
    }
    if (threadIdx.x == 0) a.chunk_cnt[(size_t)q * a.n_chunks + c] = n_cand;
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelPer = 16;                       // rows per thread per pass tile
constexpr int kSelTile = kSelThreads * kSelPer;
constexpr int kSelCap = 12288;                    // candidates k_select keeps in LDS

struct SelectShared {
    uint32_t key[kSelCap];
    int32_t row[kSelCap];
    uint32_t pre[kMaxChunks + 1];  // exclusive prefix of the chunks' candidate counts
    uint32_t h2[1024];
    uint32_t h3[1024];
    uint32_t tot[2][kSelWaves];
    uint32_t res[3];
};

// Exclusive prefix sum over the 1024 threads with one barrier; the 16-word
// slot may be written again only after another barrier.
__device__ __forceinline__ uint32_t sel_scan(uint32_t v, uint32_t *slot, uint32_t &total) {
    const uint32_t lane = lane_id(), w = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(v);
    if (lane == 63) slot[w] = x;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; i++) {
        const uint32_t t = slot[i];
        before += i < (int)w ? t : 0u;
        tot += t;
    }
    total = tot;
    return before + x - v;
}

// Radix step over 1024 * PER bins; thread t holds the counts of bins
// hi - 1 - i, hi = 1024 * PER - PER * t.  Finds the bin b with
// suffix(b) >= need > suffix(b + 1); above = suffix(b + 1).
template <int PER>
__device__ uint32_t sel_find(const uint32_t (&c)[PER], uint32_t need, uint32_t *slot, uint32_t *res,
                             uint32_t &above, uint32_t *in_bin = nullptr) {
    const int hi = kSelThreads * PER - PER * (int)threadIdx.x;
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) s += c[i];
    uint32_t total;
    const uint32_t before = sel_scan(s, slot, total);
    if (before < need && before + s >= need) {
        uint32_t run = before, bin = 0, run_at = 0, cnt = 0;
        bool found = false;
#pragma unroll
        for (int i = 0; i < PER; i++) {
            if (!found && run + c[i] >= need) {
                found = true;
                bin = (uint32_t)(hi - 1 - i);
                run_at = run;
                cnt = c[i];
            }
            run += c[i];
        }
        res[0] = bin;
        res[1] = run_at;
        res[2] = cnt;
    }
    if (threadIdx.x == kSelThreads - 1 && before + s < need) {   // as bucket_from_regs
        res[0] = 0;
        res[1] = before + s - c[PER - 1];
        res[2] = c[PER - 1];
    }
    __syncthreads();
    above = res[1];
    const uint32_t b = res[0];
    if (in_bin) *in_bin = res[2];
    __syncthreads();
    return b;
}

// grid (n_q), 1024 threads.  SCAN: the work-group finds the threshold
// bucket from the first-digit histogram itself and gathers the candidates
// by scanning the query's scores (no k_filter); otherwise k_filter's chunk
// slots are gathered.
template <bool SCAN>
__global__ __launch_bounds__(kSelThreads) void k_select(Args a) {
    __shared__ SelectShared sh;
    const int q = blockIdx.x, tid = threadIdx.x;
    const QInfo qi = query_info(a, q);
    int32_t *dst = a.sel + (size_t)q * a.sel_ld;
    // SCAN: thread t holds the first-digit counts of bins 4095 - 4t - i,
    // read before it clears them
    uint32_t c1[kHistBins / kSelThreads];
    {
        uint32_t *gh = a.hist + (size_t)q * kHistStride;
        if (SCAN) {
#pragma unroll
            for (int i = 0; i < kHistBins / kSelThreads; i++) c1[i] = gh[kHistBins - 1 - 4 * tid - i];
#pragma unroll
            for (int i = 0; i < kHistBins / kSelThreads; i++) gh[kHistBins - 1 - 4 * tid - i] = 0;
        } else {
            for (int i = tid; i < kHistBins; i += kSelThreads) gh[i] = 0;
        }
    }
    if (qi.mode != 1) {
        const int32_t cnt = qi.mode == 0 ? qi.nvis : 0;
        for (int i = tid; i < a.sel_ld; i += kSelThreads) dst[i] = i < cnt ? i : -1;
        if (tid == 0) a.sel_count[q] = cnt;
        return;
    }
    const int kp = a.kpool;
    const uint32_t keep = (uint32_t)a.keep;
    const int64_t rows = qi.rows;
    const float *s = a.scores_in + (size_t)q * a.score_ld;
    const bool vec = (reinterpret_cast<uintptr_t>(s) & 15) == 0;
    int par = 0;                                    // alternates the scan slots

    for (int i = tid; i < 1024; i += kSelThreads) {
        sh.h2[i] = 0;
        sh.h3[i] = 0;
    }
    uint32_t b1, above1, n_cand;
    bool in_lds;
    if (SCAN) {
        // the first tile of scores in flight while the bucket is found
        float v[kSelPer];
        load_scores<kSelPer>(s, kSelPer * tid, rows, vec, v);
        uint32_t in_b1;
        b1 = sel_find<kHistBins / kSelThreads>(c1, keep, sh.tot[par++ & 1], sh.res, above1, &in_b1);
        n_cand = above1 + in_b1;
        in_lds = n_cand <= (uint32_t)kSelCap;
        if (in_lds) {
            // every row whose first digit is at least b1, in row order, with
            // the second-digit histogram of bucket b1 on the way
            uint32_t base = 0;
            for (int64_t sb = 0; sb < rows; sb += kSelTile) {
                const int64_t rb = sb + kSelPer * tid;
                float vn[kSelPer];
                if (sb + kSelTile < rows) load_scores<kSelPer>(s, rb + kSelTile, rows, vec, vn);
                uint32_t keys[kSelPer];
                uint32_t m = 0;
#pragma unroll
                for (int i = 0; i < kSelPer; i++) {
                    keys[i] = order_key(v[i]);
                    const uint32_t d1 = keys[i] >> 20;
                    if (rb + i < rows && d1 >= b1) {
                        m |= 1u << i;
                        if (d1 == b1) atomicAdd(&sh.h2[(keys[i] >> 10) & 1023], 1u);
                    }
                }
                uint32_t tot;
                uint32_t pos = base + sel_scan(__builtin_popcount(m), sh.tot[par++ & 1], tot);
                base += tot;
#pragma unroll
                for (int i = 0; i < kSelPer; i++) {
                    if (!((m >> i) & 1)) continue;
                    if (pos < (uint32_t)kSelCap) {
                        sh.key[pos] = keys[i];
                        sh.row[pos] = (int32_t)(rb + i);
                    }
                    pos++;
                }
#pragma unroll
                for (int i = 0; i < kSelPer; i++) v[i] = vn[i];
            }
        } else {
            for (int64_t sb = 0; sb < rows; sb += kSelTile) {
                const int64_t rb = sb + kSelPer * tid;
                float w[kSelPer];
                load_scores<kSelPer>(s, rb, rows, vec, w);
#pragma unroll
                for (int i = 0; i < kSelPer; i++) {
                    const uint32_t k = order_key(w[i]);
                    if (rb + i < rows && (k >> 20) == b1) atomicAdd(&sh.h2[(k >> 10) & 1023], 1u);
                }
            }
        }
        __syncthreads();
    } else {
    b1 = a.thr[2 * q];
    above1 = a.thr[2 * q + 1];
    const int nch = (int)((rows + a.chunk - 1) / a.chunk);
    // candidate counts per chunk -> row-ordered offsets
    const uint32_t *cc = a.chunk_cnt + (size_t)q * a.n_chunks;
    const uint32_t my_cnt = tid < nch ? cc[tid] : 0u;
    const uint32_t my_pre = sel_scan(my_cnt, sh.tot[par++ & 1], n_cand);
    const bool any_ovf = __syncthreads_or(my_cnt > (uint32_t)a.cand_cap) != 0;
    if (tid < nch) sh.pre[tid] = my_pre;
    if (tid == 0) sh.pre[nch] = n_cand;
    in_lds = n_cand <= (uint32_t)kSelCap;
    __syncthreads();

    if (in_lds) {
        // candidates of chunks whose slots held them all: wave w copies
        // chunks w, w + 16, ..., four at a time, 128 candidates of each per
        // round, every load issued before the stores
        {
            const int w = tid >> 6, lane = tid & 63;
            for (int c0 = w; c0 < nch; c0 += 4 * kSelWaves) {
                uint32_t cnt[4], base[4], mx = 0;
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    const int c = c0 + k * kSelWaves;
                    cnt[k] = 0;
                    base[k] = 0;
                    if (c < nch) {
                        base[k] = sh.pre[c];
                        cnt[k] = sh.pre[c + 1] - base[k];
                        if (cnt[k] > (uint32_t)a.cand_cap) cnt[k] = 0;   // re-scanned below
                    }
                    mx = cnt[k] > mx ? cnt[k] : mx;
                }
                for (uint32_t j0 = 0; j0 < mx; j0 += 128) {
                    uint64_t v[4][2];
#pragma unroll
                    for (int k = 0; k < 4; k++)
#pragma unroll
                        for (int h = 0; h < 2; h++) {
                            const uint32_t jj = j0 + 64 * h + lane;
                            v[k][h] = jj < cnt[k]
                                          ? a.cand[((size_t)q * a.n_chunks + c0 + k * kSelWaves) * a.cand_cap + jj]
                                          : 0ull;
                        }
#pragma unroll
                    for (int k = 0; k < 4; k++)
#pragma unroll
                        for (int h = 0; h < 2; h++) {
                            const uint32_t jj = j0 + 64 * h + lane;
                            if (jj < cnt[k]) {
                                sh.key[base[k] + jj] = (uint32_t)(v[k][h] >> 32);
                                sh.row[base[k] + jj] = (int32_t)(uint32_t)v[k][h];
                            }
                        }
                }
            }
        }
        // chunks whose slots overflowed: compact their rows again
        for (int c = 0; any_ovf && c < nch; c++) {
            const uint32_t cnt = sh.pre[c + 1] - sh.pre[c];
            if (cnt <= (uint32_t)a.cand_cap) continue;
            const int64_t r0 = (int64_t)c * a.chunk;
            const int64_t r1 = r0 + a.chunk < rows ? r0 + a.chunk : rows;
            uint32_t base = sh.pre[c];
            for (int64_t sb = r0; sb < r1; sb += kSelTile) {
                const int64_t rb = sb + kSelPer * tid;
                float v[kSelPer];
                load_scores<kSelPer>(s, rb, r1, vec, v);
                uint32_t keys[kSelPer];
                uint32_t m = 0;
#pragma unroll
                for (int i = 0; i < kSelPer; i++) {
                    keys[i] = order_key(v[i]);
                    if (rb + i < r1 && (keys[i] >> 20) >= b1) m |= 1u << i;
                }
                uint32_t tot;
                uint32_t pos = base + sel_scan(__builtin_popcount(m), sh.tot[par++ & 1], tot);
                base += tot;
#pragma unroll
                for (int i = 0; i < kSelPer; i++) {
                    if (!((m >> i) & 1)) continue;
                    if (pos < sh.pre[c + 1]) {
                        sh.key[pos] = keys[i];
                        sh.row[pos] = (int32_t)(rb + i);
                    }
                    pos++;
                }
            }
        }
        __syncthreads();
        for (uint32_t i = tid; i < n_cand; i += kSelThreads) {
            const uint32_t k = sh.key[i];
            if ((k >> 20) == b1) atomicAdd(&sh.h2[(k >> 10) & 1023], 1u);
        }
    } else {
        for (int64_t sb = 0; sb < rows; sb += kSelTile) {
            const int64_t rb = sb + kSelPer * tid;
            float v[kSelPer];
            load_scores<kSelPer>(s, rb, rows, vec, v);
#pragma unroll
            for (int i = 0; i < kSelPer; i++) {
                const uint32_t k = order_key(v[i]);
                if (rb + i < rows && (k >> 20) == b1) atomicAdd(&sh.h2[(k >> 10) & 1023], 1u);
            }
        }
    }
    __syncthreads();
    }

    // second digit
    const uint32_t need2 = keep - above1;
    uint32_t c2[1] = {sh.h2[1023 - tid]};
    uint32_t above2;
    const uint32_t b2 = sel_find<1>(c2, need2, sh.tot[par++ & 1], sh.res, above2);
    const uint32_t pre2 = (b1 << 10) | b2;
    const uint32_t need3 = need2 - above2;
    // third digit
    if (in_lds) {
        for (uint32_t i = tid; i < n_cand; i += kSelThreads) {
            const uint32_t k = sh.key[i];
            if ((k >> 10) == pre2) atomicAdd(&sh.h3[k & 1023], 1u);
        }
    } else {
        for (int64_t sb = 0; sb < rows; sb += kSelTile) {
            const int64_t rb = sb + kSelPer * tid;
            float v[kSelPer];
            load_scores<kSelPer>(s, rb, rows, vec, v);
#pragma unroll
            for (int i = 0; i < kSelPer; i++) {
                const uint32_t k = order_key(v[i]);
                if (rb + i < rows && (k >> 10) == pre2) atomicAdd(&sh.h3[k & 1023], 1u);
            }
        }
    }
    __syncthreads();
    uint32_t c3[1] = {sh.h3[1023 - tid]};
    uint32_t above3;
    const uint32_t b3 = sel_find<1>(c3, need3, sh.tot[par++ & 1], sh.res, above3);
    const uint32_t thr = (pre2 << 10) | b3;
    const uint32_t m_eq = need3 - above3;          // rows equal to thr kept, lowest rows first

    auto put = [&](uint32_t pos, int32_t r) {
        if (pos >= keep) return;                    // never past the kept rows
        if (kp == 1) {
            dst[pos] = r;
        } else {
            for (int j = 0; j < kp; j++) dst[(size_t)pos * kp + j] = r * kp + j;
        }
    };
    if (in_lds) {
        // thread t takes candidates [per t, per (t + 1)), in row order
        constexpr int kG = kSelCap / kSelThreads;
        const uint32_t per = (n_cand + kSelThreads - 1) / kSelThreads;
        const uint32_t i0 = per * tid;
        uint32_t kk[kG];
        int32_t rr[kG];
        uint32_t n_eq = 0;
#pragma unroll
        for (int u = 0; u < kG; u++) {
            const uint32_t i = i0 + u;
            const bool ok = u < (int)per && i < n_cand;
            kk[u] = ok ? sh.key[i] : 0u;
            rr[u] = ok ? sh.row[i] : -1;
            if (!ok) kk[u] = 0u;
            n_eq += (ok && kk[u] == thr) ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t eq0 = sel_scan(n_eq, sh.tot[par++ & 1], tot);
        uint32_t take = 0, r = eq0;
#pragma unroll
        for (int u = 0; u < kG; u++) {
            const bool ok = rr[u] >= 0;
            const bool eq = ok && kk[u] == thr;
            if (ok && (kk[u] > thr || (eq && r < m_eq))) take |= 1u << u;
            r += eq ? 1u : 0u;
        }
        uint32_t pos = sel_scan(__builtin_popcount(take), sh.tot[par++ & 1], tot);
#pragma unroll
        for (int u = 0; u < kG; u++)
            if ((take >> u) & 1) put(pos++, rr[u]);
    } else {
        uint32_t eq_done = 0, out_done = 0;
        for (int64_t sb = 0; sb < rows; sb += kSelTile) {
            const int64_t rb = sb + kSelPer * tid;
            float v[kSelPer];
            load_scores<kSelPer>(s, rb, rows, vec, v);
            uint32_t gtm = 0, eqm = 0;
#pragma unroll
            for (int i = 0; i < kSelPer; i++) {
                const uint32_t k = order_key(v[i]);
                if (rb + i < rows) {
                    gtm |= (k > thr ? 1u : 0u) << i;
                    eqm |= (k == thr ? 1u : 0u) << i;
                }
            }
            uint32_t tot;
            uint32_t r = eq_done + sel_scan(__builtin_popcount(eqm), sh.tot[par++ & 1], tot);
            eq_done += tot;
            uint32_t take = gtm;
#pragma unroll
            for (int i = 0; i < kSelPer; i++) {
                if ((eqm >> i) & 1) {
                    if (r < m_eq) take |= 1u << i;
                    r++;
                }
            }
            uint32_t pos = out_done + sel_scan(__builtin_popcount(take), sh.tot[par++ & 1], tot);
            out_done += tot;
#pragma unroll
            for (int i = 0; i < kSelPer; i++)
                if ((take >> i) & 1) put(pos++, (int32_t)(rb + i));
        }
    }
    // the unpooled tail, then padding
    const int32_t pooled = a.keep * kp;
    const int32_t tail = qi.nvis - (int32_t)rows * kp;
    for (int i = tid; i < a.sel_ld - pooled; i += kSelThreads) dst[pooled + i] = i < tail ? (int32_t)rows * kp + i : -1;
    if (tid == 0) a.sel_count[q] = pooled + tail;
}

// ---------------------------------------------------------------- attention
// One work-group = (query q, split sp), all 64 heads, 512 threads = 8 waves.
// Wave w = (head group hg = w & 3, half x = w >> 2): heads 16hg..16hg+15;
// for the scores it covers half x of the D row dimensions, for the output
// half x of the 512 latent columns.  The split's row indices are staged in
// LDS first; its rows are then processed 32 at a time.  Rows reach LDS by
// DMA (global_load_lds, no registers) through a ring of three buffers, two
// steps ahead of the compute: the V part of a row (1 KiB) is one wave
// instruction into a row-major region (stride 1056 B), the 64-wide RoPE
// tail goes 8 rows per instruction into a region of 128-byte rows whose
// 16-byte pieces are XOR-swizzled by (row & 7).  A missing row (past the
// count, or an index outside the cache) is read from a zero row, so each
// wave issues a fixed number of DMA instructions per step and the wait for
// step c is an exact vmcnt.  Per step and wave:
//   QK : partial S^T[row][head] = C Q^T over its half of the dimensions on
//        MFMA 16x16x32 (A = rows from LDS, B = queries in registers), two
//        16-row blocks; the two halves are summed through LDS;
//   softmax: online per head (one head per lane column), lazy rescale
//        when the running max grows by more than 2^8;
//   PV : O^T[col][head] += V^T P^T for its 256 columns, A = V^T read by
//        ds_read_b64_tr_b16, B = P split into bf16 hi + lo.
// Two barriers per step: buffer ready, partial scores ready.
template <int D>
struct AttnCfg {
    static constexpr int ND = D / 32;            // MFMA k-steps of the score
    static constexpr int NH = ND / 2;            // k-steps per half
    static constexpr int VS = 1056;              // LDS stride of a V row (bytes)
    static constexpr int VBYTES = kAttnRows * VS;
    static constexpr int RBYTES = D > 512 ? kAttnRows * 128 : 0;
    static constexpr int BUF = VBYTES + RBYTES;
    static constexpr int NBUF = 3;
};

// Source of the DMA for rows that do not exist.
__device__ __attribute__((aligned(16))) const uint8_t kZeroRow[2 * 576] = {};

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// 16 bytes per lane from src (per-lane address) to LDS at lds + 16 * lane.
// Issued from asm so that the compiler's wait insertion, which knows
// nothing of it, adds no vmcnt wait in front of the LDS reads of the other
// buffers; the kernel waits for it itself.  The asm sets m0 (the LDS
// destination) and says so in its clobber list, so that no value the
// compiler might keep in m0 is assumed to survive it; clang warns that m0 is
// a reserved register, which is the point here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}

// The same with a uniform base address in SGPRs and a per-lane 32-bit
// offset.  The base is read out of a lane by v_readlane just before: a VALU
// write of an SGPR that a VMEM instruction reads needs five wait states (the
// compiler does not see the read inside the asm), hence s_nop 4.
__device__ __forceinline__ void dma16u(uint64_t base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS-only work-group barrier: global accesses in flight are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int D>
__global__ __launch_bounds__(512) void k_attend(Args a) {
    using Cfg = AttnCfg<D>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[Cfg::NBUF * Cfg::BUF];
    __shared__ int32_t sidx[kMaxSplitRows];
    __shared__ f32x4 sx[8][2][64];                 // partial scores per wave
    const int q = blockIdx.y, sp = blockIdx.x;
    const QInfo qi = query_info(a, q);
    const int lane = lane_id(), g = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hg = w & 3, x = w >> 2;
    const int head = 16 * hg + n;

    // a count outside [0, top_k + kpool - 1] makes the query invalid
    int32_t count = 0;
    bool invalid = qi.mode == 2;
    if (!invalid) {
        count = a.sel_count[q];
        if (count < 0 || count > a.top_k + a.kpool - 1) {
            invalid = true;
            count = 0;
        }
    }
    const int32_t start = sp * a.split_rows;
    const int32_t nrows = count > start ? (count - start < a.split_rows ? count - start : a.split_rows) : 0;
    const int nst = (nrows + kAttnRows - 1) / kAttnRows;
    const uint8_t *C = reinterpret_cast<const uint8_t *>(a.cache + (size_t)(invalid ? 0 : qi.seq) * a.cache_stride * D);

    // row indices of the split (-1: no row), padded to whole steps
    {
        const int32_t *selq = a.sel + (size_t)q * a.sel_ld + start;
        for (int r = threadIdx.x; r < nst * kAttnRows; r += 512) {
            int32_t t = -1;
            if (r < nrows) {
                t = selq[r];
                if (t < 0 || (int64_t)t >= a.cache_stride) t = -1;
            }
            sidx[r] = t;
        }
    }
    // this wave's queries: k-steps x*NH .. x*NH + NH - 1
    bf16x8 qreg[Cfg::NH];
    {
        const uint16_t *qp = a.q + ((size_t)q * kHeads + head) * D + 32 * Cfg::NH * x + 8 * g;
#pragma unroll
        for (int j = 0; j < Cfg::NH; j++) qreg[j] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qp + 32 * j));
        // complete the query loads here: no load the compiler tracks may
        // be in flight inside the loop, whose vmcnt waits count DMA only
#pragma unroll
        for (int j = 0; j < Cfg::NH; j++) asm volatile("" ::"v"(qreg[j]));
    }
    __syncthreads();

    // DMA of a step's rows into buffer slot b: V parts of rows w, w+8,
    // w+16, w+24; waves 0..3 also the RoPE tails of rows 8w..8w+7.  iv holds
    // the step's row index of lane & 31, ir that of row 8w + lane / 8.
    const bool rope_wave = D > 512 && w < 4;
    const uint64_t c_base = reinterpret_cast<uint64_t>(C), z_base = reinterpret_cast<uint64_t>(kZeroRow);
    auto issue = [&](int32_t iv, int32_t ir, int b) {
        uint8_t *vb = lds + b * Cfg::BUF;
        // the step's row addresses at once (lane r: row r, the zero row for
        // t < 0), then each of this wave's rows from two lane reads
        const uint64_t m = (uint64_t)(int64_t)(iv >> 31);
        const uint64_t av = ((c_base + (uint64_t)(uint32_t)iv * (2 * D)) & ~m) | (z_base & m);
        const uint32_t alo = (uint32_t)av, ahi = (uint32_t)(av >> 32);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r = w + 8 * i;
            const uint64_t base = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)alo, r) |
                                  ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)ahi, r) << 32);
            dma16u(base, 16 * lane, __builtin_amdgcn_readfirstlane(lds_addr(vb + r * Cfg::VS)));
        }
        if (rope_wave) {
            const int row = 8 * w + (lane >> 3);
            const uint8_t *src = ir >= 0 ? C + (size_t)ir * (2 * D) : kZeroRow;
            const int piece = (lane & 7) ^ (row & 7);
            dma16(src + 1024 + 16 * piece, __builtin_amdgcn_readfirstlane(lds_addr(vb + Cfg::VBYTES + 8 * w * 128)));
        }
    };
    // row indices of step c (-1 past the split)
    auto idx_v = [&](int c) -> int32_t { return c < nst ? sidx[kAttnRows * c + (lane & 31)] : -1; };
    auto idx_r = [&](int c) -> int32_t { return c < nst ? sidx[kAttnRows * c + 8 * (w & 3) + (lane >> 3)] : -1; };

    f32x4 acc[16];
#pragma unroll
    for (int i = 0; i < 16; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY, l_part = 0.f;

    int32_t iv_cur = idx_v(0), iv_n1 = idx_v(1), iv_n2 = idx_v(2), ir_n2 = idx_r(2);
    if (nst > 0) issue(iv_cur, idx_r(0), 0);
    if (nst > 1) issue(iv_n1, idx_r(1), 1);
    int b_cur = 0;
    for (int c = 0; c < nst; c++) {
        // this wave's DMA of step c is done (step c + 1's may be in flight),
        // then every wave's is
        if (c + 1 < nst) {
            if (rope_wave)
                wait_vm<5>();
            else
                wait_vm<4>();
        } else {
            wait_vm<0>();
        }
        lds_barrier();
        if (c + 2 < nst) issue(iv_n2, ir_n2, b_cur == 0 ? 2 : b_cur - 1);
        const uint8_t *vb = lds + b_cur * Cfg::BUF;
        b_cur = b_cur == 2 ? 0 : b_cur + 1;
        const uint64_t okmask = __ballot(lane < kAttnRows && iv_cur >= 0);
        // indices two steps ahead, read while this step computes
        iv_cur = iv_n1;
        iv_n1 = iv_n2;
        iv_n2 = idx_v(c + 3);
        ir_n2 = idx_r(c + 3);

        // partial S^T over this wave's half of the dimensions
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        {
            // all A operands first (one LDS latency for the step), then
            // the MFMA chains of the two row blocks
            const int sb = Cfg::NH * x;
            bf16x8 ra[2 * Cfg::NH];
#pragma unroll
            for (int j = 0; j < Cfg::NH; j++) {
                const int s = sb + j;
                const uint8_t *p0, *p1;
                if (D > 512 && s >= 16) {
                    const int pc = 4 * (s - 16) + g;
                    p0 = vb + Cfg::VBYTES + n * 128 + 16 * (pc ^ (n & 7));
                    p1 = vb + Cfg::VBYTES + (16 + n) * 128 + 16 * (pc ^ (n & 7));
                } else {
                    p0 = vb + n * Cfg::VS + 64 * s + 16 * g;
                    p1 = vb + (16 + n) * Cfg::VS + 64 * s + 16 * g;
                }
                ra[2 * j] = __builtin_bit_cast(bf16x8, *(const u32x4 *)p0);
                ra[2 * j + 1] = __builtin_bit_cast(bf16x8, *(const u32x4 *)p1);
            }
#pragma unroll
            for (int j = 0; j < Cfg::NH; j++) {
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[2 * j], qreg[j], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[2 * j + 1], qreg[j], s1, 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * Cfg::NH, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * Cfg::NH, 0);
        }
        sx[w][0][lane] = s0;
        sx[w][1][lane] = s1;
        lds_barrier();
        s0 += sx[w ^ 4][0][lane];
        s1 += sx[w ^ 4][1][lane];

        // online softmax over this step's rows, per head (lane column n);
        // element j of this lane is row 4g + j (j < 4) or 16 + 4g + j - 4
        float z[8];
        float cmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int rr = (j < 4 ? 0 : 16) + 4 * g + (j & 3);
            const float sv = j < 4 ? s0[j] : s1[j - 4];
            const float v = ((okmask >> rr) & 1) ? sv * a.scale_log2 : -INFINITY;
            z[j] = v;
            cmax = fmaxf(cmax, v);
        }
        cmax = xor16_max(cmax);
        cmax = xor32_max(cmax);
        const bool need = cmax > m_ref + 8.f;
        if (__any(need)) {
            const float m_new = need ? cmax : m_ref;
            const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
            m_ref = m_new;
            l_part *= alpha;
#pragma unroll
            for (int i = 0; i < 16; i++) acc[i] *= alpha;
        }
        bf16x8 phi, plo;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float p = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(z[j] - m_ref);
            l_part += p;
            const uint32_t hb = __float_as_uint(p) & 0xFFFF0000u;
            const float lo = p - __uint_as_float(hb);
            phi[j] = __builtin_bit_cast(__bf16, (uint16_t)(hb >> 16));
            plo[j] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(lo) >> 16));
        }
        // O^T += V^T P^T over this wave's 16 column blocks of 16
        {
            const int r_in = n >> 2, c_in = n & 3;
            const uint8_t *v1 = vb + (4 * g + r_in) * Cfg::VS + 8 * c_in + 512 * x;
            const uint8_t *v2 = vb + (16 + 4 * g + r_in) * Cfg::VS + 8 * c_in + 512 * x;
#pragma unroll
            for (int cb = 0; cb < 16; cb++) {
                const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(v1 + 32 * cb));
                const i16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(v2 + 32 * cb));
                typedef short i16x8 __attribute__((ext_vector_type(8)));
                const i16x8 tv = {t1[0], t1[1], t1[2], t1[3], t2[0], t2[1], t2[2], t2[3]};
                const bf16x8 av = __builtin_bit_cast(bf16x8, tv);
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, phi, acc[cb], 0, 0, 0);
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, plo, acc[cb], 0, 0, 0);
            }
            // V reads run 4 column blocks ahead of the MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int i = 0; i < 12; i++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
    }
    // total softmax mass per head over the four lane groups
    const float l_tot = xor32_sum(xor16_sum(l_part));

    const int col0 = 256 * x + 4 * g;
    if (a.n_split == 1) {
        const bool bad = invalid || l_tot == 0.f;
        const float inv = 1.f / l_tot;
        float *o = a.out + ((size_t)q * kHeads + head) * kLatent + col0;
#pragma unroll
        for (int cb = 0; cb < 16; cb++) {
            f32x4 val = acc[cb] * inv;
            if (bad) val = f32x4{NAN, NAN, NAN, NAN};
            *(f32x4 *)(o + 16 * cb) = val;
        }
        if (a.lse && x == 0 && g == 0)
            a.lse[(size_t)q * kHeads + head] = bad ? NAN : (m_ref + __log2f(l_tot)) * 0.69314718055994531f;
    } else {
        // an invalid query leaves m = -inf, l = 0 in every split: the merge
        // then writes NaN
        const size_t slot = ((size_t)q * a.n_split + sp) * kHeads + head;
        float *o = a.pacc + slot * kLatent + col0;
#pragma unroll
        for (int cb = 0; cb < 16; cb++) *(f32x4 *)(o + 16 * cb) = acc[cb];
        if (x == 0 && g == 0) {
            a.pml[2 * slot] = m_ref;
            a.pml[2 * slot + 1] = l_tot;
        }
    }
}

// Head-split attention for small batches.  One work-group = (head group hg
// of 16 heads, query q, split sp), 512 threads: a few queries still fill the
// chip, and the split partials shrink by the head factor.  The four head
// groups of a (query, split) sit on the same XCD (work-groups are dealt to
// XCDs round-robin; the head group is the slowest index over a pair count
// padded to a multiple of 8), so their shared rows come from L2.  Rows
// arrive by the same DMA ring as in k_attend.  Per step and wave w:
//   QK : row block rt = w & 1 (16 rows), dimension part kq = w >> 1 (a
//        quarter of the k-steps), S^T partial on MFMA 16x16x32 with the
//        queries of that part in registers; the four parts of each row block
//        are summed through LDS, so every wave holds S^T for all 32 rows;
//   softmax: as in k_attend (every wave, per head = lane column);
//   PV : O^T[col][head] += V^T P^T for the wave's 64 columns (4 blocks).
template <int D>
__global__ __launch_bounds__(512) void k_attend_hs(Args a) {
    using Cfg = AttnCfg<D>;
    constexpr int NKQ = (Cfg::ND + 3) / 4;        // most k-steps of a part
    __shared__ __attribute__((aligned(16))) uint8_t lds[Cfg::NBUF * Cfg::BUF];
    __shared__ int32_t sidx[kMaxSplitRows];
    __shared__ f32x4 sx[8][64];                    // partial scores per wave
    const int pairs = a.n_q * a.n_split;
    const int pairs8 = (pairs + 7) & ~7;
    const int hg = blockIdx.x / pairs8, pair = blockIdx.x % pairs8;
    if (pair >= pairs) return;
    const int q = pair / a.n_split, sp = pair % a.n_split;
    const QInfo qi = query_info(a, q);
    const int lane = lane_id(), g = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rt = w & 1, kq = w >> 1;
    const int kcnt = Cfg::ND / 4 + (kq < Cfg::ND % 4 ? 1 : 0);
    const int k0 = kq * (Cfg::ND / 4) + (kq < Cfg::ND % 4 ? kq : Cfg::ND % 4);
    const int head = 16 * hg + n;

    // a count outside [0, top_k + kpool - 1] makes the query invalid
    int32_t count = 0;
    bool invalid = qi.mode == 2;
    if (!invalid) {
        count = a.sel_count[q];
        if (count < 0 || count > a.top_k + a.kpool - 1) {
            invalid = true;
            count = 0;
        }
    }
    const int32_t start = sp * a.split_rows;
    const int32_t nrows = count > start ? (count - start < a.split_rows ? count - start : a.split_rows) : 0;
    const int nst = (nrows + kAttnRows - 1) / kAttnRows;
    const uint8_t *C = reinterpret_cast<const uint8_t *>(a.cache + (size_t)(invalid ? 0 : qi.seq) * a.cache_stride * D);

    {
        const int32_t *selq = a.sel + (size_t)q * a.sel_ld + start;
        for (int r = threadIdx.x; r < nst * kAttnRows; r += 512) {
            int32_t t = -1;
            if (r < nrows) {
                t = selq[r];
                if (t < 0 || (int64_t)t >= a.cache_stride) t = -1;
            }
            sidx[r] = t;
        }
    }
    // this wave's queries: k-steps k0 .. k0 + kcnt - 1 of heads 16 hg ..
    bf16x8 qreg[NKQ];
    {
        const uint16_t *qp = a.q + ((size_t)q * kHeads + head) * D + 32 * k0 + 8 * g;
#pragma unroll
        for (int j = 0; j < NKQ; j++)
            qreg[j] = j < kcnt ? __builtin_bit_cast(bf16x8, *(const u32x4 *)(qp + 32 * j)) : bf16x8{};
#pragma unroll
        for (int j = 0; j < NKQ; j++) asm volatile("" ::"v"(qreg[j]));
    }
    __syncthreads();

    const bool rope_wave = D > 512 && w < 4;
    auto issue = [&](int32_t iv, int32_t ir, int b) {
        uint8_t *vb = lds + b * Cfg::BUF;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r = w + 8 * i;
            const int32_t t = __builtin_amdgcn_readlane(iv, r);
            const uint8_t *src = t >= 0 ? C + (size_t)t * (2 * D) : kZeroRow;
            dma16(src + 16 * lane, __builtin_amdgcn_readfirstlane(lds_addr(vb + r * Cfg::VS)));
        }
        if (rope_wave) {
            const int row = 8 * w + (lane >> 3);
            const uint8_t *src = ir >= 0 ? C + (size_t)ir * (2 * D) : kZeroRow;
            const int piece = (lane & 7) ^ (row & 7);
            dma16(src + 1024 + 16 * piece, __builtin_amdgcn_readfirstlane(lds_addr(vb + Cfg::VBYTES + 8 * w * 128)));
        }
    };
    auto idx_v = [&](int c) -> int32_t { return c < nst ? sidx[kAttnRows * c + (lane & 31)] : -1; };
    auto idx_r = [&](int c) -> int32_t { return c < nst ? sidx[kAttnRows * c + 8 * (w & 3) + (lane >> 3)] : -1; };

    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY, l_part = 0.f;

    int32_t iv_cur = idx_v(0), iv_n1 = idx_v(1), iv_n2 = idx_v(2), ir_n2 = idx_r(2);
    if (nst > 0) issue(iv_cur, idx_r(0), 0);
    if (nst > 1) issue(iv_n1, idx_r(1), 1);
    int b_cur = 0;
    for (int c = 0; c < nst; c++) {
        if (c + 1 < nst) {
            if (rope_wave)
                wait_vm<5>();
            else
                wait_vm<4>();
        } else {
            wait_vm<0>();
        }
        lds_barrier();
        if (c + 2 < nst) issue(iv_n2, ir_n2, b_cur == 0 ? 2 : b_cur - 1);
        const uint8_t *vb = lds + b_cur * Cfg::BUF;
        b_cur = b_cur == 2 ? 0 : b_cur + 1;
        const uint64_t okmask = __ballot(lane < kAttnRows && iv_cur >= 0);
        iv_cur = iv_n1;
        iv_n1 = iv_n2;
        iv_n2 = idx_v(c + 3);
        ir_n2 = idx_r(c + 3);

        // partial S^T of row block rt over this wave's k-steps
        f32x4 sp_acc = {0.f, 0.f, 0.f, 0.f};
        {
            bf16x8 ra[NKQ];
#pragma unroll
            for (int j = 0; j < NKQ; j++) {
                const int s = k0 + j;
                const uint8_t *p0;
                if (D > 512 && s >= 16) {
                    const int pc = 4 * (s - 16) + g;
                    p0 = vb + Cfg::VBYTES + (16 * rt + n) * 128 + 16 * (pc ^ (n & 7));
                } else {
                    p0 = vb + (16 * rt + n) * Cfg::VS + 64 * s + 16 * g;
                }
                ra[j] = j < kcnt ? __builtin_bit_cast(bf16x8, *(const u32x4 *)p0) : bf16x8{};
            }
#pragma unroll
            for (int j = 0; j < NKQ; j++)
                if (j < kcnt) sp_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[j], qreg[j], sp_acc, 0, 0, 0);
        }
        sx[w][lane] = sp_acc;
        lds_barrier();
        f32x4 s0 = sx[0][lane], s1 = sx[1][lane];
#pragma unroll
        for (int k = 1; k < 4; k++) {
            s0 += sx[2 * k][lane];
            s1 += sx[2 * k + 1][lane];
        }

        // online softmax over this step's rows, per head (lane column n);
        // element j of this lane is row 4g + j (j < 4) or 16 + 4g + j - 4
        float z[8];
        float cmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int rr = (j < 4 ? 0 : 16) + 4 * g + (j & 3);
            const float sv = j < 4 ? s0[j] : s1[j - 4];
            const float v = ((okmask >> rr) & 1) ? sv * a.scale_log2 : -INFINITY;
            z[j] = v;
            cmax = fmaxf(cmax, v);
        }
        cmax = xor16_max(cmax);
        cmax = xor32_max(cmax);
        const bool need = cmax > m_ref + 8.f;
        if (__any(need)) {
            const float m_new = need ? cmax : m_ref;
            const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
            m_ref = m_new;
            l_part *= alpha;
#pragma unroll
            for (int i = 0; i < 4; i++) acc[i] *= alpha;
        }
        bf16x8 phi, plo;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float p = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(z[j] - m_ref);
            l_part += p;
            const uint32_t hb = __float_as_uint(p) & 0xFFFF0000u;
            const float lo = p - __uint_as_float(hb);
            phi[j] = __builtin_bit_cast(__bf16, (uint16_t)(hb >> 16));
            plo[j] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(lo) >> 16));
        }
        // O^T += V^T P^T over this wave's 4 column blocks of 16
        {
            const int r_in = n >> 2, c_in = n & 3;
            const uint8_t *v1 = vb + (4 * g + r_in) * Cfg::VS + 8 * c_in + 128 * w;
            const uint8_t *v2 = vb + (16 + 4 * g + r_in) * Cfg::VS + 8 * c_in + 128 * w;
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            bf16x8 av[4];
#pragma unroll
            for (int cb = 0; cb < 4; cb++) {
                const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(v1 + 32 * cb));
                const i16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(v2 + 32 * cb));
                const i16x8 tv = {t1[0], t1[1], t1[2], t1[3], t2[0], t2[1], t2[2], t2[3]};
                av[cb] = __builtin_bit_cast(bf16x8, tv);
            }
#pragma unroll
            for (int cb = 0; cb < 4; cb++) {
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[cb], phi, acc[cb], 0, 0, 0);
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[cb], plo, acc[cb], 0, 0, 0);
            }
        }
    }
    const float l_tot = xor32_sum(xor16_sum(l_part));

    const int col0 = 64 * w + 4 * g;
    if (a.n_split == 1) {
        const bool bad = invalid || l_tot == 0.f;
        const float inv = 1.f / l_tot;
        float *o = a.out + ((size_t)q * kHeads + head) * kLatent + col0;
#pragma unroll
        for (int cb = 0; cb < 4; cb++) {
            f32x4 val = acc[cb] * inv;
            if (bad) val = f32x4{NAN, NAN, NAN, NAN};
            *(f32x4 *)(o + 16 * cb) = val;
        }
        if (a.lse && w == 0 && g == 0)
            a.lse[(size_t)q * kHeads + head] = bad ? NAN : (m_ref + __log2f(l_tot)) * 0.69314718055994531f;
    } else {
        const size_t slot = ((size_t)q * a.n_split + sp) * kHeads + head;
        float *o = a.pacc + slot * kLatent + col0;
#pragma unroll
        for (int cb = 0; cb < 4; cb++) *(f32x4 *)(o + 16 * cb) = acc[cb];
        if (w == 0 && g == 0) {
            a.pml[2 * slot] = m_ref;
            a.pml[2 * slot + 1] = l_tot;
        }
    }
}

// Attention with wave-private rows, for small batches.  Same grid as
// k_attend_hs (head group hg, query q, split sp; the four head groups of a
// (query, split) on one XCD), but 256 threads whose 4 waves share nothing
// inside the row loop: the split's rows go in 16-row steps to the waves in
// turn (step s to wave s % 4).  Each wave DMAs its own steps into its own
// two LDS buffers (the layout of k_attend, 16 rows), waits for them with
// its own vmcnt and no barrier, and per step
//   QK : S^T[16 rows][16 heads] over all D dimensions on MFMA 16x16x32
//        (A = rows from LDS, B = the queries, all k-steps in registers);
//   softmax: online per head, lazy rescale as in k_attend;
//   PV : O^T[col][head] += V^T P^T for all 512 columns.  The hi and lo
//        bf16 halves of P form the 32-deep K of one MFMA: lane group g
//        holds P of rows 4g..4g+3 (the S^T accumulator layout) as
//        (hi, hi, hi, hi, lo, lo, lo, lo), and A repeats the same four V
//        rows, read by one ds_read_b64_tr_b16, in both halves.
// The four waves' (max, sum, O) are merged through LDS once at the end.
constexpr int kWvRows = 16;   // rows per step of one wave

template <int D>
struct WvCfg {
    static constexpr int ND = D / 32;                       // MFMA k-steps of the score
    static constexpr int VS = 1056;                         // LDS stride of a V row (bytes)
    static constexpr int VBYTES = kWvRows * VS;
    static constexpr int RBYTES = D > 512 ? kWvRows * 128 : 0;
    static constexpr int BUF = VBYTES + RBYTES;
    static constexpr int WAVE = 2 * BUF;                    // one wave's two buffers
    static constexpr int NDMA = kWvRows + RBYTES / 1024;    // DMA instructions per step
    static constexpr int OS = 516;                          // floats per head row of the merge
};
static_assert(4 * 16 * WvCfg<512>::OS * 4 <= 4 * WvCfg<512>::WAVE, "merge fits the row buffers");

// Row loop and merge of the wave-private attention, shared by k_attend_wv
// and k_attend_sel.  On entry sidx holds the split's row indices, wave w's
// step j in sidx[16 (w + 4 j) .. + 15] (-1: no row), nj is this wave's step
// count, and qreg holds the wave's queries (their loads may be in flight).
template <int D>
__device__ __forceinline__ void wv_rows(const Args &a, uint8_t *lds, const int32_t *sidx, float (*smx)[16],
                                        float (*ssum)[16], const bf16x8 (&qreg)[WvCfg<D>::ND], const uint8_t *C,
                                        int q, int sp, int hg, int w, int nj, bool invalid) {
    using Cfg = WvCfg<D>;
    const int lane = lane_id(), g = lane >> 4, n = lane & 15;
    uint8_t *wb = lds + w * Cfg::WAVE;
    const uint32_t voff = 16 * lane;
    const uint32_t wb_lds = __builtin_amdgcn_readfirstlane(lds_addr(wb));
    const uint64_t c_base = reinterpret_cast<uint64_t>(C), z_base = reinterpret_cast<uint64_t>(kZeroRow);
    // address of row t, or of the zero row for t outside [0, cache_stride),
    // without a branch: one unsigned 32-bit compare (a negative t is a huge
    // unsigned value) and a mask
    const uint32_t rlim = a.cache_stride >= (int64_t)0x80000000u ? 0x80000000u : (uint32_t)a.cache_stride;
    auto row_ok = [rlim](int32_t t) { return (uint32_t)t < rlim; };
    auto row_addr = [&](int32_t t) -> uint64_t {
        const uint64_t m = (uint64_t)0 - (uint64_t)row_ok(t);
        return ((c_base + (uint64_t)(uint32_t)t * (2 * D)) & m) | (z_base & ~m);
    };
    // lane & 15 holds the index of row lane & 15 of the wave's step j
    auto idx_v = [&](int j) -> int32_t { return j < nj ? sidx[kWvRows * (w + 4 * j) + (lane & 15)] : -1; };
    auto issue = [&](int j, int32_t iv, int b) {
        const uint32_t vb = wb_lds + b * Cfg::BUF;
        // the step's 16 row addresses at once (lane r: row r), then each
        // row's DMA from its two halves read out of lane r
        const uint64_t av = row_addr(iv);
        const uint32_t alo = (uint32_t)av, ahi = (uint32_t)(av >> 32);
#pragma unroll
        for (int r = 0; r < kWvRows; r++) {
            const uint64_t base = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)alo, r) |
                                  ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)ahi, r) << 32);
            dma16u(base, voff, vb + r * Cfg::VS);
        }
        if constexpr (D > 512) {
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int row = 8 * i + (lane >> 3);
                const int32_t t = sidx[kWvRows * (w + 4 * j) + row];
                const int piece = (lane & 7) ^ (row & 7);
                dma16(reinterpret_cast<const uint8_t *>(row_addr(t)) + 1024 + 16 * piece, vb + Cfg::VBYTES + 1024 * i);
            }
        }
    };

    // The running max is only raised at a wave's first step, where nothing
    // has been accumulated yet, to the step's max plus 16 (p <= 2^-16 then;
    // fp32 keeps full relative precision far below that).  A later step
    // whose max passes the reference by more than 8 raises it the same way
    // and restarts the wave's rows from its first step, so the accumulators
    // are never rescaled inside the loop.
    f32x4 acc[32];
    float m_ref = -INFINITY, l_part = 0.f;
    for (;;) {
#pragma unroll
        for (int i = 0; i < 32; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        l_part = 0.f;
        bool restart = false;
        if (nj > 0) issue(0, idx_v(0), 0);
        if (nj > 1) issue(1, idx_v(1), 1);
        // complete the query loads before the loop, whose vmcnt waits count
        // DMA only (the first pass also waits for its first two steps here)
#pragma unroll
        for (int j = 0; j < Cfg::ND; j++) asm volatile("" ::"v"(qreg[j]));
        for (int j = 0; j < nj; j++) {
            const int32_t iv = idx_v(j);
            if (j + 1 < nj)
                wait_vm<Cfg::NDMA>();
            else
                wait_vm<0>();
            const uint8_t *vb = wb + (j & 1) * Cfg::BUF;
            const uint64_t okmask = __ballot(lane < kWvRows && row_ok(iv));

            // S^T of the step's 16 rows (lane: rows 4g .. 4g + 3 of head n),
            // two independent accumulation chains
            f32x4 s;
            {
                bf16x8 ra[Cfg::ND];
#pragma unroll
                for (int k = 0; k < Cfg::ND; k++) {
                    const uint8_t *p0;
                    if (D > 512 && k >= 16)
                        p0 = vb + Cfg::VBYTES + n * 128 + 16 * ((4 * (k - 16) + g) ^ (n & 7));
                    else
                        p0 = vb + n * Cfg::VS + 64 * k + 16 * g;
                    ra[k] = __builtin_bit_cast(bf16x8, *(const u32x4 *)p0);
                }
                // all reads in flight before the first product
#pragma unroll
                for (int k = 0; k < Cfg::ND; k++) asm volatile("" ::"v"(ra[k]));
                f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < Cfg::ND; k += 2) {
                    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[k], qreg[k], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[k + 1], qreg[k + 1], s1, 0, 0, 0);
                }
                s = s0 + s1;
            }
            float z[4];
            float cmax = -INFINITY;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float v = ((okmask >> (4 * g + r)) & 1) ? s[r] * a.scale_log2 : -INFINITY;
                z[r] = v;
                cmax = fmaxf(cmax, v);
            }
            cmax = xor16_max(cmax);
            cmax = xor32_max(cmax);
            const bool need = cmax > m_ref + 8.f;
            if (__any(need)) {
                m_ref = need ? cmax + 16.f : m_ref;
                if (j > 0) {
                    restart = true;
                    break;
                }
            }
            bf16x8 pb;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float p = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(z[r] - m_ref);
                l_part += p;
                const uint32_t hb = __float_as_uint(p) & 0xFFFF0000u;
                const float lo = p - __uint_as_float(hb);
                pb[r] = __builtin_bit_cast(__bf16, (uint16_t)(hb >> 16));
                pb[4 + r] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(lo) >> 16));
            }
            // O^T += V^T P^T, 32 column blocks of 16
            {
                const uint8_t *v1 = vb + (4 * g + (n >> 2)) * Cfg::VS + 8 * (n & 3);
                typedef short i16x8 __attribute__((ext_vector_type(8)));
                i16x4 t[32];
#pragma unroll
                for (int c = 0; c < 32; c++) t[c] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(v1 + 32 * c));
#pragma unroll
                for (int c = 0; c < 32; c++) asm volatile("" ::"v"(t[c]));
#pragma unroll
                for (int c = 0; c < 32; c++) {
                    // the four V values twice (K = 16 rows x {hi, lo} of P):
                    // one v_mov_b64 (the compiler copies the pair with two
                    // v_mov_b32; fused attention at 8 x 128K 19.7 vs 20.2 us)
                    typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
                    const uint64_t t64 = __builtin_bit_cast(uint64_t, t[c]);
                    uint64_t d64;
                    asm("v_mov_b64 %0, %1" : "=v"(d64) : "v"(t64));
                    const u64x2 tv = {t64, d64};
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, tv), pb, acc[c], 0, 0, 0);
                }
            }
            // the buffer is free once its LDS reads have returned
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (j + 2 < nj) issue(j + 2, idx_v(j + 2), j & 1);
        }
        if (!restart) break;
        // drain this pass's DMA before the buffers are filled again
        wait_vm<0>();
    }

    // merge the four waves: wave w finishes column blocks 8w .. 8w + 7 of
    // the 16 heads.  Each wave's (max, sum) and the column blocks it does
    // not finish go to LDS; after one barrier a wave combines its own blocks,
    // still in registers, with the other three waves' from LDS, in the
    // accumulator layout (lane (g, n): head n, columns 16 cb + 4 g .. + 3).
    const float l_w = xor32_sum(xor16_sum(l_part));
    if (g == 0) {
        smx[w][n] = m_ref;
        ssum[w][n] = l_w;
    }
    __syncthreads();   // every wave is past its last LDS read of the row buffers
    float *const sbase = reinterpret_cast<float *>(lds);
    {
        float *so = sbase + (w * 16 + n) * Cfg::OS + 4 * g;
#pragma unroll
        for (int cb = 0; cb < 32; cb++)
            if ((cb >> 3) != w) *(f32x4 *)(so + 16 * cb) = acc[cb];
    }
    __syncthreads();
    float fk[4], M = -INFINITY, L = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ww++) M = fmaxf(M, smx[ww][n]);
#pragma unroll
    for (int ww = 0; ww < 4; ww++) {
        const float mw = smx[ww][n];
        fk[ww] = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L += ssum[ww][n] * fk[ww];
    }
    const int hd = 16 * hg + n;
    const bool bad = invalid || L == 0.f;
    const size_t slot = ((size_t)q * a.n_split + sp) * kHeads + hd;
    // the wave index is uniform: one copy of the finish per wave, so that
    // its own accumulators are indexed statically
    auto finish = [&](auto wtag) {
        constexpr int W = decltype(wtag)::value;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int cb = 8 * W + i, col = 16 * cb + 4 * g;
            f32x4 v = acc[cb] * fk[W];
#pragma unroll
            for (int ww = 0; ww < 4; ww++)
                if (ww != W) v += *(const f32x4 *)(sbase + (ww * 16 + n) * Cfg::OS + col) * fk[ww];
            if (a.n_split == 1) {
                const f32x4 o = bad ? f32x4{NAN, NAN, NAN, NAN} : v * (1.f / L);
                *(f32x4 *)(a.out + ((size_t)q * kHeads + hd) * kLatent + col) = o;
            } else {
                *(f32x4 *)(a.pacc + slot * kLatent + col) = v;
            }
        }
    };
    if (w == 0)
        finish(std::integral_constant<int, 0>());
    else if (w == 1)
        finish(std::integral_constant<int, 1>());
    else if (w == 2)
        finish(std::integral_constant<int, 2>());
    else
        finish(std::integral_constant<int, 3>());
    if (w == 0 && g == 0) {
        if (a.n_split == 1) {
            if (a.lse) a.lse[(size_t)q * kHeads + hd] = bad ? NAN : (M + __log2f(L)) * 0.69314718055994531f;
        } else {
            a.pml[2 * slot] = M;
            a.pml[2 * slot + 1] = L;
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void k_attend_wv(Args a) {
    using Cfg = WvCfg<D>;
    constexpr int kPer = kWvMaxRows / 256;                  // row indices per thread
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * Cfg::WAVE];
    __shared__ int32_t sidx[kWvMaxRows];
    __shared__ float smx[4][16], ssum[4][16];
    const int pairs = a.n_q * a.n_split;
    const int pairs8 = (pairs + 7) & ~7;
    const int hg = blockIdx.x / pairs8, pair = blockIdx.x % pairs8;
    if (pair >= pairs) return;
    const int q = pair / a.n_split, sp = pair % a.n_split;
    const int32_t count_in = a.sel_count[q];   // issued with the query's own loads
    const QInfo qi = query_info(a, q);
    const int lane = lane_id(), g = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int head = 16 * hg + n;
    const int32_t start = sp * a.split_rows;

    // The count, the split's row indices and the queries are loaded in one
    // round trip; indices past the count are read (inside the caller's row
    // stride) and dropped once the count is known.  Wave w reads the indices
    // of its own steps w, w + 4, ...: lane l of rix[i] holds row l & 15 of
    // the wave's step 4 i + l / 16, and the wave keeps them in its own part
    // of sidx, so no barrier is needed before its first DMA.
    int32_t rix[kPer];
    {
        const int32_t *selq = a.sel + (size_t)q * a.sel_ld + start;
#pragma unroll
        for (int i = 0; i < kPer; i++) {
            const int r = kWvRows * (w + 4 * (4 * i + g)) + n;
            rix[i] = (r < a.split_rows && start + r < a.sel_ld) ? selq[r] : -1;
        }
    }
    bf16x8 qreg[Cfg::ND];
    {
        const uint16_t *qp = a.q + ((size_t)q * kHeads + head) * D + 8 * g;
#pragma unroll
        for (int j = 0; j < Cfg::ND; j++) qreg[j] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qp + 32 * j));
    }
    // a count outside [0, top_k + kpool - 1] makes the query invalid
    const bool invalid = qi.mode == 2 || count_in < 0 || count_in > a.top_k + a.kpool - 1;
    const int32_t count = invalid ? 0 : count_in;
    const int32_t nrows = count > start ? (count - start < a.split_rows ? count - start : a.split_rows) : 0;
    const int nst = (nrows + kWvRows - 1) / kWvRows;
    const int nj = nst > w ? (nst - w + 3) / 4 : 0;   // this wave's steps w, w + 4, ...
    const uint8_t *C = reinterpret_cast<const uint8_t *>(a.cache + (size_t)(invalid ? 0 : qi.seq) * a.cache_stride * D);
#pragma unroll
    for (int i = 0; i < kPer; i++) {
        const int r = kWvRows * (w + 4 * (4 * i + g)) + n;
        int32_t t = rix[i];
        if (r >= nrows || t < 0 || (int64_t)t >= a.cache_stride) t = -1;
        if (4 * i + g < nj) sidx[r] = t;
    }

    wv_rows<D>(a, lds, sidx, smx, ssum, qreg, C, q, sp, hg, w, nj, invalid);
}

// ---------------------------------------------------------------- top-k inside the attention work-group
// k_attend_sel: the wave-private attention of k_attend_wv with the exact
// top-k (same definition as k_select) done by every attention work-group
// of the query itself, in LDS, before its rows are fetched: no k_select
// launch, and no selection written to and read back from memory.  The
// work-group takes the candidates of the query (k_filter's chunk slots, or
// in SCAN mode, rows of at most 16,384, every row whose first digit reaches
// the threshold bucket of a histogram it builds itself), resolves digits 2
// and 3 of the keep-th order key, ranks the kept rows in ascending row
// order, and keeps the token positions of its own split.  The candidate
// arrays alias the row buffers, which are free until the first DMA.  When
// the candidates exceed the LDS, the same decisions are made from passes
// over the query's scores.
constexpr int kAsCap = 12288;            // candidates kept in LDS
constexpr int kAsPer = 16;               // rows per thread per pass tile
constexpr int kAsTile = 256 * kAsPer;

struct AsShared {
    uint64_t kr[kAsCap];                 // candidates in row order: order key << 32 | row
    uint32_t pre[kMaxChunks + 1];        // exclusive prefix of the chunks' candidate counts
    uint32_t h1[kHistBins];              // first digit (SCAN mode)
    uint32_t h2[1024];
    uint32_t h3[1024];
    uint32_t scan[4];
    uint32_t res[4];
    uint32_t epos[256];                  // emission: first position of each thread's kept rows
    uint64_t etake[256];                 // and the mask of its kept candidates
};
static_assert(sizeof(AsShared) <= 4 * WvCfg<512>::WAVE, "the selection fits the row buffers");

// Copies every row r in [r0, r1) whose first digit is at least b1 as (key,
// r), in row order, to sh.key / sh.row from position `base` on; entries at
// or past `limit` are counted but not stored.  Returns the number found.
__device__ __forceinline__ uint32_t as_compact(const float *s, bool vec, int64_t r0, int64_t r1, uint32_t b1, uint32_t base,
                               uint32_t limit, AsShared &sh, const u32x4 *first = nullptr) {
    uint32_t found = 0;
    for (int64_t sb = r0; sb < r1; sb += kAsTile) {
        const int64_t rb = sb + kAsPer * threadIdx.x;
        float v[kAsPer];
        if (first && sb == r0) {
            // the first tile's scores, already in registers
#pragma unroll
            for (int i = 0; i < kAsPer; i++) v[i] = __uint_as_float(first[i >> 2][i & 3]);
        } else {
            load_scores<kAsPer>(s, rb, r1, vec, v);
        }
        uint32_t keys[kAsPer];
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < kAsPer; i++) {
            keys[i] = order_key(v[i]);
            if (rb + i < r1 && (keys[i] >> 20) >= b1) m |= 1u << i;
        }
        uint32_t tot;
        uint32_t pos = base + found + block_excl_scan(__builtin_popcount(m), sh.scan, tot);
        found += tot;
#pragma unroll
        for (int i = 0; i < kAsPer; i++) {
            if (!((m >> i) & 1)) continue;
            if (pos < limit) sh.kr[pos] = ((uint64_t)keys[i] << 32) | (uint32_t)(rb + i);
            pos++;
        }
    }
    return found;
}

// One pass over rows [0, rows) of the query's scores adding the order keys
// k with (k >> shift) == match to h[(k >> hshift) & (nb - 1)].
__device__ __forceinline__ void as_hist_pass(const float *s, bool vec, int64_t rows, int shift, uint32_t match, int hshift,
                             uint32_t nb, uint32_t *h) {
    for (int64_t sb = 0; sb < rows; sb += kAsTile) {
        const int64_t rb = sb + kAsPer * threadIdx.x;
        float v[kAsPer];
        load_scores<kAsPer>(s, rb, rows, vec, v);
#pragma unroll
        for (int i = 0; i < kAsPer; i++) {
            const uint32_t k = order_key(v[i]);
            if (rb + i < rows && (shift >= 32 || (k >> shift) == match)) atomicAdd(&h[(k >> hshift) & (nb - 1)], 1u);
        }
    }
}

// The selection of query q, restricted to token positions [start, start +
// split_rows): sidx[P - start] = the token at position P of the ascending
// selection (kept pools expanded, then the unpooled tail), -1 past the
// count.  With write_sel the same positions go to sel (and, for the last
// split, the padding after the splits up to sel_ld; for the first split the
// count).  Returns the selection count.  All 256 threads call it.
// The filter-mode selection's first loads, issued at the kernel's start,
// before the query's fields return (none of them depends on those): the
// threshold bucket b1 and the rows above it (k_filter), the second-digit
// histogram of bucket b1 (thread t: bins 1023 - 4t - i), the chunk
// candidate counts (thread t: chunks 4t .. 4t + 3; lane l of wave w also
// chunk w + 4 (l % 16)), and the first 128 slots of the wave's chunks
// w + 4u, read before the counts say how many are filled.  The plan's chunk
// count bounds them; as_select drops what lies past the query's own.
constexpr int kAsU = 16;
struct AsPre {
    u32x4 sv[kAsU];
    uint32_t cw, c4[4], h4[4], b1, above1;
};

__device__ __forceinline__ void as_preload(const Args &a, int q, AsPre &p) {
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const uint64_t *cq = a.cand + (size_t)q * a.n_chunks * a.cand_cap;
    const uint32_t *cc = a.chunk_cnt + (size_t)q * a.n_chunks;
    const uint32_t *gh2 = a.hist + (size_t)q * kHistStride + kHistH2;
#pragma unroll
    for (int u = 0; u < kAsU; u++) {
        const int c = w + 4 * u;
        p.sv[u] = c < a.n_chunks ? *(const u32x4 *)(cq + (size_t)c * a.cand_cap + 2 * lane) : u32x4{0u, 0u, 0u, 0u};
    }
    const int cl = w + 4 * (lane & 15);
    p.cw = cl < a.n_chunks ? cc[cl] : 0u;
#pragma unroll
    for (int i = 0; i < 4; i++) p.c4[i] = 4 * tid + i < a.n_chunks ? cc[4 * tid + i] : 0u;
    p.b1 = a.thr[2 * q];
    p.above1 = a.thr[2 * q + 1];
#pragma unroll
    for (int i = 0; i < 4; i++) p.h4[i] = gh2[1023 - 4 * tid - i];
}

template <bool SCAN, class IssueQ>
__device__ __forceinline__ int32_t as_select(const Args &a, AsShared &sh, int32_t *sidx, int q, const QInfo &qi,
                                             int sp, bool write_sel, IssueQ issue_q, const AsPre &pre) {
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int kp = a.kpool;
    const int32_t start = sp * a.split_rows, split_end = start + a.split_rows;
    int32_t count = 0;
    int32_t pooled = 0, tail = 0;   // sparse: positions [0, pooled) are kept pools, then `tail` tail tokens
    if (qi.mode != 1) issue_q();
    // kept row number p (ascending) -> token positions p kp .. p kp + kp - 1
    // of this split (the exported selection is copied from sidx later)
    auto emit = [&](uint32_t p, int32_t r) {
        if (kp == 1) {
            const int32_t P = (int32_t)p;
            if (P >= start && P < split_end) sidx[P - start] = r;
            return;
        }
#pragma unroll 1
        for (int j = 0; j < kp; j++) {
            const int32_t P = (int32_t)p * kp + j;
            if (P >= start && P < split_end) sidx[P - start] = r * kp + j;
        }
    };
    if (qi.mode == 1) {
        const uint32_t keep = (uint32_t)a.keep;
        const int64_t rows = qi.rows;
        const float *s = a.scores_in + (size_t)q * a.score_ld;
        const bool vec = (reinterpret_cast<uintptr_t>(s) & 15) == 0;
        for (int i = tid; i < 1024; i += 256) sh.h3[i] = 0;
        uint32_t b1, above1, n_cand = 0, b2, above2;
        bool in_lds;
        if (SCAN) {
            issue_q();
            for (int i = tid; i < 1024; i += 256) sh.h2[i] = 0;
            if (a.hist_on) {
                // the scorer's first-digit histogram, read at the kernel's
                // start (pre.sv[j]: bins 4095 - 16 t - 4 j - 3 .. + 3)
                uint32_t hc[16], in_b1;
#pragma unroll
                for (int i = 0; i < 16; i++) hc[i] = pre.sv[(15 - i) >> 2][(15 - i) & 3];
                b1 = bucket_from_regs<16>(hc, keep, sh.scan, sh.res, above1, &in_b1);
                n_cand = above1 + in_b1;
            } else {
                for (int i = tid; i < kHistBins; i += 256) sh.h1[i] = 0;
                __syncthreads();
                as_hist_pass(s, vec, rows, 32, 0u, 20, kHistBins, sh.h1);
                __syncthreads();
                b1 = find_bucket<kHistBins>(sh.h1, keep, sh.scan, sh.res, above1);
                n_cand = above1 + sh.h1[b1];
            }
            in_lds = n_cand <= (uint32_t)kAsCap;
            if (in_lds) {
                as_compact(s, vec, 0, rows, b1, 0u, (uint32_t)kAsCap, sh, pre.sv + 4);
                __syncthreads();
                for (uint32_t i0 = 0; i0 < n_cand; i0 += 256 * 8) {
                    uint32_t k[8];
#pragma unroll
                    for (int u = 0; u < 8; u++) {
                        const uint32_t i = i0 + tid + 256 * u;
                        k[u] = i < n_cand ? (uint32_t)(sh.kr[i] >> 32) : 0u;
                    }
#pragma unroll
                    for (int u = 0; u < 8; u++) {
                        const uint32_t i = i0 + tid + 256 * u;
                        if (i < n_cand && (k[u] >> 20) == b1) atomicAdd(&sh.h2[(k[u] >> 10) & 1023], 1u);
                    }
                }
            } else {
                as_hist_pass(s, vec, rows, 20, b1, 10, 1024, sh.h2);
            }
            __syncthreads();
            b2 = find_bucket<1024>(sh.h2, keep - above1, sh.scan, sh.res, above2);
        } else {
            // the preloaded round trip (as_preload); chunks past the
            // query's own are dropped
            const int nch = (int)((rows + a.chunk - 1) / a.chunk);
            const uint64_t *cq = a.cand + (size_t)q * a.n_chunks * a.cand_cap;
            constexpr int kU = kAsU;
            const u32x4 *sv = pre.sv;
            const int cl = w + 4 * (lane & 15);
            const uint32_t cw = cl < nch ? pre.cw : 0u;
            uint32_t c4[4];
#pragma unroll
            for (int i = 0; i < 4; i++) c4[i] = 4 * tid + i < nch ? pre.c4[i] : 0u;
            b1 = pre.b1;
            above1 = pre.above1;
            const uint32_t(&h4)[4] = pre.h4;
            issue_q();
            uint32_t run = block_excl_scan(c4[0] + c4[1] + c4[2] + c4[3], sh.scan, n_cand);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if (4 * tid + i < nch) sh.pre[4 * tid + i] = run;
                run += c4[i];
            }
            const bool long_chunk = nch > 4 * kU || c4[0] > 128u || c4[1] > 128u || c4[2] > 128u || c4[3] > 128u;
            const bool any_long = __syncthreads_or(long_chunk) != 0;   // also publishes pre
            b2 = bucket_from_regs<4>(h4, keep - above1, sh.scan, sh.res, above2);
            in_lds = n_cand <= (uint32_t)kAsCap;
            if (in_lds) {
                // chunk offsets into scalar registers, then the wave's slots
                // stored to their row-ordered places
                const uint32_t pv = cl < nch ? sh.pre[cl] : 0u;
#pragma unroll
                for (int u = 0; u < kU; u++) {
                    if (w + 4 * u >= nch) break;
                    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)pv, u);
                    const uint32_t n = (uint32_t)__builtin_amdgcn_readlane((int)cw, u);
                    if (n > (uint32_t)a.cand_cap) continue;       // compacted again below
                    const uint32_t j = 2 * lane;
                    if (j < n) sh.kr[b + j] = (uint64_t)sv[u][0] | ((uint64_t)sv[u][1] << 32);
                    if (j + 1 < n) sh.kr[b + j + 1] = (uint64_t)sv[u][2] | ((uint64_t)sv[u][3] << 32);
                }
                if (any_long) {
                    // slots past the first 128 of a chunk, and chunks beyond
                    // the first 64; chunks whose slots overflowed are
                    // compacted again from the scores
                    for (int c = w; c < nch; c += 4) {
                        const uint32_t b = sh.pre[c], n = (c + 1 < nch ? sh.pre[c + 1] : n_cand) - b;
                        if (n > (uint32_t)a.cand_cap) continue;
                        for (uint32_t j = (c < 4 * kU ? 128u : 0u) + lane; j < n; j += 64)
                            sh.kr[b + j] = cq[(size_t)c * a.cand_cap + j];
                    }
                    for (int c = 0; c < nch; c++) {
                        const uint32_t b = sh.pre[c], e = c + 1 < nch ? sh.pre[c + 1] : n_cand;
                        if (e - b <= (uint32_t)a.cand_cap) continue;
                        const int64_t r0 = (int64_t)c * a.chunk;
                        const int64_t r1 = r0 + a.chunk < rows ? r0 + a.chunk : rows;
                        as_compact(s, vec, r0, r1, b1, b, e, sh);
                    }
                }
            }
        }
        __syncthreads();
        const uint32_t pre2 = (b1 << 10) | b2;
        const uint32_t need3 = keep - above1 - above2;
        // thread t takes candidates [per t, per (t + 1)), in row order (per
        // a multiple of 2 and <= 48, so that its candidates fit 64-bit
        // masks; read two at a time).  One pass over them settles all but
        // the candidates of bucket (b1, b2): those above its two-digit
        // prefix are kept (gtm), those below dropped; the bucket's go to
        // the third-digit histogram and are marked (unc) for a second look
        // once the threshold is known.
        const uint32_t per = ((n_cand + 255) / 256 + 1) & ~1u;
        const uint32_t i0 = per * tid, i1 = i0 + per < n_cand ? i0 + per : n_cand;
        uint64_t gtm = 0, unc = 0;
        if (in_lds) {
#pragma unroll 4
            for (uint32_t i = i0; i < i1; i += 2) {
                const u32x4 x = *reinterpret_cast<const u32x4 *>(&sh.kr[i]);
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const uint32_t k = x[2 * h + 1];
                    const bool in = i + h < i1;
                    const uint64_t bit = 1ull << (i + h - i0);
                    gtm |= in && (k >> 10) > pre2 ? bit : 0ull;
                    if (in && (k >> 10) == pre2) {
                        unc |= bit;
                        atomicAdd(&sh.h3[k & 1023], 1u);
                    }
                }
            }
        } else {
            as_hist_pass(s, vec, rows, 10, pre2, 0, 1024, sh.h3);
        }
        __syncthreads();
        uint32_t above3;
        const uint32_t b3 = find_bucket<1024>(sh.h3, need3, sh.scan, sh.res, above3);
        const uint32_t thr = (pre2 << 10) | b3;
        const uint32_t m_eq = need3 - above3;         // rows equal to thr kept, lowest rows first

        if (in_lds) {
            // the bucket's candidates against the threshold
            uint64_t eqm = 0;
            for (uint64_t u = unc; u; u &= u - 1ull) {
                const uint32_t bi = (uint32_t)__builtin_ctzll(u);
                const uint32_t k = (uint32_t)(sh.kr[i0 + bi] >> 32);
                gtm |= k > thr ? 1ull << bi : 0ull;
                eqm |= k == thr ? 1ull << bi : 0ull;
            }
            // one scan of both counts (each total < 2^16): the rows at the
            // threshold before this thread's, and the rows above it
            const uint32_t n_gt = (uint32_t)__builtin_popcountll(gtm), n_eq = (uint32_t)__builtin_popcountll(eqm);
            uint32_t tot;
            const uint32_t pk = block_excl_scan((n_eq << 16) | n_gt, sh.scan, tot);
            const uint32_t gt_before = pk & 0xFFFFu, eq_before = pk >> 16;
            // the lowest rows at the threshold are kept, m_eq of them in all
            const uint32_t eq_keep = eq_before >= m_eq ? 0u : (m_eq - eq_before < n_eq ? m_eq - eq_before : n_eq);
            uint64_t take = gtm;
            {
                uint64_t e = eqm;
                for (uint32_t j = 0; j < eq_keep; j++) {
                    const uint64_t low = e & (~e + 1ull);
                    take |= low;
                    e ^= low;
                }
            }
            // kept rows before this thread's: its first position
            sh.epos[tid] = gt_before + (eq_before < m_eq ? eq_before : m_eq);
            sh.etake[tid] = take;
            __syncthreads();
            // each token position of the split below the kept pools: the
            // thread owning its kept row (the last whose first position is
            // not past it), then the row's set bit in that thread's mask
            const int32_t lim = split_end < (int32_t)keep * kp ? split_end : (int32_t)keep * kp;
            for (int32_t P = start + tid; P < lim; P += 256) {
                const uint32_t j = kp == 1 ? (uint32_t)P : (uint32_t)P / (uint32_t)kp;
                int t = 0;
#pragma unroll
                for (int st = 128; st > 0; st >>= 1)
                    if (sh.epos[t + st] <= j) t += st;
                uint32_t k = j - sh.epos[t];
                const uint64_t m = sh.etake[t];
                uint32_t w32 = (uint32_t)m, bit = 0;
                const uint32_t c32 = (uint32_t)__builtin_popcount(w32);
                if (k >= c32) {
                    k -= c32;
                    w32 = (uint32_t)(m >> 32);
                    bit = 32;
                }
#pragma unroll
                for (int half = 16; half > 0; half >>= 1) {
                    const uint32_t c = (uint32_t)__builtin_popcount(w32 & ((1u << half) - 1u));
                    if (k >= c) {
                        k -= c;
                        w32 >>= half;
                        bit += half;
                    }
                }
                const int32_t r = (int32_t)(uint32_t)sh.kr[per * (uint32_t)t + bit];
                sidx[P - start] = kp == 1 ? r : r * kp + (int32_t)((uint32_t)P - j * (uint32_t)kp);
            }
        } else {
            uint32_t eq_done = 0, out_done = 0;
            for (int64_t sb = 0; sb < rows; sb += kAsTile) {
                const int64_t rb = sb + kAsPer * tid;
                float v[kAsPer];
                load_scores<kAsPer>(s, rb, rows, vec, v);
                uint32_t gtm = 0, eqm = 0;
#pragma unroll
                for (int i = 0; i < kAsPer; i++) {
                    const uint32_t k = order_key(v[i]);
                    if (rb + i < rows) {
                        gtm |= (k > thr ? 1u : 0u) << i;
                        eqm |= (k == thr ? 1u : 0u) << i;
                    }
                }
                uint32_t tot;
                uint32_t r = eq_done + block_excl_scan(__builtin_popcount(eqm), sh.scan, tot);
                eq_done += tot;
                uint32_t take = gtm;
#pragma unroll
                for (int i = 0; i < kAsPer; i++) {
                    if ((eqm >> i) & 1) {
                        if (r < m_eq) take |= 1u << i;
                        r++;
                    }
                }
                uint32_t p = out_done + block_excl_scan(__builtin_popcount(take), sh.scan, tot);
                out_done += tot;
#pragma unroll
                for (int i = 0; i < kAsPer; i++)
                    if ((take >> i) & 1) emit(p++, (int32_t)(rb + i));
            }
        }
        pooled = a.keep * kp;
        tail = qi.nvis - (int32_t)rows * kp;
        count = pooled + tail;
    } else if (qi.mode == 0) {
        count = qi.nvis;
    }
    // positions not taken by kept pools: the unpooled tail, the dense
    // selection, or padding
    for (int32_t P = start + tid; P < split_end; P += 256) {
        if (P < pooled) continue;
        int32_t tok = -1;
        if (qi.mode == 1)
            tok = P - pooled < tail ? (int32_t)qi.rows * kp + (P - pooled) : -1;
        else if (qi.mode == 0)
            tok = P < count ? P : -1;
        sidx[P - start] = tok;
    }
    if (write_sel && sp == 0 && tid == 0) a.sel_count[q] = count;
    return count;
}

// The split's part of the exported selection, copied from sidx once it is
// complete (coalesced, every thread), then the padding after the last split.
__device__ __forceinline__ void as_export(const Args &a, const int32_t *sidx, int q, int sp) {
    int32_t *dst = a.sel + (size_t)q * a.sel_ld;
    const int32_t start = sp * a.split_rows;
    int32_t end = start + a.split_rows;
    end = end < a.sel_ld ? end : a.sel_ld;
    for (int32_t P = start + (int32_t)threadIdx.x; P < end; P += 256) dst[P] = sidx[P - start];
    if (sp == a.n_split - 1)
        for (int32_t P = start + a.split_rows + (int32_t)threadIdx.x; P < a.sel_ld; P += 256) dst[P] = -1;
}

// grid (4 * pairs rounded up to 8), 256 threads, as k_attend_wv; SCAN: the
// queries' rows fit the one-pass selection (no k_filter ran).
template <int D, bool SCAN>
__global__ __launch_bounds__(256) void k_attend_sel(Args a) {
    using Cfg = WvCfg<D>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * Cfg::WAVE];
    __shared__ int32_t sidx[kWvMaxRows];
    __shared__ float smx[4][16], ssum[4][16];
    const int pairs = a.n_q * a.n_split;
    const int pairs8 = (pairs + 7) & ~7;
    const int hg = blockIdx.x / pairs8, pair = blockIdx.x % pairs8;
    if (pair >= pairs) return;
    const int q = pair / a.n_split, sp = pair % a.n_split;
    AsPre pre;
    if (!SCAN) {
        as_preload(a, q, pre);
    } else {
        // the one-pass top-k takes its first digit from the scorer's
        // histogram (k_reduce clears it after this kernel), and the first
        // kAsTile scores (rows 16 t .. 16 t + 15; read up to the score
        // row's length, rows past the query's own are not used) go to
        // registers too
        if (a.hist_on) {
            const uint32_t *gh = a.hist + (size_t)q * kHistStride + (kHistBins - 16 * (threadIdx.x + 1));
#pragma unroll
            for (int j = 0; j < 4; j++) pre.sv[j] = *(const u32x4 *)(gh + 4 * j);
        }
        const float *sq = a.scores_in + (size_t)q * a.score_ld;
        float v[kAsPer];
        load_scores<kAsPer>(sq, kAsPer * threadIdx.x, a.score_ld < kAsTile ? a.score_ld : kAsTile,
                            (reinterpret_cast<uintptr_t>(sq) & 15) == 0, v);
#pragma unroll
        for (int i = 0; i < kAsPer; i++) pre.sv[4 + (i >> 2)][i & 3] = __float_as_uint(v[i]);
    }
    const QInfo qi = query_info(a, q);
    const int lane = lane_id(), g = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int head = 16 * hg + n;
    bf16x8 qreg[Cfg::ND];
    // the queries are requested once the selection's own first loads are
    // on their way
    const uint16_t *qp = a.q + ((size_t)q * kHeads + head) * D + 8 * g;
    auto issue_q = [&qreg, qp] {
#pragma unroll
        for (int j = 0; j < Cfg::ND; j++) qreg[j] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qp + 32 * j));
    };
    if (!SCAN) {
        // k_filter has read the query's first-digit histogram: this
        // work-group clears its slice of it for the next call.  (The
        // second-digit histogram that follows it is read here by every
        // work-group of the query; the next call's scorer clears it.)
        const int slices = 4 * a.n_split, slice = 4 * sp + hg;
        const int per = (kHistBins + slices - 1) / slices;
        uint32_t *gh = a.hist + (size_t)q * kHistStride;
        for (int i = slice * per + threadIdx.x; i < (slice + 1) * per && i < kHistBins; i += 256) gh[i] = 0;
    }
    // a position the selection leaves unset (only possible where the
    // workspace's histograms do not match the scores) reads as no row
    for (int r = threadIdx.x; r < a.split_rows; r += 256) sidx[r] = -1;
    AsShared &sh = *reinterpret_cast<AsShared *>(lds);
    const int32_t count = as_select<SCAN>(a, sh, sidx, q, qi, sp, a.sel_export && hg == 0, issue_q, pre);
    const bool invalid = qi.mode == 2;
    const int32_t start = sp * a.split_rows;
    const int32_t nrows = count > start ? (count - start < a.split_rows ? count - start : a.split_rows) : 0;
    const int nst = (nrows + kWvRows - 1) / kWvRows;
    const int nj = nst > w ? (nst - w + 3) / 4 : 0;
    const uint8_t *C = reinterpret_cast<const uint8_t *>(a.cache + (size_t)(invalid ? 0 : qi.seq) * a.cache_stride * D);
    __syncthreads();   // sidx complete, and the selection's LDS (the row buffers) no longer read
    if (a.sel_export && hg == 0) as_export(a, sidx, q, sp);
    wv_rows<D>(a, lds, sidx, smx, ssum, qreg, C, q, sp, hg, w, nj, invalid);
}

// Merge the splits of each (query, head): grid (64, n_q), 128 threads, each
// thread four output columns.  Up to MB splits are loaded in one round trip
// and merged online (running max, rescaled sums).  MB = 32 serves 17 to 32
// splits (a k-pool query's 16 splits and its tail) in one round trip.
template <int MB>
__global__ __launch_bounds__(128) void k_reduce(Args a) {
    const int q = blockIdx.y, h = blockIdx.x, lane = lane_id();
    // the fused step's one-pass top-k read the query's first-digit histogram
    // from the scorer in the kernel before: work-group h clears bins
    // 64 h .. 64 h + 63 of it for the next call
    if (a.attn_sel && a.select_scan && a.hist_on && threadIdx.x < kHistBins / kHeads)
        a.hist[(size_t)q * kHistStride + (kHistBins / kHeads) * h + threadIdx.x] = 0;
    const size_t slot0 = (size_t)q * a.n_split * kHeads + h;
    float M = -INFINITY, L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.n_split; s0 += MB) {
        const int nb = a.n_split - s0 < MB ? a.n_split - s0 : MB;
        // every load of the round in flight before any use: lane i < nb
        // reads split s0 + i's (max, sum) (a vector load, so that no
        // scalar-load wait sits between them), every thread its four
        // columns of each split's partial
        float2 ml = {-INFINITY, 0.f};
        if (lane < nb) ml = *(const float2 *)(a.pml + 2 * (slot0 + (size_t)(s0 + lane) * kHeads));
        f32x4 v[MB];
#pragma unroll
        for (int i = 0; i < MB; i++)
            v[i] = i < nb ? *(const f32x4 *)(a.pacc + (slot0 + (size_t)(s0 + i) * kHeads) * kLatent + 4 * threadIdx.x)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
        float m[MB], l[MB];
#pragma unroll
        for (int i = 0; i < MB; i++) {
            m[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ml.x), i));
            l[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ml.y), i));
        }
        float Mn = M;
#pragma unroll
        for (int i = 0; i < MB; i++) Mn = fmaxf(Mn, m[i]);
        if (Mn == -INFINITY) continue;
        const float fo = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
        L *= fo;
        o *= fo;
#pragma unroll
        for (int i = 0; i < MB; i++) {
            const float f = m[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[i] - Mn);
            L += l[i] * f;
            o += v[i] * f;
        }
        M = Mn;
    }
    const QInfo qi = query_info(a, q);
    const bool bad = qi.mode == 2 || L == 0.f;
    o = bad ? f32x4{NAN, NAN, NAN, NAN} : o * (1.f / L);
    *(f32x4 *)(a.out + ((size_t)q * kHeads + h) * kLatent + 4 * threadIdx.x) = o;
    if (a.lse && threadIdx.x == 0)
        a.lse[(size_t)q * kHeads + h] = bad ? NAN : (M + __log2f(L)) * 0.69314718055994531f;
}

// ---------------------------------------------------------------- pool keys
// k-pool key producer ("GLM-5.3-Flash on WASTE", "DeepSeek Sparse Attention,
// k-pool flavour": one 128-wide key per pool of four tokens, computed when
// the pool's last token arrives, beside a rolling buffer of the pool being
// filled; TensorSharp2 "GLM-5.3-Flash (glm5next)": [key|gate] per cell, a
// softmax over the gates plus a per-slot position embedding compresses the
// pool).  Per key dimension d:
//   K[d] = sum_j softmax_j(gate_j[d] + E[j][d]) * key_j[d],  j over the 4 slots,
// in fp32, stored as bf16 rounded to nearest even.
// grid (ceil(pools per call / 4), n_seq), 256 threads: wave w of block b
// compresses pool n_tok / 4 + 4 b + w of its sequence if the call completes
// it; lane l takes dimensions 2l and 2l + 1.  Block 0 then moves the cells of
// the pool left incomplete into the rolling buffer (its wave 0 is the only
// reader of that buffer, so the barrier orders the reads before the writes).
constexpr int kCell = 2 * kIdxDim;   // bf16 per cell: key, then gate

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__global__ __launch_bounds__(256) void k_pool_append(PoolArgs a) {
    const int s = blockIdx.y, w = threadIdx.x >> 6, lane = lane_id();
    const int64_t n_tok = a.n_tok[s], n_new = a.n_new[s];
    if (n_tok < 0 || n_new < 0 || n_new > a.max_new) return;
    const int64_t end = n_tok + n_new;
    const int64_t p0 = n_tok / 4, p1 = end / 4;     // pools [p0, p1) complete after the call
    const uint16_t *roll = a.rolling + (size_t)s * 4 * kCell;
    const uint16_t *nk = a.new_kg + (size_t)s * a.new_stride * kCell;
    const int64_t p = p0 + 4 * (int64_t)blockIdx.x + w;
    if (p < p1 && p < a.pool_stride) {
        float key[4][2], lg[4][2];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int64_t t = 4 * p + j;
            const uint16_t *c = t < n_tok ? roll + j * kCell : nk + (t - n_tok) * kCell;
            const uint32_t kv = *(const uint32_t *)(c + 2 * lane);
            const uint32_t gv = *(const uint32_t *)(c + kIdxDim + 2 * lane);
            key[j][0] = __uint_as_float(kv << 16);
            key[j][1] = __uint_as_float(kv & 0xFFFF0000u);
            lg[j][0] = __uint_as_float(gv << 16) + a.pos_emb[j * kIdxDim + 2 * lane];
            lg[j][1] = __uint_as_float(gv & 0xFFFF0000u) + a.pos_emb[j * kIdxDim + 2 * lane + 1];
        }
        uint32_t packed = 0;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const float m = fmaxf(fmaxf(lg[0][h], lg[1][h]), fmaxf(lg[2][h], lg[3][h]));
            float num = 0.f, den = 0.f;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float e = __builtin_amdgcn_exp2f((lg[j][h] - m) * 1.4426950408889634f);
                num += e * key[j][h];
                den += e;
            }
            packed |= (uint32_t)bf16_rne(num / den) << (16 * h);
        }
        *(uint32_t *)(a.pool_keys + ((size_t)s * a.pool_stride + p) * kIdxDim + 2 * lane) = packed;
    }
    if (blockIdx.x != 0) return;
    __syncthreads();
    // cells of the incomplete pool that arrived in this call
    uint16_t *rw = a.rolling + (size_t)s * 4 * kCell;
    for (int64_t t = (4 * p1 > n_tok ? 4 * p1 : n_tok) + w; t < end; t += 4) {
        const uint32_t *src = (const uint32_t *)(nk + (t - n_tok) * kCell);
        uint32_t *dst = (uint32_t *)(rw + (t % 4) * kCell);
        dst[lane] = src[lane];
        dst[64 + lane] = src[64 + lane];
    }
}

// ---------------------------------------------------------------- absorption
// The per-head key and value up-projections on either side of the attention
// ("GLM 5.2 in pure C", "Attention: Multi head Latent Attention With a Tiny
// KV Cache": the query absorbs the key up-projection once and the pooled
// latent is projected back out per head; TensorSharp2 "The block"):
//   q_abs[m][h][n] = bf16( sum_k q_nope[m][h][k] W_UK[h][k][n] ),  n < 512, then q_rope
//   ctx[m][h][i]   = sum_j o[m][h][j] W_UV[h][i][j],                i < 256
// Both as C^T = W' X^T on MFMA 16x16x32 bf16: A = 16 weight rows (output
// features) x 32 k; B = 16 queries x 32 k, loaded directly (k contiguous);
// D lands as 4 consecutive features of one query per lane.  A work-group
// owns 64 output features of one head (four 16-feature tiles) and a chunk of
// up to kAbsorbRows queries.  With four or more 16-query blocks, wave w takes
// blocks w, w + 4, ... and all four tiles, so every query row is read once
// per work-group; with fewer, wave w takes tile w of every block.
constexpr int kNope = 256;   // q_nope width per head
constexpr int kVdim = 256;   // value width per head (output of the projection)
constexpr int kAbsorbRows = 256;  // queries per work-group (the grid spreads the rest)

// Work-group -> (output slice, head, query chunk) over a 1-D grid of
// S x 64 x C work-groups.  Work-groups are dealt to the eight XCDs in turn,
// so XCD x takes heads x, x + 8, ..., and the S x C work-groups of one head
// run side by side there and share the head's weights and activations in
// that XCD's L2 instead of each fetching them from HBM.
struct AbsTile {
    int slice, head, chunk;
};
__device__ __forceinline__ AbsTile abs_tile(int S, int C) {
    const int L = blockIdx.x, x = L & 7, j = L >> 3, per = S * C;
    const int hi = j / per, rem = j - hi * per;
    return {rem % S, x + 8 * hi, rem / S};
}

// grid 8 slices of 64 latent dimensions x 64 heads x query chunks (abs_tile),
// 256 threads.  W_UK[h] rows are latent-contiguous, so the slice is staged in
// LDS (row stride 144 B) and read transposed with ds_read_b64_tr_b16 for
// every query block.
__global__ __launch_bounds__(256) void k_absorb(AbsorbArgs a) {
    constexpr int RS = 144;
    constexpr int KS = kNope / 32;
    __shared__ __attribute__((aligned(16))) uint8_t wl[kNope * RS];
    const AbsTile tl = abs_tile(kLatent / 64, (a.n_q + kAbsorbRows - 1) / kAbsorbRows);
    const int h = tl.head, n0 = 64 * tl.slice;
    const int lane = lane_id(), w = threadIdx.x >> 6, g = lane >> 4, n = lane & 15;
    const int m_begin = kAbsorbRows * tl.chunk;
    const int m_end = m_begin + kAbsorbRows < a.n_q ? m_begin + kAbsorbRows : a.n_q;
    const bool by_tile = m_end - m_begin <= 48;        // fewer than four 16-query blocks
    const int mb0 = by_tile ? m_begin : m_begin + 16 * w, mstep = by_tile ? 16 : 64;
    // this lane's query row of a 16-query block, k = 32 ks + 8 g .. + 7
    auto load_q = [&](int m0, bf16x8 (&bq)[KS]) {
        const int m = m0 + n;
        const uint16_t *qn = a.q_nope + ((size_t)(m < m_end ? m : m_begin) * kHeads + h) * kNope + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) bq[ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qn + 32 * ks));
    };
    bf16x8 bq[KS];
    if (mb0 < m_end) load_q(mb0, bq);          // in flight while the weights are staged
    {
        const uint8_t *W = reinterpret_cast<const uint8_t *>(a.w_uk + (size_t)h * kNope * kLatent + n0);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int e = threadIdx.x + 256 * i, r = e >> 3, pc = e & 7;
            *(u32x4 *)(wl + r * RS + 16 * pc) = *(const u32x4 *)(W + (size_t)r * kLatent * 2 + 16 * pc);
        }
    }
    __syncthreads();
    // A operand of tile t, k-step ks, read transposed from the staged slice
    auto wtile = [&](int t, int ks) {
        const int r_in = n >> 2, c_in = n & 3;
        const uint8_t *p1 = wl + (32 * ks + 8 * g + r_in) * RS + (16 * t + 4 * c_in) * 2;
        const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p1);
        const i16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p1 + 4 * RS));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 tv = {t1[0], t1[1], t1[2], t1[3], t2[0], t2[1], t2[2], t2[3]};
        return __builtin_bit_cast(bf16x8, tv);
    };
    const int D = kLatent + a.d_rope;
    auto block = [&](int m0, const bf16x8 (&b)[KS]) {
        const int m = m0 + n;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            if (by_tile && t != w) continue;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ks++) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wtile(t, ks), b[ks], acc, 0, 0, 0);
            if (m < m_end) {
                const uint32_t lo = (uint32_t)bf16_rne(acc[0]) | ((uint32_t)bf16_rne(acc[1]) << 16);
                const uint32_t hi = (uint32_t)bf16_rne(acc[2]) | ((uint32_t)bf16_rne(acc[3]) << 16);
                uint16_t *dst = a.q_abs + ((size_t)m * kHeads + h) * D + n0 + 16 * t + 4 * g;
                *(uint2 *)dst = make_uint2(lo, hi);
            }
        }
    };
    // two query blocks per trip, each one's operands loaded a block ahead
    bf16x8 bq2[KS];
    for (int m0 = mb0; m0 < m_end; m0 += 2 * mstep) {
        // keeps the weight reads inside the loop: hoisted, they would take
        // 128 registers and halve the waves per SIMD
        asm volatile("" ::: "memory");
        if (m0 + mstep < m_end) load_q(m0 + mstep, bq2);
        block(m0, bq);
        if (m0 + mstep >= m_end) break;
        if (m0 + 2 * mstep < m_end) load_q(m0 + 2 * mstep, bq);
        block(m0 + mstep, bq2);
    }
    // the RoPE part, appended unchanged
    if (tl.slice == 0 && a.d_rope > 0) {
        for (int e = threadIdx.x; e < (m_end - m_begin) * (a.d_rope / 8); e += 256) {
            const int m = m_begin + e / (a.d_rope / 8), pc = e % (a.d_rope / 8);
            *(u32x4 *)(a.q_abs + ((size_t)m * kHeads + h) * D + kLatent + 8 * pc) =
                *(const u32x4 *)(a.q_rope + ((size_t)m * kHeads + h) * a.d_rope + 8 * pc);
        }
    }
}

// grid 4 slices of 64 value dimensions x 64 heads x query chunks (abs_tile),
// 256 threads.  W_UV[h] rows are k-contiguous: the slice's 64 rows (64 KiB)
// are staged in LDS (row stride 1,040 B, so the 16-byte A-operand reads of
// eight rows at a time fall in distinct banks) and read per k-step.  o
// (fp32) enters the MFMA as bf16 hi + lo (the truncated value and the
// rounded remainder, ~16 bits); a block's o rows are loaded in two halves of
// k, the first half computed while the second is in flight (two work-groups
// per CU hide the rest).
__global__ __launch_bounds__(256) void k_project(AbsorbArgs a) {
    constexpr int RS = kLatent * 2 + 16;
    constexpr int KS = kLatent / 32, KH = KS / 2;
    __shared__ __attribute__((aligned(16))) uint8_t wl[64 * RS];
    const AbsTile tl = abs_tile(kVdim / 64, (a.n_q + kAbsorbRows - 1) / kAbsorbRows);
    const int h = tl.head, i0 = 64 * tl.slice;
    const int lane = lane_id(), w = threadIdx.x >> 6, g = lane >> 4, n = lane & 15;
    const int m_begin = kAbsorbRows * tl.chunk;
    const int m_end = m_begin + kAbsorbRows < a.n_q ? m_begin + kAbsorbRows : a.n_q;
    const bool by_tile = m_end - m_begin <= 48;
    const int mb0 = by_tile ? m_begin : m_begin + 16 * w, mstep = by_tile ? 16 : 64;
    // half hf of this lane's o row in a 16-query block: k = 32 ks + 8 g .. + 7
    // for ks in [KH hf, KH hf + KH)
    auto load_o = [&](int m0, int hf, f32x4 (&x)[2 * KH]) {
        const int m = m0 + n;
        const float *op = a.o + ((size_t)(m < m_end ? m : m_begin) * kHeads + h) * kLatent + 8 * g + 32 * KH * hf;
#pragma unroll
        for (int ks = 0; ks < KH; ks++) {
            x[2 * ks] = *(const f32x4 *)(op + 32 * ks);
            x[2 * ks + 1] = *(const f32x4 *)(op + 32 * ks + 4);
        }
    };
    {
        const uint8_t *W = reinterpret_cast<const uint8_t *>(a.w_uv + ((size_t)h * kVdim + i0) * kLatent);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int e = threadIdx.x + 256 * i, r = e >> 6, pc = e & 63;
            *(u32x4 *)(wl + r * RS + 16 * pc) = *(const u32x4 *)(W + (size_t)r * kLatent * 2 + 16 * pc);
        }
    }
    __syncthreads();
    // one tile per wave (ONE: tile w) or all four; a lane past m_end reads
    // a valid row and stores nothing
    auto run = [&](auto one_tile) {
        constexpr bool ONE = decltype(one_tile)::value;
        constexpr int NT = ONE ? 1 : 4;
        const int tb = ONE ? w : 0;
        for (int m0 = mb0; m0 < m_end; m0 += mstep) {
            // keeps the weight reads inside the loop: hoisted, the 64 KiB
            // slice would take 256 registers and leave one wave per SIMD
            asm volatile("" ::: "memory");
            f32x4 xa[2 * KH], xb[2 * KH];
            load_o(m0, 0, xa);
            load_o(m0, 1, xb);
            f32x4 acc[NT];
#pragma unroll
            for (int tt = 0; tt < NT; tt++) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            auto half = [&](int hf, const f32x4 (&x)[2 * KH]) {
#pragma unroll
                for (int ks = 0; ks < KH; ks++) {
                    bf16x8 bh, bl;
#pragma unroll
                    for (int j = 0; j < 8; j++) {
                        const float v = j < 4 ? x[2 * ks][j] : x[2 * ks + 1][j - 4];
                        const uint32_t hb = __float_as_uint(v) & 0xFFFF0000u;
                        bh[j] = __builtin_bit_cast(__bf16, (uint16_t)(hb >> 16));
                        bl[j] = (__bf16)(v - __uint_as_float(hb));     // exact difference, rounded to nearest even
                    }
                    const int kk = KH * hf + ks;
#pragma unroll
                    for (int tt = 0; tt < NT; tt++) {
                        const bf16x8 wa = __builtin_bit_cast(
                            bf16x8, *(const u32x4 *)(wl + (16 * (tb + tt) + n) * RS + 64 * kk + 16 * g));
                        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, bh, acc[tt], 0, 0, 0);
                        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, bl, acc[tt], 0, 0, 0);
                    }
                }
            };
            half(0, xa);
            half(1, xb);
            const int m = m0 + n;
            if (m < m_end) {
#pragma unroll
                for (int tt = 0; tt < NT; tt++)
                    *(f32x4 *)(a.ctx + ((size_t)m * kHeads + h) * kVdim + i0 + 16 * (tb + tt) + 4 * g) = acc[tt];
            }
        }
    };
    if (by_tile)
        run(std::true_type{});
    else
        run(std::false_type{});
}

// ---------------------------------------------------------------- launchers
// A launch that, given events, takes them as its own start and stop marks
// (hipExtLaunchKernel stamps them from the dispatch itself, so their
// interval is the kernel's execution time, as a kernel trace reports it).
#define DSA_LAUNCH(EV0, EV1, KERNEL, GRID, BLOCK, ST, ...)                                    \
    do {                                                                                      \
        if ((EV0) || (EV1))                                                                   \
            hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, ST, EV0, EV1, 0, __VA_ARGS__);      \
        else                                                                                  \
            hipLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, ST, __VA_ARGS__);                      \
    } while (0)

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st) {
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    size_t blocks = (words + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, st, (uint32_t *)p, words);
    return hipGetLastError();
}

template <bool F16>
hipError_t launch_score_fmt(const Args &a, int64_t max_rows, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if (a.prefill) {
        const unsigned ranges = (unsigned)((max_rows + kPfRange - 1) / kPfRange);
        const unsigned runs = (unsigned)((a.n_q + a.pf_run - 1) / a.pf_run);
        const unsigned per = (unsigned)((a.pf_run + kPfQ - 1) / kPfQ);
        DSA_LAUNCH(ev0, nullptr, k_score_prefill<F16>, dim3(ranges, runs * per), dim3(kPfWaves * 64), st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // in prefill mode k_score only picks up queries outside their block's
    // sequence: one work-group per query, striding over the tiles
    if (a.prefill)
        DSA_LAUNCH(nullptr, ev1, (k_score<true, F16, 4>), dim3(1, a.n_q), dim3(256), st, a);
    else if (!F16 && a.score_valu)
        DSA_LAUNCH(ev0, ev1, k_score_valu, dim3((unsigned)((max_rows + 255) / 256), a.n_q), dim3(256), st, a);
    else if (a.score_waves == 8)
        DSA_LAUNCH(ev0, ev1, (k_score<false, F16, 8>),
                   dim3((unsigned)((max_rows + a.score_tile - 1) / a.score_tile), a.n_q), dim3(512), st, a);
    else
        DSA_LAUNCH(ev0, ev1, (k_score<false, F16, 4>),
                   dim3((unsigned)((max_rows + a.score_tile - 1) / a.score_tile), a.n_q), dim3(256), st, a);
    return hipGetLastError();
}

hipError_t launch_score(const Args &a, int64_t max_rows, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    return a.idx_f16 ? launch_score_fmt<true>(a, max_rows, st, ev0, ev1)
                     : launch_score_fmt<false>(a, max_rows, st, ev0, ev1);
}

hipError_t launch_hist(const Args &a, hipStream_t st) {
    hipLaunchKernelGGL(k_hist, dim3(a.n_chunks, a.n_q), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_filter(const Args &a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if (a.chunk >= 16384)
        DSA_LAUNCH(ev0, ev1, k_filter<16>, dim3(a.n_chunks, a.n_q), dim3(256), st, a);
    else
        DSA_LAUNCH(ev0, ev1, k_filter<8>, dim3(a.n_chunks, a.n_q), dim3(256), st, a);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st) {
    // 2,048 work-groups of 256 threads: 8 per CU, each wave a few loads in flight
    hipLaunchKernelGGL(k_stream_read, dim3(2048), dim3(256), 0, st, static_cast<const u32x4 *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_select(const Args &a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if (a.select_scan)
        DSA_LAUNCH(ev0, ev1, k_select<true>, dim3(a.n_q), dim3(kSelThreads), st, a);
    else
        DSA_LAUNCH(ev0, ev1, k_select<false>, dim3(a.n_q), dim3(kSelThreads), st, a);
    return hipGetLastError();
}

// The attention kernel takes ev[0] and ev[1], the split merge ev[2] and
// ev[3] (not recorded when there is no merge); ev may be NULL.
hipError_t launch_attend(const Args &a, hipStream_t st, const hipEvent_t *ev) {
    const hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
    if (a.attn_sel) {
        const unsigned pairs8 = (unsigned)((a.n_q * a.n_split + 7) & ~7);
        if (a.D == 576) {
            if (a.select_scan)
                DSA_LAUNCH(e0, e1, (k_attend_sel<576, true>), dim3(4 * pairs8), dim3(256), st, a);
            else
                DSA_LAUNCH(e0, e1, (k_attend_sel<576, false>), dim3(4 * pairs8), dim3(256), st, a);
        } else {
            if (a.select_scan)
                DSA_LAUNCH(e0, e1, (k_attend_sel<512, true>), dim3(4 * pairs8), dim3(256), st, a);
            else
                DSA_LAUNCH(e0, e1, (k_attend_sel<512, false>), dim3(4 * pairs8), dim3(256), st, a);
        }
    } else if (a.attn_hs == 2) {
        const unsigned pairs8 = (unsigned)((a.n_q * a.n_split + 7) & ~7);
        if (a.D == 576)
            DSA_LAUNCH(e0, e1, k_attend_wv<576>, dim3(4 * pairs8), dim3(256), st, a);
        else
            DSA_LAUNCH(e0, e1, k_attend_wv<512>, dim3(4 * pairs8), dim3(256), st, a);
    } else if (a.attn_hs) {
        const unsigned pairs8 = (unsigned)((a.n_q * a.n_split + 7) & ~7);
        if (a.D == 576)
            DSA_LAUNCH(e0, e1, k_attend_hs<576>, dim3(4 * pairs8), dim3(512), st, a);
        else
            DSA_LAUNCH(e0, e1, k_attend_hs<512>, dim3(4 * pairs8), dim3(512), st, a);
    } else if (a.D == 576) {
        DSA_LAUNCH(e0, e1, k_attend<576>, dim3(a.n_split, a.n_q), dim3(512), st, a);
    } else {
        DSA_LAUNCH(e0, e1, k_attend<512>, dim3(a.n_split, a.n_q), dim3(512), st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.n_split == 1) return e;
    if (a.n_split > 16 && a.n_split <= 32)
        DSA_LAUNCH(ev ? ev[2] : nullptr, ev ? ev[3] : nullptr, k_reduce<32>, dim3(kHeads, a.n_q), dim3(128), st, a);
    else
        DSA_LAUNCH(ev ? ev[2] : nullptr, ev ? ev[3] : nullptr, k_reduce<16>, dim3(kHeads, a.n_q), dim3(128), st, a);
    return hipGetLastError();
}

}  // namespace dsa

namespace dsa {
hipError_t launch_pool_append(const PoolArgs &a, hipStream_t st) {
    const int64_t pools = (a.max_new + 3) / 4;
    const unsigned gx = (unsigned)((pools + 3) / 4 > 0 ? (pools + 3) / 4 : 1);
    hipLaunchKernelGGL(k_pool_append, dim3(gx, a.n_seq), dim3(256), 0, st, a);
    return hipGetLastError();
}
}  // namespace dsa

namespace dsa {
hipError_t launch_absorb(const AbsorbArgs &a, hipStream_t st) {
    static_assert(kHeads == 64, "abs_tile deals 8 heads to each of 8 XCDs");
    hipLaunchKernelGGL(k_absorb, dim3(kLatent / 64 * kHeads * ((a.n_q + kAbsorbRows - 1) / kAbsorbRows)), dim3(256),
                       0, st, a);
    return hipGetLastError();
}
hipError_t launch_project(const AbsorbArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(k_project, dim3(kVdim / 64 * kHeads * ((a.n_q + kAbsorbRows - 1) / kAbsorbRows)), dim3(256), 0,
                       st, a);
    return hipGetLastError();
}
}  // namespace dsa

// ---------------------------------------------------------------- indexer input preparation
// Rope on the tail 64 dimensions, then the orthonormal Walsh-Hadamard
// rotation, then rounding to the indexer's 16-bit format, for the indexer
// queries of a step and for the keys it appends to the key cache.  A wave
// takes four 128-wide vectors side by side.  Vector s (lane bits 2-3) is
// spread over 16 lanes; its piece c (dimensions 8c .. 8c+7, two 16-byte
// loads and one 16-byte store) sits on lane (c & 3) | 4 s | 16 (c >> 2).
// Dimension bits 0-2 are inside the lane: three butterfly stages in
// registers.  Bits 3-4 are lane bits 0-1, whose partner comes by DPP within
// the quad; bits 5-6 are lane bits 4-5, whose pairs permlane16/32_swap hand
// over as (lower lane's value, upper lane's value), so each stage element is
// one multiply-add.  The rope slice is lanes 32-63; pair (64+2j, 65+2j)
// lies inside the lane holding piece 8 + j/4.  The (cos, sin) of every pair
// a wave needs is computed once into a per-wave LDS table: 32 entries when
// the four vectors are heads of one query (one position), 4 x 32 otherwise.
// Angles are formed and reduced modulo pi/2 in double (pair 0 turns by the
// position in radians, up to 2^31), and the reduced angle, at most pi/4,
// goes through Taylor polynomials in float (truncation below 2e-9).
namespace dsa {
constexpr int kPrepRows = 4;   // vectors per wave

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// (cos t, sin t) for t = pos * inv_freq radians
__device__ __forceinline__ float2 rope_cos_sin(int64_t pos, double inv_freq) {
    const double t = (double)pos * inv_freq;
    const double q = rint(t * 0.6366197723675814);                       // 2 / pi
    double rd = fma(-q, 1.5707963267948966, t);                           // pi / 2, high part
    rd = fma(-q, 6.123233995736766e-17, rd);                              // pi / 2, low part
    const float r = (float)rd, r2 = r * r;
    // sin r = r - r^3/3! + ... + r^9/9!,  cos r = 1 - r^2/2! + ... - r^10/10!
    float sp = 2.7557319e-6f;                                             // 1/9!
    sp = fmaf(sp, r2, -1.9841270e-4f);                                   // 1/7!
    sp = fmaf(sp, r2, 8.3333333e-3f);                                    // 1/5!
    sp = fmaf(sp, r2, -1.6666667e-1f);                                   // 1/3!
    const float sr = fmaf(sp * r2, r, r);
    float cp = -2.7557319e-7f;                                            // 1/10!
    cp = fmaf(cp, r2, 2.4801587e-5f);                                    // 1/8!
    cp = fmaf(cp, r2, -1.3888889e-3f);                                   // 1/6!
    cp = fmaf(cp, r2, 4.1666667e-2f);                                    // 1/4!
    cp = fmaf(cp, r2, -0.5f);
    const float cr = fmaf(cp, r2, 1.f);
    const int n = (int)((int64_t)q & 3);                                  // quadrant
    const float c = (n & 1) ? sr : cr, s_ = (n & 1) ? cr : sr;
    return make_float2((n == 1 || n == 2) ? -c : c, (n >= 2) ? -s_ : s_);
}

__global__ __launch_bounds__(256) void k_index_prep(PrepArgs a) {
    __shared__ float2 tab[4][kPrepRows][32];       // per wave: (cos, sin) of (vector, pair)
    const int lane = lane_id(), w = threadIdx.x >> 6;
    const int sv = (lane >> 2) & 3;                 // vector of the wave
    const int c = (lane & 3) | ((lane >> 4) << 2);  // piece of the vector
    const int64_t n_qv = (int64_t)a.n_q * kIdxHeads;
    const int64_t total = n_qv + a.n_new;
    const int64_t v0 = ((int64_t)blockIdx.x * 4 + w) * kPrepRows;
    if (v0 >= total) return;
    const int64_t v = v0 + sv;

    const float *src = nullptr;
    uint16_t *dst = nullptr;
    int64_t pos = 0;
    if (v < n_qv) {
        pos = (int64_t)a.q_nvis[v / kIdxHeads] - 1;
        src = a.q_in + v * kIdxDim;
        dst = a.q_out + v * kIdxDim;
    } else if (v < total) {
        // the key's own row is read before its destination is known
        const int64_t k = v - n_qv;
        src = a.k_in + k * kIdxDim;
        const int64_t seq = a.k_seq ? a.k_seq[k] : k;
        const int64_t p = a.k_pos[k];
        pos = p;
        if (seq >= 0 && seq < a.n_seq && p >= 0 && p < a.key_stride)
            dst = a.k_cache + (seq * a.key_stride + p) * kIdxDim;
    }
    f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
    if (src) {
        x0 = __builtin_nontemporal_load((const f32x4 *)(src + 8 * c));
        x1 = __builtin_nontemporal_load((const f32x4 *)(src + 8 * c + 4));
    }
    float e[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};

    if (a.rope) {
        // the four vectors' positions (piece 0 of vector r is lane 4 r), and
        // the frequency of pair j = lane & 31: the host's base^(-4i/32) for
        // i = j/4, times base^(-1/32) per further step
        int64_t pv[kPrepRows];
#pragma unroll
        for (int r = 0; r < kPrepRows; r++) {
            const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)pos, 4 * r);
            const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)pos >> 32), 4 * r);
            pv[r] = (int64_t)(((uint64_t)hi << 32) | lo);
        }
        const int j = lane & 31;
        double inv_freq = a.inv_freq[0];
#pragma unroll
        for (int i = 1; i < 8; i++) inv_freq = (j >> 2) == i ? a.inv_freq[i] : inv_freq;
#pragma unroll
        for (int m = 1; m < 4; m++) inv_freq = (j & 3) >= m ? inv_freq * a.freq_ratio : inv_freq;
        const bool one_pos = v0 + kPrepRows <= n_qv;   // four heads of one query
        if (one_pos) {
            if (lane < 32) tab[w][0][j] = rope_cos_sin(pv[0], inv_freq);
        } else {
            const int r0 = lane >> 5;
            tab[w][r0][j] = rope_cos_sin(r0 ? pv[1] : pv[0], inv_freq);
            tab[w][r0 + 2][j] = rope_cos_sin(r0 ? pv[3] : pv[2], inv_freq);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        if (lane >= 32) {
            const float2 *cs = &tab[w][one_pos ? 0 : sv][4 * (c - 8)];
#pragma unroll
            for (int m = 0; m < 4; m++) {
                const float2 t = cs[m];
                const float a0 = e[2 * m], b0 = e[2 * m + 1];
                e[2 * m] = a0 * t.x - b0 * t.y;
                e[2 * m + 1] = a0 * t.y + b0 * t.x;
            }
        }
    }
    // dimension bits 0-2: inside the lane
#pragma unroll
    for (int b = 1; b < 8; b <<= 1) {
#pragma unroll
        for (int k = 0; k < 8; k++) {
            if (k & b) continue;
            const float lo = e[k], hi = e[k | b];
            e[k] = lo + hi;
            e[k | b] = lo - hi;
        }
    }
    // bits 3-4: lane bits 0-1, partner by DPP (lower: own + partner, upper:
    // partner - own)
    const float s0 = (lane & 1) ? -1.f : 1.f, s1 = (lane & 2) ? -1.f : 1.f;
#pragma unroll
    for (int k = 0; k < 8; k++) e[k] = s0 * e[k] + dpp_mov<0xB1>(e[k]);      // quad_perm [1,0,3,2]
#pragma unroll
    for (int k = 0; k < 8; k++) e[k] = s1 * e[k] + dpp_mov<0x4E>(e[k]);      // quad_perm [2,3,0,1]
    // bits 5-6: lane bits 4-5; the swap gives (lower lane's, upper lane's)
    const float s4 = (lane & 16) ? -1.f : 1.f, s5 = (lane & 32) ? -1.f : 1.f;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const u32x2 p = __builtin_amdgcn_permlane16_swap(__float_as_uint(e[k]), __float_as_uint(e[k]), false, false);
        e[k] = fmaf(s4, __uint_as_float(p[1]), __uint_as_float(p[0]));
    }
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const u32x2 p = __builtin_amdgcn_permlane32_swap(__float_as_uint(e[k]), __float_as_uint(e[k]), false, false);
        e[k] = fmaf(s5, __uint_as_float(p[1]), __uint_as_float(p[0]));
    }

    if (!dst) return;
    const float norm = 0.08838834764831845f;   // 1 / sqrt(128)
    u32x4 packed;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const float y0 = e[2 * k] * norm, y1 = e[2 * k + 1] * norm;
        if (a.f16)
            packed[k] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y0) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y1) << 16);
        else
            packed[k] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)y0) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)y1) << 16);
    }
    *(u32x4 *)(dst + 8 * c) = packed;
}

hipError_t launch_index_prep(const PrepArgs &a, hipStream_t st) {
    const int64_t total = (int64_t)a.n_q * kIdxHeads + a.n_new;
    const int64_t per_block = 4 * kPrepRows;
    const unsigned blocks = (unsigned)((total + per_block - 1) / per_block);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_index_prep, dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}
}  // namespace dsa

// ---------------------------------------------------------------- scratch of the allocation-free step
// The workspace of dsa_decode_step_noalloc: a file-scope device array that
// each GPU the library runs on holds from module load until the process
// ends.  In host code the name `scratch` is only a stand-in for the array,
// never its device address: host code uses the address hipGetSymbolAddress
// returns, looked up once per device with that device current and kept per
// device.  Only its histogram region (the first sixteenth) must start at
// zero; every call leaves it zero again, and the first use on a device (or
// the first after a failed launch) clears it with a fill kernel.
static __device__ __attribute__((aligned(256))) uint8_t scratch[dsa::kScratchBytes];

#include <mutex>

namespace dsa {
namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kScratchDevices];        // device address of each device's copy
bool g_scratch_clear[kScratchDevices];   // its histogram region is known to be zero
}  // namespace

hipError_t scratch_acquire(hipStream_t st, void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    if (!g_scratch_clear[dev]) {
        e = launch_fill_zero(g_scratch[dev], hist_region_bytes(kScratchBytes), st);
        if (e != hipSuccess) return e;
        g_scratch_clear[dev] = true;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

void scratch_mark_dirty() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    g_scratch_clear[dev] = false;
}
}  // namespace dsa
