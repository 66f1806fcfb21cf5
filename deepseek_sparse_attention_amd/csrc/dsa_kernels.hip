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
// query, issued on MFMA with the key rows streamed straight from HBM into the
// B operand; its epilogue applies ReLU and the head weights and feeds a
// 2048-bin histogram of the scores' order keys.  Top-k is an exact radix
// select: the histogram fixes the threshold bucket, one pass collects that
// bucket's candidates, the last work-group of each query resolves the exact
// threshold and each chunk's output offset, and a final pass emits indices
// in ascending order.  Attention gathers the selected rows into LDS, computes
// S^T = C Q^T on MFMA, keeps an online softmax in fp32, and computes
// O^T = V^T P^T on MFMA with V read through ds_read_b64_tr_b16 and P split
// into two bf16 halves (hi + lo) so that P carries ~16 mantissa bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <functional>

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

// Radix step: with hist[0..NB) of the items still in play and `need` of
// them still to take from the top, find the bin b holding the need-th
// largest: suffix(b) >= need > suffix(b+1).  Returns b, sets above =
// suffix(b+1).  256 threads; thread t owns the PER bins just below
// NB - PER*t, kept in registers.
template <int NB>
__device__ uint32_t find_bucket(const uint32_t *hist, uint32_t need, uint32_t *smem, uint32_t *res,
                                uint32_t &above) {
    constexpr int PER = NB / 256;
    const int hi = NB - PER * (int)threadIdx.x;
    uint32_t c[PER];
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) {
        c[i] = hist[hi - 1 - i];
        s += c[i];
    }
    uint32_t total;
    const uint32_t before = block_excl_scan(s, smem, total);   // items in higher bins
    if (before < need && before + s >= need) {
        uint32_t run = before, bin = 0, run_at = 0;
        bool found = false;
#pragma unroll
        for (int i = 0; i < PER; i++) {
            if (!found && run + c[i] >= need) {
                found = true;
                bin = (uint32_t)(hi - 1 - i);
                run_at = run;
            }
            run += c[i];
        }
        res[0] = bin;
        res[1] = run_at;
    }
    __syncthreads();
    above = res[1];
    const uint32_t b = res[0];
    __syncthreads();
    return b;
}

// ---------------------------------------------------------------- workspace
__global__ void k_fill_zero(uint32_t *p, size_t n_words) {
    size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n_words; i += stride) p[i] = 0u;
}

// ---------------------------------------------------------------- scores
// grid (tiles, n_q), 256 threads.  Wave w of a work-group takes 64-row
// steps t0 + 64 (w + 4 i).  Keys are read with fully coalesced 16-byte loads
// (one wave instruction = 1 KiB = 4 rows), the next step's 16 KiB already in
// flight in registers while the current one is computed; each step is staged
// in the wave's own LDS tile with the 16-byte pieces of row r stored at
// slot (piece ^ (r & 7)), so that both the row-major store and the MFMA
// operand reads below are free of bank conflicts.  Per 16 rows:
// A = idx_q (heads x d, two 16-head blocks, from registers), B = keys^T
// (d x rows): lane (g = l/16, n = l%16) takes row n, d in [32 s + 8 g, +8)
// for k-step s.  D[head][row] lands as lane (g, n) holding heads 4g + r
// (+16) of row n; the epilogue applies ReLU and the head weights and sums
// the four lane groups.
__global__ __launch_bounds__(256) void k_score(Args a) {
    __shared__ uint32_t lhist[kHistBins];
    __shared__ __attribute__((aligned(16))) uint8_t tiles[4][64 * 256];
    const int q = blockIdx.y;
    const QInfo qi = query_info(a, q);
    if (qi.mode == 2) return;
    if (a.fused && qi.mode == 0) return;
    const int64_t t0 = (int64_t)blockIdx.x * a.score_tile;
    const int64_t rows = qi.rows;
    if (t0 >= rows) return;
    const bool hist = a.fused != 0;
    if (hist) {
        for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0;
        __syncthreads();
    }
    const int lane = lane_id(), w = threadIdx.x >> 6, g = lane >> 4, n = lane & 15;

    bf16x8 qa[2][4];
    float wt[2][4];
    const uint16_t *qip = a.idx_q + (size_t)q * kIdxHeads * kIdxDim;
#pragma unroll
    for (int mb = 0; mb < 2; mb++) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            u32x4 v = *(const u32x4 *)(qip + (16 * mb + n) * kIdxDim + 32 * s + 8 * g);
            qa[mb][s] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int r = 0; r < 4; r++) wt[mb][r] = a.idx_w[(size_t)q * kIdxHeads + 16 * mb + 4 * g + r];
    }
    const uint8_t *K = reinterpret_cast<const uint8_t *>(a.idx_k + (size_t)qi.seq * a.key_stride * kIdxDim);
    float *srow = a.scores + (size_t)q * a.score_ld;
    const int st_mine = 2 * (g & 1) + (g >> 1);
    uint8_t *tb = tiles[w];
    const int64_t end = t0 + a.score_tile < rows ? t0 + a.score_tile : rows;

    u32x4 v[16];
    auto fetch = [&](int64_t base) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            int64_t r = base + 4 * i + (lane >> 4);
            r = r < rows ? r : rows - 1;
            v[i] = __builtin_nontemporal_load((const u32x4 *)(K + r * 256 + 16 * (lane & 15)));
        }
    };
    int64_t base = t0 + 64 * w;
    if (base < end) fetch(base);
    for (; base < end; base += 256) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int r = 4 * i + (lane >> 4), pc = lane & 15;
            *(u32x4 *)(tb + r * 256 + 16 * (pc ^ (r & 7))) = v[i];
        }
        if (base + 256 < end) fetch(base + 256);
        __builtin_amdgcn_wave_barrier();
        float p[4];
#pragma unroll
        for (int st = 0; st < 4; st++) {
            const int r = 16 * st + n;
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; s++) {
                const bf16x8 b = __builtin_bit_cast(bf16x8, *(const u32x4 *)(tb + r * 256 + 16 * ((4 * s + g) ^ (r & 7))));
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[0][s], b, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[1][s], b, acc1, 0, 0, 0);
            }
            float x = 0.f;
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
                x += wt[0][rr] * fmaxf(acc0[rr], 0.f);
                x += wt[1][rr] * fmaxf(acc1[rr], 0.f);
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
        if (row < end) {
            srow[row] = score;
            if (hist) atomicAdd(&lhist[order_key(score) >> 20], 1u);
        }
    }
    if (hist) {
        __syncthreads();
        uint32_t *gh = a.hist + (size_t)q * kHistBins;
        for (int i = threadIdx.x; i < kHistBins; i += 256)
            if (lhist[i]) atomicAdd(&gh[i], lhist[i]);
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
    uint32_t *gh = a.hist + (size_t)q * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += 256)
        if (lhist[i]) atomicAdd(&gh[i], lhist[i]);
}

// ---------------------------------------------------------------- top-k
// Exact radix select over 32-bit order keys, ranked by (key descending,
// row ascending), three digits: bits 31..20 (4096-bin histogram from the
// score kernel or k_hist), bits 19..10 and bits 9..0.
//   k_filter (grid chunks x queries): from the first-digit histogram find the
//     bucket b1 holding the keep-th row; count the chunk's rows above b1 and
//     copy the bucket's rows (key, row) into the chunk's own candidate slots.
//   k_resolve (one work-group per query): gathers all candidates into LDS,
//     resolves the exact threshold (second and third digit) and each
//     chunk's output offset and share of the rows equal to the threshold.
//   k_emit (chunks x queries): writes each chunk's selected rows in
//     ascending order at the chunk's offset.
// No global atomics: chunks own their candidate slots.

__device__ __forceinline__ void load_hist(const uint32_t *gh, uint32_t *lh) {
    uint32_t v[kHistBins / 256];
#pragma unroll
    for (int i = 0; i < kHistBins / 256; i++) v[i] = gh[threadIdx.x + 256 * i];
#pragma unroll
    for (int i = 0; i < kHistBins / 256; i++) lh[threadIdx.x + 256 * i] = v[i];
}

// grid (n_chunks, n_q), 256 threads.
__global__ __launch_bounds__(256) void k_filter(Args a) {
    __shared__ uint32_t hist[kHistBins];
    __shared__ uint32_t scan[8];
    __shared__ uint32_t res[4];
    const int q = blockIdx.y, c = blockIdx.x;
    const QInfo qi = query_info(a, q);
    if (qi.mode != 1) return;
    const int64_t rows = qi.rows;
    const int nch = (int)((rows + a.chunk - 1) / a.chunk);
    if (c >= nch) return;
    const float *s = a.scores_in + (size_t)q * a.score_ld;
    const int64_t r0 = (int64_t)c * a.chunk;
    const int64_t r1 = r0 + a.chunk < rows ? r0 + a.chunk : rows;
    // first block of scores in flight while the threshold bucket is found
    float sv[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int64_t r = r0 + 256 * i + threadIdx.x;
        sv[i] = r < r1 ? s[r] : 0.f;
    }
    load_hist(a.hist + (size_t)q * kHistBins, hist);
    __syncthreads();
    uint32_t n_gt1;
    const uint32_t b1 = find_bucket<kHistBins>(hist, (uint32_t)a.keep, scan, res, n_gt1);

    uint64_t *slots = a.cand + ((size_t)q * a.n_chunks + c) * a.cand_cap;
    uint32_t gt = 0, n_cand = 0;
    for (int64_t sb = r0; sb < r1; sb += 2048) {
        if (sb != r0) {
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int64_t r = sb + 256 * i + threadIdx.x;
                sv[i] = r < r1 ? s[r] : 0.f;
            }
        }
        uint32_t keys[8];
        uint32_t n_c = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int64_t r = sb + 256 * i + threadIdx.x;
            const uint32_t key = order_key(sv[i]);
            const bool ok = r < r1;
            const uint32_t d1 = key >> 20;
            gt += (ok && d1 > b1) ? 1u : 0u;
            const bool is_c = ok && d1 == b1;
            keys[i] = is_c ? key : 0u;
            n_c += is_c ? 1u : 0u;
        }
        uint32_t tot;
        uint32_t pos = n_cand + block_excl_scan(n_c, scan, tot);
        n_cand += tot;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            if (!keys[i]) continue;      // order keys of real scores are never 0
            const int64_t r = sb + 256 * i + threadIdx.x;
            if (pos < (uint32_t)a.cand_cap) slots[pos] = ((uint64_t)keys[i] << 32) | (uint32_t)r;
            pos++;
        }
    }
    gt = block_sum(gt, scan);
    if (threadIdx.x == 0) {
        ChunkInfo info;
        info.gt = gt;
        info.n_cand = n_cand;
        a.chunks[(size_t)q * a.n_chunks + c] = info;
    }
}

constexpr int kLdsCand = 8192;   // candidates k_resolve keeps in LDS

struct ResolveShared {
    uint32_t h[kHistBins];        // first digit, then the second (1024 bins)
    uint32_t h3[1024];            // third digit
    uint32_t pre[kMaxChunks + 1]; // exclusive prefix of the chunks' candidate counts
    uint32_t gtc[kMaxChunks];     // per chunk: bucket rows above the threshold
    uint32_t eqc[kMaxChunks];     // per chunk: rows equal to the threshold
    uint64_t cand[kLdsCand];
    uint32_t scan[8];
    uint32_t res[4];
};

// One work-group per sparse query: gathers the candidates of all chunks
// into LDS, finds the second and third digits of the keep-th key (the
// threshold), and writes each chunk's output offset and its share of the
// rows equal to the threshold (lowest chunks first).  grid (n_q), 256
// threads.  If some chunk's bucket rows overflowed its slots, or all of
// them overflow the LDS copy, the bucket rows are re-derived from the
// scores (slow, exact).
__global__ __launch_bounds__(256) void k_resolve(Args a) {
    __shared__ ResolveShared sh;
    const int q = blockIdx.x;
    const QInfo qi = query_info(a, q);
    if (qi.mode != 1) return;
    const int64_t rows = qi.rows;
    const int nch = (int)((rows + a.chunk - 1) / a.chunk);
    const uint32_t keep = (uint32_t)a.keep;
    const float *s = a.scores_in + (size_t)q * a.score_ld;
    ChunkInfo *ci = a.chunks + (size_t)q * a.n_chunks;
    const uint64_t *slots = a.cand + (size_t)q * a.n_chunks * a.cand_cap;
    const uint32_t ch = (uint32_t)a.chunk;

    const int per = (nch + 255) / 256;
    const int c0 = threadIdx.x * per;
    uint32_t ncs[kMaxChunks / 256], gts[kMaxChunks / 256];
    uint32_t my_nc = 0;
    bool overflow = false;
#pragma unroll
    for (int j = 0; j < kMaxChunks / 256; j++) {
        ncs[j] = gts[j] = 0;
        if (j < per && c0 + j < nch) {
            const ChunkInfo info = ci[c0 + j];
            gts[j] = info.gt;
            overflow |= info.n_cand > (uint32_t)a.cand_cap;
            ncs[j] = info.n_cand < (uint32_t)a.cand_cap ? info.n_cand : (uint32_t)a.cand_cap;
            my_nc += ncs[j];
        }
    }
    load_hist(a.hist + (size_t)q * kHistBins, sh.h);
    uint32_t n_all;
    uint32_t run = block_excl_scan(my_nc, sh.scan, n_all);
#pragma unroll
    for (int j = 0; j < kMaxChunks / 256; j++) {
        if (j < per && c0 + j < nch) {
            sh.pre[c0 + j] = run;
            sh.gtc[c0 + j] = 0;
            sh.eqc[c0 + j] = 0;
            run += ncs[j];
        }
    }
    if (threadIdx.x == 0) sh.pre[nch] = n_all;
    overflow = __syncthreads_or(overflow) || n_all > (uint32_t)kLdsCand;
    uint32_t n_gt1;
    const uint32_t b1 = find_bucket<kHistBins>(sh.h, keep, sh.scan, sh.res, n_gt1);
    const uint32_t need1 = keep - n_gt1;

    uint32_t *h2 = sh.h;
    __syncthreads();
    for (int i = threadIdx.x; i < 1024; i += 256) {
        h2[i] = 0;
        sh.h3[i] = 0;
    }
    __syncthreads();
    if (!overflow) {
        // candidates of all chunks packed into LDS, 16 loads per thread a round
        for (uint32_t base = 0; base < n_all; base += 16 * 256) {
            uint64_t e[16];
#pragma unroll
            for (int j = 0; j < 16; j++) {
                const uint32_t i = base + 256 * j + threadIdx.x;
                e[j] = 0;
                if (i < n_all) {
                    int lo = 0, hi = nch;          // chunk k with pre[k] <= i < pre[k+1]
                    while (hi - lo > 1) {
                        const int mid = (lo + hi) >> 1;
                        if (sh.pre[mid] <= i) lo = mid;
                        else hi = mid;
                    }
                    e[j] = slots[(size_t)lo * a.cand_cap + (i - sh.pre[lo])];
                }
            }
#pragma unroll
            for (int j = 0; j < 16; j++) {
                const uint32_t i = base + 256 * j + threadIdx.x;
                if (i < n_all) {
                    sh.cand[i] = e[j];
                    atomicAdd(&h2[(uint32_t)(e[j] >> 42) & 0x3FF], 1u);
                }
            }
        }
    } else {
        for (int64_t r = threadIdx.x; r < rows; r += 256) {
            const uint32_t key = order_key(s[r]);
            if ((key >> 20) == b1) atomicAdd(&h2[(key >> 10) & 0x3FF], 1u);
        }
    }
    __syncthreads();
    uint32_t n_gt2;
    const uint32_t b2 = find_bucket<1024>(h2, need1, sh.scan, sh.res, n_gt2);
    const uint32_t need2 = need1 - n_gt2;
    const uint32_t pre2 = (b1 << 10) | b2;   // key >> 10 of the level-2 bucket
    auto pass3 = [&](uint32_t key, uint32_t r) {
        const uint32_t k10 = key >> 10;
        if (k10 > pre2) atomicAdd(&sh.gtc[r / ch], 1u);
        else if (k10 == pre2) atomicAdd(&sh.h3[key & 0x3FF], 1u);
    };
    if (!overflow) {
        for (uint32_t i = threadIdx.x; i < n_all; i += 256) pass3((uint32_t)(sh.cand[i] >> 32), (uint32_t)sh.cand[i]);
    } else {
        for (int64_t r = threadIdx.x; r < rows; r += 256) {
            const uint32_t key = order_key(s[r]);
            if ((key >> 20) == b1) pass3(key, (uint32_t)r);
        }
    }
    __syncthreads();
    uint32_t n_gt3;
    const uint32_t b3 = find_bucket<1024>(sh.h3, need2, sh.scan, sh.res, n_gt3);
    const uint32_t thr = (pre2 << 10) | b3;
    const uint32_t m_eq = need2 - n_gt3;     // rows equal to thr that are kept
    auto pass4 = [&](uint32_t key, uint32_t r) {
        if ((key >> 10) != pre2) return;
        if (key > thr) atomicAdd(&sh.gtc[r / ch], 1u);
        else if (key == thr) atomicAdd(&sh.eqc[r / ch], 1u);
    };
    if (!overflow) {
        for (uint32_t i = threadIdx.x; i < n_all; i += 256) pass4((uint32_t)(sh.cand[i] >> 32), (uint32_t)sh.cand[i]);
    } else {
        for (int64_t r = threadIdx.x; r < rows; r += 256) {
            const uint32_t key = order_key(s[r]);
            if ((key >> 20) == b1) pass4(key, (uint32_t)r);
        }
    }
    __syncthreads();
    // equal rows go to the lowest chunks first; offsets are the exclusive
    // prefix of each chunk's selected count
    uint32_t eq_sum = 0;
#pragma unroll
    for (int j = 0; j < kMaxChunks / 256; j++)
        if (j < per && c0 + j < nch) eq_sum += sh.eqc[c0 + j];
    uint32_t tot;
    uint32_t eq_before = block_excl_scan(eq_sum, sh.scan, tot);
    uint32_t takes[kMaxChunks / 256], sel_sum = 0;
#pragma unroll
    for (int j = 0; j < kMaxChunks / 256; j++) {
        takes[j] = 0;
        if (j < per && c0 + j < nch) {
            const uint32_t e = sh.eqc[c0 + j];
            takes[j] = eq_before >= m_eq ? 0u : (m_eq - eq_before < e ? m_eq - eq_before : e);
            eq_before += e;
            sel_sum += gts[j] + sh.gtc[c0 + j] + takes[j];
        }
    }
    uint32_t off = block_excl_scan(sel_sum, sh.scan, tot);
#pragma unroll
    for (int j = 0; j < kMaxChunks / 256; j++) {
        if (j < per && c0 + j < nch) {
            ci[c0 + j].off = off;
            ci[c0 + j].eq_take = takes[j];
            off += gts[j] + sh.gtc[c0 + j] + takes[j];
        }
    }
    if (threadIdx.x == 0) a.thr[q] = thr;
}

// Writes the selection in ascending token order.  grid (n_chunks, n_q),
// 256 threads; each thread takes 4 consecutive rows per 1024-row step.
__global__ __launch_bounds__(256) void k_emit(Args a) {
    __shared__ uint32_t scan[8];
    const int q = blockIdx.y, c = blockIdx.x;
    const QInfo qi = query_info(a, q);
    int32_t *dst = a.sel + (size_t)q * a.sel_ld;
    if (qi.mode != 1) {
        if (c != 0) return;
        const int32_t cnt = qi.mode == 0 ? qi.nvis : 0;
        for (int i = threadIdx.x; i < a.sel_ld; i += 256) dst[i] = i < cnt ? i : -1;
        if (threadIdx.x == 0) a.sel_count[q] = cnt;
        return;
    }
    const int64_t rows = qi.rows;
    const int nch = (int)((rows + a.chunk - 1) / a.chunk);
    if (c >= nch) return;
    const uint32_t keep = (uint32_t)a.keep;
    const float *s = a.scores_in + (size_t)q * a.score_ld;
    const int64_t r0 = (int64_t)c * a.chunk;
    const int64_t r1 = r0 + a.chunk < rows ? r0 + a.chunk : rows;
    float sv[4];
    {
        const int64_t rb = r0 + 4 * threadIdx.x;
#pragma unroll
        for (int i = 0; i < 4; i++) sv[i] = rb + i < r1 ? s[rb + i] : 0.f;
    }
    const uint32_t thr = a.thr[q];
    const ChunkInfo info = a.chunks[(size_t)q * a.n_chunks + c];
    const int kp = a.kpool;
    uint32_t eq_base = 0, out_base = info.off;
    for (int64_t base = r0; base < r1; base += 1024) {
        const int64_t rb = base + 4 * threadIdx.x;
        if (base != r0) {
#pragma unroll
            for (int i = 0; i < 4; i++) sv[i] = rb + i < r1 ? s[rb + i] : 0.f;
        }
        bool gt[4], eq[4];
        uint32_t n_eq = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const bool ok = rb + i < r1;
            const uint32_t key = order_key(sv[i]);
            gt[i] = ok && key > thr;
            eq[i] = ok && key == thr;
            n_eq += eq[i];
        }
        uint32_t tot_eq;
        uint32_t eq_rank = eq_base + block_excl_scan(n_eq, scan, tot_eq);
        bool take[4];
        uint32_t n_take = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            take[i] = gt[i];
            if (eq[i]) {
                take[i] = eq_rank < info.eq_take;
                eq_rank++;
            }
            n_take += take[i];
        }
        uint32_t tot_take;
        uint32_t pos = out_base + block_excl_scan(n_take, scan, tot_take);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (!take[i]) continue;
            if (pos >= keep) break;                 // never past the kept rows
            const int32_t r = (int32_t)(rb + i);
            if (kp == 1) {
                dst[pos] = r;
            } else {
                for (int j = 0; j < kp; j++) dst[(size_t)pos * kp + j] = r * kp + j;
            }
            pos++;
        }
        eq_base += tot_eq;
        out_base += tot_take;
    }
    if (c == 0) {
        const int32_t pooled = a.keep * kp;
        const int32_t tail = qi.nvis - qi.rows * kp;
        const int32_t cnt = pooled + tail;
        for (int i = threadIdx.x; i < a.sel_ld - pooled; i += 256)
            dst[pooled + i] = i < tail ? qi.rows * kp + i : -1;
        if (threadIdx.x == 0) a.sel_count[q] = cnt;
    }
}

// Zeroes a query's first-digit histogram (after a standalone
// top-k; the fused step does this in the attention kernel).  grid (n_q).
__device__ __forceinline__ void clear_topk_state(const Args &a, int q) {
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) a.hist[(size_t)q * kHistBins + i] = 0;
}

__global__ __launch_bounds__(256) void k_topk_clear(Args a) { clear_topk_state(a, blockIdx.x); }

// ---------------------------------------------------------------- attention
// One work-group = (query q, split sp, head group hg of 16 heads); 256
// threads = 4 waves.  The split's selected rows are processed 32 at a time,
// staged row-major in LDS (row stride D*2 + 32 bytes) with the next step's
// rows already in flight in registers.  Per step:
//   QK : S^T[row][head] = C Q^T; wave (b = w & 1, kh = w >> 1) multiplies
//        row block b (16 rows) by its half of the k-steps, the two halves
//        are added through LDS;
//   softmax: online, per head (one head per lane column), lazy rescale
//        (only when the running max grows by more than 2^8); every wave
//        keeps the same running max so that all rescale alike;
//   PV : O^T[col][head] += V^T P^T for the wave's 128 output columns, with
//        A = V^T read by ds_read_b64_tr_b16 and B = P split into bf16 hi + lo.
// Work-group ids are laid out so that the four head groups of one (q, sp)
// are dispatched to the same XCD and read the gathered rows through one L2.
template <int D>
struct AttnCfg {
    static constexpr int ND = D / 32;            // MFMA k-steps of the score
    static constexpr int NH = ND / 2;            // k-steps per half
    static constexpr int RS = D * 2 + 32;        // LDS row stride in bytes
    static constexpr int PPR = D / 8;            // 16-byte pieces per row
    static constexpr int PER = kAttnRows * PPR / 256;
};

template <int D>
__global__ __launch_bounds__(256) void k_attend(Args a) {
    using Cfg = AttnCfg<D>;
    __shared__ __attribute__((aligned(16))) uint8_t rowbuf[kAttnRows * Cfg::RS];
    __shared__ int32_t sidx[kMaxSplitRows];
    __shared__ f32x4 sx[2][64];
    __shared__ f32x4 pbuf[2][64];
    __shared__ float bmax[2][16];

    const int n_pairs = a.n_q * a.n_split;
    const int within = blockIdx.x & 31;
    const int pair = (blockIdx.x >> 5) * 8 + (within & 7);
    const int hg = within >> 3;
    if (pair >= n_pairs) return;
    const int q = pair / a.n_split, sp = pair % a.n_split;
    if (a.clear_topk && sp == 0 && hg == 0) clear_topk_state(a, q);
    const QInfo qi = query_info(a, q);
    const int lane = lane_id(), w = threadIdx.x >> 6, g = lane >> 4, n = lane & 15;
    const int b = w & 1, kh = w >> 1;
    const int head = 16 * hg + n;

    int32_t count = 0;
    if (qi.mode != 2) {
        count = a.sel_count[q];
        count = count < 0 ? 0 : (count > a.sel_ld ? a.sel_ld : count);
    }
    const int32_t start = sp * a.split_rows;
    const int32_t nrows = (start + a.split_rows < count ? start + a.split_rows : count) - start;
    const int32_t *selq = a.sel + (size_t)q * a.sel_ld;
    for (int i = threadIdx.x; i < nrows; i += 256) {
        int32_t t = selq[start + i];
        sidx[i] = (t >= 0 && (int64_t)t < a.cache_stride) ? t : -1;
    }

    bf16x8 qreg[Cfg::NH];
    {
        const uint16_t *qp = a.q + ((size_t)q * kHeads + head) * D + 32 * Cfg::NH * kh;
#pragma unroll
        for (int s = 0; s < Cfg::NH; s++)
            qreg[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qp + 32 * s + 8 * g));
    }
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY, l_part = 0.f;
    const uint16_t *C = a.cache + (size_t)(qi.mode == 2 ? 0 : qi.seq) * a.cache_stride * D;
    const int nch = (nrows + kAttnRows - 1) / kAttnRows;
    __syncthreads();

    u32x4 v[Cfg::PER];
    auto fetch = [&](int c) {
#pragma unroll
        for (int i = 0; i < Cfg::PER; i++) {
            const int e = threadIdx.x + 256 * i;
            const int rr = e / Cfg::PPR, pc = e % Cfg::PPR;
            const int r = kAttnRows * c + rr;
            const int32_t t = r < nrows ? sidx[r] : -1;
            v[i] = t >= 0 ? *(const u32x4 *)(C + (size_t)t * D + 8 * pc) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    if (nch > 0) fetch(0);

    for (int c = 0; c < nch; c++) {
        if (c > 0) __syncthreads();                  // previous step's PV is done with rowbuf
#pragma unroll
        for (int i = 0; i < Cfg::PER; i++) {
            const int e = threadIdx.x + 256 * i;
            const int rr = e / Cfg::PPR, pc = e % Cfg::PPR;
            *(u32x4 *)(rowbuf + rr * Cfg::RS + 16 * pc) = v[i];
        }
        if (c + 1 < nch) fetch(c + 1);
        __syncthreads();

        // QK: this wave's row block and half of the k-steps
        f32x4 sa = {0.f, 0.f, 0.f, 0.f};
        {
            const uint8_t *rp = rowbuf + (16 * b + n) * Cfg::RS + 64 * Cfg::NH * kh + 16 * g;
#pragma unroll
            for (int s = 0; s < Cfg::NH; s++) {
                bf16x8 av = __builtin_bit_cast(bf16x8, *(const u32x4 *)(rp + 64 * s));
                sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qreg[s], sa, 0, 0, 0);
            }
        }
        if (kh == 1) sx[b][lane] = sa;
        __syncthreads();
        float z[4];
        if (kh == 0) {
            sa += sx[b][lane];
            float bm = -INFINITY;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int row = kAttnRows * c + 16 * b + 4 * g + r;
                const bool ok = row < nrows && sidx[row] >= 0;
                z[r] = ok ? sa[r] * a.scale_log2 : -INFINITY;
                bm = fmaxf(bm, z[r]);
            }
            bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
            bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
            if (g == 0) bmax[b][n] = bm;
        }
        __syncthreads();
        {
            const float cmax = fmaxf(bmax[0][n], bmax[1][n]);
            const bool need = cmax > m_ref + 8.f;
            if (__any(need)) {
                const float m_new = need ? cmax : m_ref;
                const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
                m_ref = m_new;
                l_part *= alpha;
#pragma unroll
                for (int i = 0; i < 8; i++) acc[i] *= alpha;
            }
        }
        if (kh == 0) {
            f32x4 p;
#pragma unroll
            for (int r = 0; r < 4; r++)
                p[r] = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(z[r] - m_ref);
            pbuf[b][lane] = p;
        }
        __syncthreads();
        bf16x8 phi, plo;
        {
            const f32x4 p0 = pbuf[0][lane], p1 = pbuf[1][lane];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const float p = j < 4 ? p0[j] : p1[j - 4];
                l_part += p;
                const uint32_t hb = __float_as_uint(p) & 0xFFFF0000u;
                const float lo = p - __uint_as_float(hb);
                phi[j] = __builtin_bit_cast(__bf16, (uint16_t)(hb >> 16));
                plo[j] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(lo) >> 16));
            }
        }
        {
            const int r_in = n >> 2, c_in = n & 3;
            const uint8_t *v1 = rowbuf + (4 * g + r_in) * Cfg::RS + 256 * w + 8 * c_in;
            const uint8_t *v2 = rowbuf + (16 + 4 * g + r_in) * Cfg::RS + 256 * w + 8 * c_in;
#pragma unroll
            for (int cb = 0; cb < 8; cb++) {
                const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(v1 + 32 * cb));
                const i16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(v2 + 32 * cb));
                typedef short i16x8 __attribute__((ext_vector_type(8)));
                const i16x8 tv = {t1[0], t1[1], t1[2], t1[3], t2[0], t2[1], t2[2], t2[3]};
                const bf16x8 av = __builtin_bit_cast(bf16x8, tv);
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, phi, acc[cb], 0, 0, 0);
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, plo, acc[cb], 0, 0, 0);
            }
        }
    }
    // total softmax mass per head over the four lane groups
    float l_tot = l_part + __shfl_xor(l_part, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);

    const int col0 = 128 * w + 4 * g;
    if (a.n_split == 1) {
        const bool bad = qi.mode == 2 || l_tot == 0.f;
        const float inv = 1.f / l_tot;
        float *o = a.out + ((size_t)q * kHeads + head) * kLatent + col0;
#pragma unroll
        for (int cb = 0; cb < 8; cb++) {
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
        for (int cb = 0; cb < 8; cb++) *(f32x4 *)(o + 16 * cb) = acc[cb];
        if (w == 0 && g == 0) {
            a.pml[2 * slot] = m_ref;
            a.pml[2 * slot + 1] = l_tot;
        }
    }
}

// Merge the splits of each (query, head): grid (64, n_q), 128 threads, each
// thread four output columns.  Up to 16 splits are loaded in one round trip
// and merged online (running max, rescaled sums).
__global__ __launch_bounds__(128) void k_reduce(Args a) {
    constexpr int MB = 16;
    const int q = blockIdx.y, h = blockIdx.x;
    const QInfo qi = query_info(a, q);
    const size_t slot0 = (size_t)q * a.n_split * kHeads + h;
    float M = -INFINITY, L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.n_split; s0 += MB) {
        f32x4 v[MB];
        float m[MB], l[MB];
#pragma unroll
        for (int i = 0; i < MB; i++) {
            m[i] = -INFINITY;
            l[i] = 0.f;
            v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (s0 + i < a.n_split) {
                const size_t slot = slot0 + (size_t)(s0 + i) * kHeads;
                m[i] = a.pml[2 * slot];
                l[i] = a.pml[2 * slot + 1];
                v[i] = *(const f32x4 *)(a.pacc + slot * kLatent + 4 * threadIdx.x);
            }
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
    const bool bad = qi.mode == 2 || L == 0.f;
    o = bad ? f32x4{NAN, NAN, NAN, NAN} : o * (1.f / L);
    *(f32x4 *)(a.out + ((size_t)q * kHeads + h) * kLatent + 4 * threadIdx.x) = o;
    if (a.lse && threadIdx.x == 0)
        a.lse[(size_t)q * kHeads + h] = bad ? NAN : (M + __log2f(L)) * 0.69314718055994531f;
}

// ---------------------------------------------------------------- launchers
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st) {
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    size_t blocks = (words + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, st, (uint32_t *)p, words);
    return hipGetLastError();
}

hipError_t launch_score(const Args &a, int64_t max_rows, hipStream_t st) {
    const unsigned tiles = (unsigned)((max_rows + a.score_tile - 1) / a.score_tile);
    hipLaunchKernelGGL(k_score, dim3(tiles, a.n_q), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_hist(const Args &a, hipStream_t st) {
    hipLaunchKernelGGL(k_hist, dim3(a.n_chunks, a.n_q), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_filter(const Args &a, hipStream_t st) {
    hipLaunchKernelGGL(k_filter, dim3(a.n_chunks, a.n_q), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_resolve(const Args &a, hipStream_t st) {
    hipLaunchKernelGGL(k_resolve, dim3(a.n_q), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_topk_clear(const Args &a, hipStream_t st) {
    hipLaunchKernelGGL(k_topk_clear, dim3(a.n_q), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_emit(const Args &a, hipStream_t st) {
    hipLaunchKernelGGL(k_emit, dim3(a.n_chunks, a.n_q), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_attend(const Args &a, hipStream_t st, const std::function<void()> &between) {
    // 4 head groups per (query, split); groups of 8 (query, split) pairs
    const unsigned blocks = (unsigned)(((a.n_q * a.n_split + 7) / 8) * 32);
    if (a.D == 576)
        hipLaunchKernelGGL(k_attend<576>, dim3(blocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(k_attend<512>, dim3(blocks), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (between) between();
    if (e != hipSuccess || a.n_split == 1) return e;
    hipLaunchKernelGGL(k_reduce, dim3(kHeads, a.n_q), dim3(128), 0, st, a);
    return hipGetLastError();
}

}  // namespace dsa
