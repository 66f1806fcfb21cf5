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

constexpr int kPfQ = 8;          // queries per prefill work-group

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

__device__ __forceinline__ int query_seq(const Args &a, int q) { return a.q_seq ? a.q_seq[q] : q; }

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
template <bool STRIDE>
__global__ __launch_bounds__(256) void k_score(Args a) {
    __shared__ uint32_t lhist[kHistBins];
    __shared__ __attribute__((aligned(16))) uint8_t tiles[4][64 * 256];
    const int q = blockIdx.y;
    const QInfo qi = query_info(a, q);
    if (qi.mode == 2) return;
    if (a.fused && qi.mode == 0) return;
    if (a.prefill && qi.seq == query_seq(a, q - q % kPfQ)) return;   // done by k_score_prefill
    const int64_t rows = qi.rows;
    if ((int64_t)blockIdx.x * a.score_tile >= rows) return;
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
    u32x4 v[16];
    auto fetch = [&](int64_t base) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            int64_t r = base + 4 * i + (lane >> 4);
            r = r < rows ? r : rows - 1;
            v[i] = __builtin_nontemporal_load((const u32x4 *)(K + r * 256 + 16 * (lane & 15)));
        }
    };
    // tiles t0 = blockIdx.x * tile, stepping by the grid (one pass in the
    // common case; the prefill fix-up grid has one work-group per query)
    for (int64_t t0 = (int64_t)blockIdx.x * a.score_tile; t0 < rows;
         t0 = STRIDE ? t0 + (int64_t)gridDim.x * a.score_tile : rows) {
    const int64_t end = t0 + a.score_tile < rows ? t0 + a.score_tile : rows;
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
    }
    if (hist) {
        __syncthreads();
        uint32_t *gh = a.hist + (size_t)q * kHistBins;
        for (int i = threadIdx.x; i < kHistBins; i += 256)
            if (lhist[i]) atomicAdd(&gh[i], lhist[i]);
    }
}

// Chunked-prefill indexer: a dense [8 queries x 32 heads] x [128 x keys]
// contraction per work-group.  grid (key ranges, query blocks of 8), 512
// threads = 8 waves, wave w computes query 8*blockIdx.y + w.  The block's
// queries are consecutive positions of one sequence (the leader's); a
// query of another sequence is left to the fix-up pass of k_score.  Key
// tiles of 128 rows are loaded with coalesced 16-byte loads (512 threads
// x 4 = 32 KiB), staged swizzled in LDS (double buffer) and shared by the
// eight queries; causality masks the scores and the histogram per query
// (a query scores rows < rows(q)).  Per-query first-digit histograms live
// in LDS as 16-bit counters, two to a word.
constexpr int kPfTile = 128;     // key rows per LDS tile
constexpr int kPfRange = 4096;   // key rows per work-group

__global__ __launch_bounds__(512) void k_score_prefill(Args a) {
    __shared__ __attribute__((aligned(16))) uint8_t ktile[2][kPfTile * 256];
    __shared__ uint32_t lh[kPfQ][kHistBins / 2];
    __shared__ int32_t sh_rows[kPfQ];
    const int w = threadIdx.x >> 6, lane = lane_id(), g = lane >> 4, n = lane & 15;
    const int q0 = blockIdx.y * kPfQ;
    const int q = q0 + w;
    const int lead = query_seq(a, q0);
    const bool hist = a.fused != 0;
    // does this wave's query take part, and up to which row
    if (lane == 0) {
        int32_t rr = 0;
        if (q < a.n_q) {
            const QInfo qi = query_info(a, q);
            const bool part = qi.mode != 2 && !(a.fused && qi.mode == 0) && qi.seq == lead;
            rr = part ? qi.rows : 0;
        }
        sh_rows[w] = rr;
    }
    __syncthreads();
    int32_t kmax = 0;
#pragma unroll
    for (int i = 0; i < kPfQ; i++) kmax = sh_rows[i] > kmax ? sh_rows[i] : kmax;
    const int64_t k0 = (int64_t)blockIdx.x * kPfRange;
    if (k0 >= kmax) return;
    const int64_t k1 = k0 + kPfRange < kmax ? k0 + kPfRange : kmax;
    const int32_t my_rows = sh_rows[w];
    if (hist)
        for (int i = threadIdx.x; i < kPfQ * kHistBins / 2; i += 512) (&lh[0][0])[i] = 0;

    bf16x8 qa[2][4];
    float wt[2][4];
    {
        const int qq = q < a.n_q ? q : q0;
        const uint16_t *qip = a.idx_q + (size_t)qq * kIdxHeads * kIdxDim;
#pragma unroll
        for (int mb = 0; mb < 2; mb++) {
#pragma unroll
            for (int s = 0; s < 4; s++)
                qa[mb][s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qip + (16 * mb + n) * kIdxDim + 32 * s + 8 * g));
#pragma unroll
            for (int r = 0; r < 4; r++) wt[mb][r] = a.idx_w[(size_t)qq * kIdxHeads + 16 * mb + 4 * g + r];
        }
    }
    const uint8_t *K = reinterpret_cast<const uint8_t *>(a.idx_k + (size_t)lead * a.key_stride * kIdxDim);
    float *srow = a.scores + (size_t)(q < a.n_q ? q : 0) * a.score_ld;
    const int st_mine = 2 * (g & 1) + (g >> 1);

    u32x4 v[4];
    auto fetch = [&](int64_t base) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int e = threadIdx.x + 512 * i;        // 16-byte piece of the tile
            int64_t r = base + (e >> 4);
            r = r < kmax ? r : kmax - 1;
            v[i] = __builtin_nontemporal_load((const u32x4 *)(K + r * 256 + 16 * (e & 15)));
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int e = threadIdx.x + 512 * i;
            const int r = e >> 4, pc = e & 15;
            *(u32x4 *)(&ktile[buf][r * 256 + 16 * (pc ^ (r & 7))]) = v[i];
        }
    };
    fetch(k0);
    int buf = 0;
    for (int64_t base = k0; base < k1; base += kPfTile, buf ^= 1) {
        stage(buf);
        if (base + kPfTile < k1) fetch(base + kPfTile);
        __syncthreads();
        const uint8_t *tb = ktile[buf];
#pragma unroll
        for (int j = 0; j < 2; j++) {                    // two groups of 64 keys
            float p[4];
#pragma unroll
            for (int st = 0; st < 4; st++) {
                const int r = 64 * j + 16 * st + n;
                f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; s++) {
                    const bf16x8 bv = __builtin_bit_cast(bf16x8, *(const u32x4 *)(tb + r * 256 + 16 * ((4 * s + g) ^ (r & 7))));
                    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[0][s], bv, acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[1][s], bv, acc1, 0, 0, 0);
                }
                float x = 0.f;
#pragma unroll
                for (int rr = 0; rr < 4; rr++) {
                    x += wt[0][rr] * fmaxf(acc0[rr], 0.f);
                    x += wt[1][rr] * fmaxf(acc1[rr], 0.f);
                }
                p[st] = x;
            }
            const bool b0 = g & 1, b1 = (g >> 1) & 1;
            const float send0 = b0 ? p[0] : p[2], send1 = b0 ? p[1] : p[3];
            const float keep0 = b0 ? p[2] : p[0], keep1 = b0 ? p[3] : p[1];
            const float q0s = keep0 + __shfl_xor(send0, 16, 64);
            const float q1s = keep1 + __shfl_xor(send1, 16, 64);
            const float score = (b1 ? q1s : q0s) + __shfl_xor(b1 ? q0s : q1s, 32, 64);
            const int64_t row = base + 64 * j + 16 * st_mine + n;
            if (row < my_rows) {
                srow[row] = score;
                if (hist) {
                    const uint32_t bin = order_key(score) >> 20;
                    atomicAdd(&lh[w][bin >> 1], 1u << (16 * (bin & 1)));
                }
            }
        }
        __syncthreads();                                  // buffer free for the tile after next
    }
    if (hist) {
        for (int i = threadIdx.x; i < kPfQ * kHistBins / 2; i += 512) {
            const int qq = q0 + i / (kHistBins / 2);
            const uint32_t word = (&lh[0][0])[i];
            if (!word || qq >= a.n_q) continue;
            const int bin = 2 * (i % (kHistBins / 2));
            uint32_t *gh = a.hist + (size_t)qq * kHistBins + bin;
            if (word & 0xFFFFu) atomicAdd(gh, word & 0xFFFFu);
            if (word >> 16) atomicAdd(gh + 1, word >> 16);
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
// buffers; the kernel waits for it itself.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory");
}

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
    if (a.clear_topk && sp == 0) clear_topk_state(a, q);
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

    // DMA of step c's rows into buffer slot b: V parts of rows w, w+8,
    // w+16, w+24; waves 0..3 also the RoPE tails of rows 8w..8w+7
    const bool rope_wave = D > 512 && w < 4;
    auto issue = [&](int c, int b) {
        uint8_t *vb = lds + b * Cfg::BUF;
        const int32_t *si = sidx + kAttnRows * c;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r = w + 8 * i;
            const int32_t t = si[r];
            const uint8_t *src = t >= 0 ? C + (size_t)t * (2 * D) : kZeroRow;
            dma16(src + 16 * lane, __builtin_amdgcn_readfirstlane(lds_addr(vb + r * Cfg::VS)));
        }
        if (rope_wave) {
            const int row = 8 * w + (lane >> 3);
            const int32_t t = si[row];
            const uint8_t *src = t >= 0 ? C + (size_t)t * (2 * D) : kZeroRow;
            const int piece = (lane & 7) ^ (row & 7);
            dma16(src + 1024 + 16 * piece, __builtin_amdgcn_readfirstlane(lds_addr(vb + Cfg::VBYTES + 8 * w * 128)));
        }
    };

    f32x4 acc[16];
#pragma unroll
    for (int i = 0; i < 16; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY, l_part = 0.f;

    if (nst > 0) issue(0, 0);
    if (nst > 1) issue(1, 1);
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
        if (c + 2 < nst) issue(c + 2, b_cur == 0 ? 2 : b_cur - 1);
        const uint8_t *vb = lds + b_cur * Cfg::BUF;
        b_cur = b_cur == 2 ? 0 : b_cur + 1;
        const uint64_t okmask = __ballot(lane < kAttnRows && sidx[kAttnRows * c + (lane & 31)] >= 0);

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
        cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
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
    float l_tot = l_part + __shfl_xor(l_part, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);

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
    if (a.prefill) {
        const unsigned ranges = (unsigned)((max_rows + kPfRange - 1) / kPfRange);
        hipLaunchKernelGGL(k_score_prefill, dim3(ranges, (a.n_q + kPfQ - 1) / kPfQ), dim3(512), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // in prefill mode k_score only picks up queries outside their block's
    // sequence: one work-group per query, striding over the tiles
    if (a.prefill)
        hipLaunchKernelGGL(k_score<true>, dim3(1, a.n_q), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(k_score<false>, dim3((unsigned)((max_rows + a.score_tile - 1) / a.score_tile), a.n_q),
                           dim3(256), 0, st, a);
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
    if (a.D == 576)
        hipLaunchKernelGGL(k_attend<576>, dim3(a.n_split, a.n_q), dim3(512), 0, st, a);
    else
        hipLaunchKernelGGL(k_attend<512>, dim3(a.n_split, a.n_q), dim3(512), 0, st, a);
    hipError_t e = hipGetLastError();
    if (between) between();
    if (e != hipSuccess || a.n_split == 1) return e;
    hipLaunchKernelGGL(k_reduce, dim3(kHeads, a.n_q), dim3(128), 0, st, a);
    return hipGetLastError();
}

}  // namespace dsa
