// Page selection for one chunk (WorldAttention review, "HKV: Page-Level
// Multi-Tier Memory"): optional prompt stage, then the page stage
//   qbar = mean over the chunk's queries,
//   alpha_j = sum_{h,c} qbar[h,c] * kbar_j[h,c] / sqrt(d),
//   idx = top-K_p candidates by (alpha desc, page id asc).
// Everything after the bf16/fp32 inputs is fp64, with fixed reduction orders,
// so the selection is decided in the same precision as the fp64 reference.
//
// Three launches, no host synchronisation:
//   stage 1  blocks [0, q_blocks): fp64 partial column sums of Q (HBM stream);
//            blocks [q_blocks, q_blocks + n_chunks): cosine of the current
//            prompt with one past chunk's prompt (prompt stage only);
//   stage 2  one block per 64 columns: finish qbar for those columns (16
//            lanes per column, fixed order), derive the candidate list
//            (prompt stage: rank the chunks), and write each candidate's
//            partial dot product over those columns;
//   stage 3  one block: add the column-group partials of each candidate with
//            a butterfly (fixed order), scale, and take the top K_p by K_p
//            rounds of a wavefront-shuffle argmax.
#include <math.h>

#include "colsum.h"
#include "wa_internal.h"

namespace wa {

static constexpr int kGroupCols = 64;     // columns per stage-2 block
static constexpr int kStage2Threads = 1024;
static constexpr int kStage3Threads = 256;

SelectWs select_workspace(int32_t dtype, int64_t hd, int32_t n_q, int32_t n_cand,
                          int32_t n_chunks) {
    SelectWs w;
    w.q_plan = colsum_plan(dtype, hd, n_q, 256, 16);
    w.groups = (int)((hd + kGroupCols - 1) / kGroupCols);
    size_t off = 0;
    w.partial_q = off;
    off = align_up(off + (size_t)w.q_plan.blocks * hd * sizeof(double), 256);
    w.cosine = off;
    off = align_up(off + (size_t)(n_chunks > 0 ? n_chunks : 1) * sizeof(double), 256);
    w.alpha_part = off;
    off = align_up(off + (size_t)w.groups * n_cand * sizeof(double), 256);
    w.cand = off;
    off = align_up(off + (size_t)n_cand * sizeof(int32_t), 256);
    w.total = off;
    return w;
}

// (score desc, id asc) total order; an id < 0 marks "no item" and ranks last.
__device__ __forceinline__ bool ranks_before(double sa, int ia, double sb, int ib) {
    if (ib < 0) return ia >= 0;
    if (ia < 0) return false;
    return sa > sb || (sa == sb && ia < ib);
}

// Butterfly argmax over the 64 lanes of a wavefront; every lane ends with the
// same winner because the order is total.
__device__ __forceinline__ void wave_argmax(double &s, int &id, int &src) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double os = __shfl_xor(s, off, 64);
        const int oid = __shfl_xor(id, off, 64);
        const int osrc = __shfl_xor(src, off, 64);
        if (ranks_before(os, oid, s, id)) {
            s = os;
            id = oid;
            src = osrc;
        }
    }
}

// Fixed-order block reduction of three doubles (any blockDim.x).
__device__ void block_sum3(double &a, double &b, double &c, double *sh) {
    const int t = threadIdx.x;
    sh[t] = a;
    sh[blockDim.x + t] = b;
    sh[2 * blockDim.x + t] = c;
    __syncthreads();
    for (int n = blockDim.x; n > 1;) {
        const int half = (n + 1) >> 1;
        if (t < n - half) {
            sh[t] += sh[t + half];
            sh[blockDim.x + t] += sh[blockDim.x + t + half];
            sh[2 * blockDim.x + t] += sh[2 * blockDim.x + t + half];
        }
        __syncthreads();
        n = half;
    }
    a = sh[0];
    b = sh[blockDim.x];
    c = sh[2 * blockDim.x];
}

template <bool BF16>
__global__ void k_select_stage1(const uint4 *__restrict__ q, int64_t n_q, int chunks,
                                int row_lanes, int rows_per_block, int q_blocks,
                                double *__restrict__ partial_q,
                                const float *__restrict__ chunk_prompts,
                                const float *__restrict__ cur_prompt, int emb_dim,
                                double *__restrict__ cosine) {
    extern __shared__ double lds[];
    constexpr int VEC = BF16 ? 8 : 4;
    if ((int)blockIdx.x < q_blocks) {
        colsum_block<BF16>(q, nullptr, nullptr, nullptr, n_q, chunks, row_lanes, rows_per_block,
                           blockIdx.x, lds, partial_q + (int64_t)blockIdx.x * chunks * VEC);
        return;
    }
    // prompt stage: cosine of the current prompt with chunk m's prompt
    const int m = blockIdx.x - q_blocks;
    const float *pm = chunk_prompts + (int64_t)m * emb_dim;
    double dot = 0.0, nn = 0.0, pp = 0.0;
    for (int e = threadIdx.x; e < emb_dim; e += blockDim.x) {
        const double a = (double)cur_prompt[e];
        const double b = (double)pm[e];
        dot += a * b;
        nn += b * b;
        pp += a * a;
    }
    block_sum3(dot, nn, pp, lds);
    if (threadIdx.x == 0) cosine[m] = dot / (sqrt(pp) * sqrt(nn));
}

// Rank the chunks by (cosine desc, id asc) and write the first n_keep chunk
// ids to `kept` (shared memory).  Run by one wavefront; n_keep rounds.
__device__ void rank_chunks(const double *__restrict__ cosine, int n_chunks, int n_keep,
                            int *kept) {
    const int lane = threadIdx.x & 63;
    const int per_lane = (n_chunks + 63) / 64;   // <= 64
    unsigned long long mine = 0ull;
    for (int r = 0; r < n_keep; ++r) {
        double bs = 0.0;
        int bid = -1, bsrc = -1;
        for (int u = 0; u < per_lane; ++u) {
            const int m = lane + 64 * u;
            if (m >= n_chunks || ((mine >> u) & 1ull)) continue;
            const double cs = cosine[m];
            if (ranks_before(cs, m, bs, bid)) {
                bs = cs;
                bid = m;
                bsrc = u;
            }
        }
        wave_argmax(bs, bid, bsrc);
        // the lane that owns the winner marks it taken
        if (bid >= 0 && (bid & 63) == lane) mine |= 1ull << (bid / 64);
        if (lane == 0) kept[r] = bid;
    }
}

__global__ __launch_bounds__(kStage2Threads) void k_select_stage2(const double *__restrict__ partial_q, int q_blocks, int hd,
                                int64_t n_q, const double *__restrict__ page_means,
                                int max_pages, const int32_t *__restrict__ cand_in, int n_cand,
                                const double *__restrict__ cosine, int n_chunks,
                                const int32_t *__restrict__ chunk_pages, int pages_per_chunk,
                                int n_keep, int32_t *__restrict__ cand_ws,
                                int32_t *__restrict__ out_chunks, int32_t *__restrict__ out_cand,
                                double *__restrict__ alpha_part) {
    __shared__ double qbar[kGroupCols];
    __shared__ double red[16 * kGroupCols];
    __shared__ int kept[WA_MAX_CANDIDATES];
    const int t = threadIdx.x;
    const int g = blockIdx.x;
    const bool prompt = cosine != nullptr;

    // qbar for this block's columns (block partials added in a fixed order)
    const double tot = reduce_partials_64(partial_q, q_blocks, hd, g * kGroupCols, red);
    if (t < kGroupCols) {
        const int col = g * kGroupCols + t;
        qbar[t] = col < hd ? tot / (double)n_q : 0.0;
    }
    if (prompt && t >= 64 && t < 128) rank_chunks(cosine, n_chunks, n_keep, kept);
    __syncthreads();

    // candidate id of position j
    auto cand_of = [&](int j) -> int {
        if (prompt) {
            const int r = j / pages_per_chunk;
            const int m = kept[r];
            return chunk_pages[(int64_t)m * pages_per_chunk + (j % pages_per_chunk)];
        }
        return cand_in ? cand_in[j] : j;
    };

    if (g == 0) {
        for (int j = t; j < n_cand; j += blockDim.x) {
            const int id = cand_of(j);
            cand_ws[j] = id;
            if (out_cand) out_cand[j] = id;
        }
        if (prompt && out_chunks)
            for (int r = t; r < n_keep; r += blockDim.x) out_chunks[r] = kept[r];
    }

    // partial dot products: one wavefront per candidate, butterfly sum
    const int wave = t >> 6, lane = t & 63, n_waves = blockDim.x >> 6;
    const int col = g * kGroupCols + lane;
    for (int j = wave; j < n_cand; j += n_waves) {
        const int id = cand_of(j);
        double v = 0.0;
        if (id >= 0 && id < max_pages && col < hd)
            v = qbar[lane] * page_means[(int64_t)id * hd + col];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) alpha_part[(int64_t)g * n_cand + j] = v;
    }
}

// One block.  alpha_j: lane g of a wavefront holds the column-group-g partial
// of candidate j and a butterfly adds them (fixed order); wavefronts take
// candidates in turn.  Then wavefront 0 takes the top K_p: candidate j lives
// in lane j % 64, slot j / 64, and each round is a wavefront-shuffle argmax.
__global__ __launch_bounds__(kStage3Threads) void k_select_stage3(
    const double *__restrict__ alpha_part, int groups, int n_cand,
    const int32_t *__restrict__ cand_ws, int max_pages, double sqrt_d, int k_p,
    int32_t *__restrict__ out_idx, double *__restrict__ out_scores) {
    __shared__ double sc[WA_MAX_CANDIDATES];
    __shared__ int ids[WA_MAX_CANDIDATES];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    for (int j = wave; j < n_cand; j += kStage3Threads / 64) {
        double v = lane < groups ? alpha_part[(int64_t)lane * n_cand + j] : 0.0;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) {
            const int id = cand_ws[j];
            const bool valid = id >= 0 && id < max_pages;
            const double s = valid ? v / sqrt_d : -INFINITY;
            sc[j] = s;
            ids[j] = id;
            if (out_scores) out_scores[j] = s;
        }
    }
    __syncthreads();
    if (wave != 0) return;
    const int per_lane = (n_cand + 63) / 64;   // <= 64
    unsigned long long taken = 0ull;
    for (int u = 0; u < per_lane; ++u) {
        const int j = lane + 64 * u;
        // past the end, or an id outside the pool: never selected
        if (j >= n_cand || ids[j] < 0 || ids[j] >= max_pages) taken |= 1ull << u;
    }
    for (int r = 0; r < k_p; ++r) {
        double bs = 0.0;
        int bid = -1, bslot = -1;
        for (int u = 0; u < per_lane; ++u) {
            if ((taken >> u) & 1ull) continue;
            const int j = lane + 64 * u;
            if (ranks_before(sc[j], ids[j], bs, bid)) {
                bs = sc[j];
                bid = ids[j];
                bslot = j;
            }
        }
        wave_argmax(bs, bid, bslot);
        if (bslot >= 0 && (bslot & 63) == lane) taken |= 1ull << (bslot >> 6);
        if (lane == 0) out_idx[r] = bid;     // -1 when nothing valid is left
    }
}

hipError_t launch_select(const wa_layout &L, const void *q, int32_t n_q, const double *page_means,
                         const int32_t *cand, int32_t n_cand, const wa_prompt_stage *prompt,
                         int32_t k_p, int32_t *out_idx, double *out_scores, void *ws,
                         hipStream_t s) {
    const int64_t hd = (int64_t)L.n_heads * L.head_dim;
    const int n_chunks = prompt ? prompt->n_chunks : 0;
    const SelectWs w = select_workspace(L.dtype, hd, n_q, n_cand, n_chunks);
    char *base = (char *)ws;
    double *partial_q = (double *)(base + w.partial_q);
    double *cosine = prompt ? (double *)(base + w.cosine) : nullptr;
    double *alpha_part = (double *)(base + w.alpha_part);
    int32_t *cand_ws = (int32_t *)(base + w.cand);
    const ColSumPlan &p = w.q_plan;

    size_t lds = (size_t)p.row_lanes * hd * sizeof(double);
    if (prompt && lds < 3 * (size_t)p.threads * sizeof(double))
        lds = 3 * (size_t)p.threads * sizeof(double);
    const int blocks1 = p.blocks + n_chunks;
    const float *cp = prompt ? prompt->chunk_prompts : nullptr;
    const float *cur = prompt ? prompt->cur_prompt : nullptr;
    const int emb = prompt ? prompt->emb_dim : 0;
    if (L.dtype == WA_BF16)
        hipLaunchKernelGGL(k_select_stage1<true>, dim3(blocks1), dim3(p.threads), lds, s,
                           (const uint4 *)q, (int64_t)n_q, p.chunks, p.row_lanes,
                           p.rows_per_block, p.blocks, partial_q, cp, cur, emb, cosine);
    else
        hipLaunchKernelGGL(k_select_stage1<false>, dim3(blocks1), dim3(p.threads), lds, s,
                           (const uint4 *)q, (int64_t)n_q, p.chunks, p.row_lanes,
                           p.rows_per_block, p.blocks, partial_q, cp, cur, emb, cosine);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    hipLaunchKernelGGL(k_select_stage2, dim3(w.groups), dim3(kStage2Threads), 0, s,
                       (const double *)partial_q, p.blocks, (int)hd, (int64_t)n_q, page_means,
                       L.max_pages, prompt ? nullptr : cand, n_cand, (const double *)cosine,
                       n_chunks, prompt ? prompt->chunk_pages : nullptr,
                       prompt ? prompt->pages_per_chunk : 1, prompt ? prompt->n_keep : 0,
                       cand_ws, prompt ? prompt->out_chunks : nullptr,
                       prompt ? prompt->out_cand : nullptr, alpha_part);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    hipLaunchKernelGGL(k_select_stage3, dim3(1), dim3(kStage3Threads), 0, s, (const double *)alpha_part,
                       w.groups, n_cand, (const int32_t *)cand_ws, L.max_pages,
                       sqrt((double)L.head_dim), k_p, out_idx, out_scores);
    return hipGetLastError();
}

}  // namespace wa
