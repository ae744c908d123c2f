// Page selection for one chunk (WorldAttention review, "HKV: Page-Level
// Multi-Tier Memory"): optional prompt stage, then the page stage
//   qbar = mean over the chunk's queries,
//   alpha_j = sum_{h,c} qbar[h,c] * kbar_j[h,c] / sqrt(d),
//   idx = top-K_p candidates by (alpha desc, page id asc).
// Everything after the bf16/fp32 inputs is fp64, with fixed reduction orders,
// so the selection is decided in the same precision as the fp64 reference,
// and repeated calls are bitwise equal.
//
// With at most kFusedMaxCand candidates (with a prompt stage: at most
// kFusedMaxCand pages in all the past chunks): one launch.  Block (column
// group, row block) forms the fp64 column sums of its rows of Q and, since
// alpha is linear in qbar, each candidate's dot product with them over the
// group's columns (with a prompt stage, every chunk's pages; further blocks
// form the prompt cosines); the block that finishes last (a completion
// counter) adds the block partials of each candidate in block order, ranks
// the chunks and keeps their pages (prompt stage), scales, ranks and writes
// the result, then clears the counter.
// With 65 to 256 candidates and no prompt stage: one launch in two levels.
// Block (column group, row block) publishes its column sums; the last row
// block of each column group adds them and forms every candidate's partial
// dot product over the group's columns; the last group adds those, ranks
// (K_p rounds of a wavefront argmax) and clears the counters.
// Otherwise three launches, no host synchronisation:
//   stage 1  blocks (column group, row block): fp64 partial column sums of Q
//            (HBM stream); then one block per past chunk: cosine of the
//            current prompt with that chunk's prompt (prompt stage only).
//   stage 2  one block per 64 columns: finish qbar for those columns (16
//            lanes per column, fixed order), derive the candidate list
//            (prompt stage: rank the chunks), and write each candidate's
//            partial dot product over those columns.
//   stage 3  one block: alpha_j = the column-group partials of candidate j
//            added in group order, scaled; then the top K_p.
// Ranking (both paths): with at most one candidate per thread, a candidate's
// rank (the number of candidates ordered before it) is counted by a group of
// lanes, each comparing a share of the list, and summed over the group; beyond
// that, K_p rounds of a wavefront-shuffle argmax.
// The one-launch path hands its partials over with agent-scope atomic stores
// and loads (written through to, and read from, the device's coherent level,
// so no L2 write-back or invalidate is needed), ordered by waiting for the
// stores before the counter's increment.
#include <math.h>

#include <mutex>

#include "colsum.h"
#include "wa_internal.h"

namespace wa {

// Workspace of wa_select_pages_noalloc: one fixed array per device, in the
// library's device image, for callers that cannot allocate.  Every call on a
// device shares it (calls that overlap on one device race).  The selection
// writes every entry it reads except the one-launch paths' completion
// counters, which are zero when the image is loaded and which every call
// leaves at zero, so nothing needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[WA_SELECT_NOALLOC_MAX_WORKSPACE];

static constexpr int kMaxDevices = 64;

hipError_t select_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        // the array's name is a host-side stand-in: the device address of this
        // device's copy comes from the runtime, with the device current
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

static constexpr int kGroupCols = 64;     // columns per stage-2 block
static constexpr int kStage2Threads = 1024;
static constexpr int kStage3Threads = 1024;
static constexpr int kQRowsPerLane = 8;   // rows each stage-1 lane adds
static constexpr int kFusedMaxCand = 64;  // candidates of the one-launch path
static constexpr int kFusedRowsPerLane = 16;
static constexpr int kFusedBatch = 16;      // rows of a lane in flight together
// One-launch column groups of 16 sixteen-byte vectors (x 256 rows per block):
// each block then reads a quarter of the page-mean bytes that groups of 64
// vectors need.  On a 4,680 x 1,536 bf16 chunk: 10.9-11.3 us with groups of
// 16, 32 or 64 vectors at 16 candidates, but 14.4 us against 16.0 (32) and
// 17.0 us (64) at 48 candidates.
static constexpr int kFusedGroupChunks = 16;
// Candidates of the two-level one-launch path (more than kFusedMaxCand, no
// prompt stage); its ranking takes K_p rounds of a wavefront argmax beyond
// 64 candidates (a per-candidate count would compare every pair).
static constexpr int kWideMaxCand = 256;
static constexpr int kWideGroupChunks = 8;   // column group: 8 vectors (64 bf16 columns)
static constexpr int kWideRounds = 8;        // candidate rounds of partial dots in flight
// (At 136 candidates on a 4,680 x 1,536 bf16 chunk: 16.9 us against 22.4 us
// for the three launches; groups of 16 or 4 vectors measured slower, 2 or 4
// rounds in flight no faster.)

// Two-level one launch: kFusedMaxCand + 1 ... kWideMaxCand candidates, no
// prompt stage (and at most 63 column groups, checked with the plan).
static bool select_wide(int32_t n_cand, int32_t n_chunks) {
    return n_chunks == 0 && n_cand > kFusedMaxCand && n_cand <= kWideMaxCand;
}

// One launch: at most kFusedMaxCand candidates, or with a prompt stage at
// most kFusedMaxCand pages in all the past chunks (every chunk's pages are
// scored, and the last block keeps those of the chunks the prompts select).
static bool select_one_launch(int32_t n_cand, int32_t n_chunks, int32_t pages_per_chunk) {
    if (n_chunks == 0) return n_cand <= kFusedMaxCand;
    return (int64_t)n_chunks * pages_per_chunk <= kFusedMaxCand;
}

SelectWs select_workspace(int32_t dtype, int64_t hd, int32_t n_q, int32_t n_cand,
                          int32_t n_chunks, int32_t pages_per_chunk) {
    SelectWs w;
    // [0, 256): the one-launch paths' completion counters (one; or, in two
    // levels, the final one and one per column group), zero between calls;
    // the three-launch path leaves them alone
    size_t off = 256;
    w.one_launch = select_one_launch(n_cand, n_chunks, pages_per_chunk);
    w.wide = false;
    if (!w.one_launch && select_wide(n_cand, n_chunks) &&
        colsum_plan(dtype, hd, n_q, kFusedRowsPerLane, kWideGroupChunks).groups < 64) {
        // [0, 256) holds the final counter, then one counter per column group
        w.wide = true;
        w.q_plan = colsum_plan(dtype, hd, n_q, kFusedRowsPerLane, kWideGroupChunks);
        w.groups = w.q_plan.groups;
        w.partial_q = off;    // [row blocks][hd] column sums
        off = align_up(off + (size_t)w.q_plan.blocks * hd * sizeof(double), 256);
        w.alpha_part = off;   // [groups][n_cand]
        off = align_up(off + (size_t)w.groups * n_cand * sizeof(double), 256);
        w.cosine = w.cand = 0;
        w.total = off;
        return w;
    }
    if (w.one_launch) {
        // scored candidates: the list, or with a prompt stage every chunk's pages
        const int64_t n_all = n_chunks > 0 ? (int64_t)n_chunks * pages_per_chunk : n_cand;
        w.q_plan = colsum_plan(dtype, hd, n_q, kFusedRowsPerLane, kFusedGroupChunks);
        w.groups = w.q_plan.groups;
        w.alpha_part = off;   // [groups * row blocks][n_all]
        off = align_up(off + (size_t)w.q_plan.groups * w.q_plan.blocks * n_all * sizeof(double), 256);
        w.cosine = 0;
        if (n_chunks > 0) {   // [n_chunks] prompt cosines
            w.cosine = off;
            off = align_up(off + (size_t)n_chunks * sizeof(double), 256);
        }
        w.partial_q = w.cand = 0;
        w.total = off;
        return w;
    }
    w.q_plan = colsum_plan(dtype, hd, n_q, kQRowsPerLane);
    w.groups = (int)((hd + kGroupCols - 1) / kGroupCols);
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

// Total order of (score, id, position) items: score descending, then id
// ascending, then list position ascending (a repeated id is taken once per
// occurrence, in list order).  An id < 0 marks "no item" and ranks last.
__device__ __forceinline__ bool ranks_before(double sa, int ia, int ja, double sb, int ib, int jb) {
    const bool tie = (sa == sb) & ((ia < ib) | ((ia == ib) & (ja < jb)));
    return (ia >= 0) & ((ib < 0) | (sa > sb) | tie);
}

// Butterfly argmax over the 64 lanes of a wavefront; every lane ends with the
// same winner because the order is total.
// x from another lane of the wavefront by a DPP lane permutation (CTRL; every
// lane's source exists), both 32-bit halves.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
    const long long u = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)u, CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), CTRL, 0xf, 0xf, false);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Maximum over the 64 lanes, in every lane: within quads (DPP quad_perm
// [1,0,3,2], [2,3,0,1]), half-rows (row_half_mirror) and rows (row_mirror),
// then across rows and halves (permlane16 / permlane32 swaps).  All lanes
// must be active.
__device__ __forceinline__ double wave_max_f64(double m) {
    m = fmax(m, dpp_f64<0xb1>(m));
    m = fmax(m, dpp_f64<0x4e>(m));
    m = fmax(m, dpp_f64<0x141>(m));
    m = fmax(m, dpp_f64<0x140>(m));
    {
        const long long u = __double_as_longlong(m);
        const auto lo = __builtin_amdgcn_permlane16_swap((unsigned)u, (unsigned)u, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap((unsigned)(u >> 32), (unsigned)(u >> 32),
                                                         false, false);
        m = fmax(__longlong_as_double(((long long)hi[0] << 32) | lo[0]),
                 __longlong_as_double(((long long)hi[1] << 32) | lo[1]));
    }
    {
        const long long u = __double_as_longlong(m);
        const auto lo = __builtin_amdgcn_permlane32_swap((unsigned)u, (unsigned)u, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((unsigned)(u >> 32), (unsigned)(u >> 32),
                                                         false, false);
        m = fmax(__longlong_as_double(((long long)hi[0] << 32) | lo[0]),
                 __longlong_as_double(((long long)hi[1] << 32) | lo[1]));
    }
    return m;
}

// The highest score among the lanes holding an item comes from a maximum over
// the score alone; a ballot then finds the lanes holding it, and only when
// several do (a tie) does a butterfly over the whole order run among them.
// All 64 lanes must be active.
__device__ __forceinline__ void wave_argmax(double &s, int &id, int &pos) {
    const double m = wave_max_f64(id >= 0 ? s : -INFINITY);
    const unsigned long long tied = __builtin_amdgcn_ballot_w64(id >= 0 && s == m);
    if (tied == 0ull) {   // no lane holds an item
        s = 0.0;
        id = -1;
        pos = -1;
        return;
    }
    if ((tied & (tied - 1ull)) == 0ull) {   // one lane holds the highest score
        const int l = __builtin_ctzll(tied);
        s = m;
        id = __builtin_amdgcn_readlane(id, l);
        pos = __builtin_amdgcn_readlane(pos, l);
        return;
    }
    if (!((tied >> (threadIdx.x & 63)) & 1ull)) {
        s = 0.0;
        id = -1;
        pos = -1;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double os = __shfl_xor(s, off, 64);
        const int oid = __shfl_xor(id, off, 64);
        const int opos = __shfl_xor(pos, off, 64);
        if (ranks_before(os, oid, opos, s, id, pos)) {
            s = os;
            id = oid;
            pos = opos;
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

// Cosine of the current prompt `cur` with a past chunk's prompt `pm` (fp64,
// every thread of the block, a fixed order); the result is in thread 0.  A
// prompt of zero norm has no direction: its cosine is -inf, so that chunk
// ranks after every other (ties to the lower chunk id), and a zero current
// prompt leaves the chunks in id order.  `lds` holds 3 * blockDim.x doubles.
__device__ double prompt_cosine(const float *__restrict__ cur, const float *__restrict__ pm,
                                int emb_dim, double *lds) {
    double dot = 0.0, nn = 0.0, pp = 0.0;
    for (int e = threadIdx.x; e < emb_dim; e += blockDim.x) {
        const double a = (double)cur[e];
        const double c = (double)pm[e];
        dot += a * c;
        nn += c * c;
        pp += a * a;
    }
    block_sum3(dot, nn, pp, lds);
    return (pp > 0.0 && nn > 0.0) ? dot / (sqrt(pp) * sqrt(nn)) : -INFINITY;
}

// Blocks [0, groups * q_blocks): column sums of Q, block b -> (column group
// b % groups, row block b / groups).  Blocks after those: prompt cosines.
template <bool BF16>
__global__ __launch_bounds__(256) void k_select_stage1(
    const uint4 *__restrict__ q, int64_t n_q, int chunks, int group_chunks, int groups,
    int row_lanes, int rows_per_block, int q_blocks, double *__restrict__ partial_q,
    const float *__restrict__ chunk_prompts, const float *__restrict__ cur_prompt, int emb_dim,
    double *__restrict__ cosine) {
    __shared__ double lds[256 * (BF16 ? 8 : 4)];   // >= 3 * blockDim.x for block_sum3
    constexpr int VEC = BF16 ? 8 : 4;
    const int b = blockIdx.x;
    if (b < groups * q_blocks) {
        const int g = b % groups, rb = b / groups;
        colsum_block<BF16>(q, nullptr, nullptr, nullptr, n_q, chunks, g * group_chunks,
                           group_chunks, row_lanes, rows_per_block, rb, lds,
                           partial_q + (int64_t)rb * chunks * VEC);
        return;
    }
    // prompt stage: cosine of the current prompt with chunk m's prompt
    const int m = b - groups * q_blocks;
    const double cs = prompt_cosine(cur_prompt, chunk_prompts + (int64_t)m * emb_dim, emb_dim, lds);
    if (threadIdx.x == 0) cosine[m] = cs;
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
        int bid = -1, bpos = -1;
        for (int u = 0; u < per_lane; ++u) {
            const int m = lane + 64 * u;
            if (m >= n_chunks || ((mine >> u) & 1ull)) continue;
            const double cs = cosine[m];
            if (ranks_before(cs, m, m, bs, bid, bpos)) {
                bs = cs;
                bid = m;
                bpos = m;
            }
        }
        wave_argmax(bs, bid, bpos);
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

// The scores of the candidates and their ranking, run by every thread of one
// block: alpha_of(j) gives candidate j's unscaled score (a sum in a fixed
// order), id_of(j) its page id.  With a sliding window (n_recent > 0,
// Inferix summary, "Dual access patterns": range access to the most recent
// pages plus index-based selective fetch), the window's ids are written
// first and take no part in the ranking, which fills the k_p entries after
// them; their scores are still reported.  MAXC >= n_cand.
// NT: the block's thread count.  (The block size is a template argument, not
// blockDim: reading it, or __syncthreads_count, fetches the launch's size
// from memory on the critical path.)
template <int NT, int MAXC, int RANK_MAX = NT, class AlphaOf, class IdOf>
__device__ void finish_select(AlphaOf alpha_of, IdOf id_of, int n_cand, int max_pages,
                              double denom, int k_p, const int32_t *__restrict__ recent,
                              int n_recent, int32_t *__restrict__ out_idx,
                              double *__restrict__ out_scores) {
    __shared__ double sc[MAXC];
    __shared__ int ids[MAXC];
    __shared__ int win[WA_MAX_WINDOW];
    const int t = threadIdx.x;
    for (int r = t; r < n_recent; r += NT) {
        const int id = recent[r];
        win[r] = id;
        out_idx[r] = id;
    }
    __syncthreads();
    out_idx += n_recent;
    // an id outside the pool scores -inf and is never selected
    for (int j = t; j < n_cand; j += NT) {
        const double v = alpha_of(j);
        const int id = id_of(j);
        const bool valid = id >= 0 && id < max_pages;
        const double s = valid ? v / denom : -INFINITY;
        bool in_window = false;
        for (int w = 0; w < n_recent; ++w) in_window |= win[w] == id;
        sc[j] = s;
        ids[j] = valid && !in_window ? id : -1;
        if (out_scores) out_scores[j] = s;
    }
    __syncthreads();

    if (n_cand <= RANK_MAX) {
        // rank of candidate j = number of candidates ordered before it, found
        // by lpc consecutive lanes (lpc = NT / ncp, at most a wavefront; ncp =
        // n_cand rounded up to a power of two): lane sub compares candidates
        // sub, sub + lpc, ... with j, then the lanes' counts are added in a
        // butterfly (rank in the low 16 bits, valid candidates in the high).
        // The lanes of candidate 0 fill the places past the valid ones with -1.
        static_assert((NT & (NT - 1)) == 0, "block size must be a power of two");
        int sh = 0;                 // ncp = 1 << sh
        while ((1 << sh) < n_cand) ++sh;
        constexpr int kLogNT = __builtin_ctz(NT);
        const int lsh = kLogNT - sh < 6 ? kLogNT - sh : 6;
        const int lpc = 1 << lsh;
        const int j = t >> lsh, sub = t & (lpc - 1);
        const bool live = j < n_cand && ids[j] >= 0;
        const double s = live ? sc[j] : 0.0;
        const int id = live ? ids[j] : -1;
        int x = 0;
        for (int i = sub; i < n_cand; i += lpc) {
            const int ii = ids[i];
            x += (int)ranks_before(sc[i], ii, i, s, id, j) + (ii >= 0 ? 1 << 16 : 0);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1)
            if (off < lpc) x += __shfl_xor(x, off, 64);
        const int rank = x & 0xffff, valid = x >> 16;
        if (sub == 0 && live && rank < k_p) out_idx[rank] = id;
        if (j == 0)
            for (int r = valid + sub; r < k_p; r += lpc) out_idx[r] = -1;
        return;
    }

    // many candidates: wavefront 0 takes K_p rounds of an argmax; candidate
    // j lives in lane j % 64, slot j / 64
    if (t >= 64) return;
    const int lane = t;
    if constexpr (MAXC <= 4 * 64) {
        // at most 4 candidates per lane: held in registers for every round
        constexpr int PL = (MAXC + 63) / 64;
        double sv[PL];
        int iv[PL];
#pragma unroll
        for (int u = 0; u < PL; ++u) {
            const int j = lane + 64 * u;
            sv[u] = j < n_cand ? sc[j] : 0.0;
            iv[u] = j < n_cand ? ids[j] : -1;   // -1: no item, never ranked
        }
        unsigned taken = 0u;
        for (int r = 0; r < k_p; ++r) {
            double bs = 0.0;
            int bid = -1, bpos = -1;
#pragma unroll
            for (int u = 0; u < PL; ++u) {
                const int j = lane + 64 * u;
                if (!((taken >> u) & 1u) && ranks_before(sv[u], iv[u], j, bs, bid, bpos)) {
                    bs = sv[u];
                    bid = iv[u];
                    bpos = j;
                }
            }
            wave_argmax(bs, bid, bpos);
            if (bpos >= 0 && (bpos & 63) == lane) taken |= 1u << (bpos >> 6);
            if (lane == 0) out_idx[r] = bid;     // -1 when nothing valid is left
        }
        return;
    }
    const int per_lane = (n_cand + 63) / 64;   // <= 64
    unsigned long long taken = 0ull;
    for (int u = 0; u < per_lane; ++u) {
        const int j = lane + 64 * u;
        if (j >= n_cand || ids[j] < 0) taken |= 1ull << u;
    }
    for (int r = 0; r < k_p; ++r) {
        double bs = 0.0;
        int bid = -1, bpos = -1;
        for (int u = 0; u < per_lane; ++u) {
            if ((taken >> u) & 1ull) continue;
            const int j = lane + 64 * u;
            if (ranks_before(sc[j], ids[j], j, bs, bid, bpos)) {
                bs = sc[j];
                bid = ids[j];
                bpos = j;
            }
        }
        wave_argmax(bs, bid, bpos);
        if (bpos >= 0 && (bpos & 63) == lane) taken |= 1ull << (bpos >> 6);
        if (lane == 0) out_idx[r] = bid;     // -1 when nothing valid is left
    }
}

// One block of kStage3Threads threads: alpha_j = the group partials of
// candidate j added in group order.
__global__ __launch_bounds__(kStage3Threads) void k_select_stage3(
    const double *__restrict__ alpha_part, int groups, int n_cand,
    const int32_t *__restrict__ cand_ws, int max_pages, double sqrt_d, int k_p,
    const int32_t *__restrict__ recent, int n_recent,
    int32_t *__restrict__ out_idx, double *__restrict__ out_scores) {
    auto alpha_of = [&](int j) -> double {
        double v = 0.0;
        for (int g0 = 0; g0 < groups; g0 += 16) {
            double x[16];   // 16 loads in flight, then added in group order
#pragma unroll
            for (int u = 0; u < 16; ++u)
                x[u] = g0 + u < groups ? alpha_part[(int64_t)(g0 + u) * n_cand + j] : 0.0;
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (g0 + u < groups) v += x[u];
        }
        return v;
    };
    auto id_of = [&](int j) -> int { return cand_ws[j]; };
    finish_select<kStage3Threads, WA_MAX_CANDIDATES>(alpha_of, id_of, n_cand, max_pages, sqrt_d,
                                                     k_p, recent, n_recent, out_idx, out_scores);
}

// The one-launch path: kFusedThreads threads per block, block b < blocks ->
// (column group b % groups, row block b / groups), `blocks` = groups * row
// blocks.  With a prompt stage (PROMPT) the candidates scored are every page
// of every past chunk (cand_in = chunk_pages, n_cand = n_chunks x
// pages_per_chunk), and blocks blocks ... blocks + n_chunks - 1 each form one
// chunk's prompt cosine; the last block ranks the chunks, keeps the pages of
// the first n_keep in rank order, and ranks those.
static constexpr int kFusedThreads = 256;
struct OnePrompt {
    const float *chunk_prompts;   // [n_chunks][emb_dim]
    const float *cur_prompt;      // [emb_dim]
    int emb_dim, n_chunks, pages_per_chunk, n_keep;
    int32_t *out_chunks;          // [n_keep] or null
    int32_t *out_cand;            // [n_keep * pages_per_chunk] or null
    double *cosine;               // workspace [n_chunks]
};
template <bool BF16, bool PROMPT>
__global__ __launch_bounds__(kFusedThreads) void k_select_one(
    const uint4 *__restrict__ q, int64_t n_q, int chunks, int group_chunks, int groups,
    int row_lanes, int rows_per_block, int blocks, int grid_blocks,
    const double *__restrict__ page_means, int64_t hd, int max_pages,
    const int32_t *__restrict__ cand_in, int n_cand, double denom, int k_p,
    const int32_t *__restrict__ recent, int n_recent, int *__restrict__ counter,
    double *__restrict__ alpha_blk, int32_t *__restrict__ out_idx,
    double *__restrict__ out_scores, OnePrompt pr) {
    constexpr int VEC = BF16 ? 8 : 4;
    __shared__ double lds[kFusedThreads * VEC];   // row-lane partials of colsum_block
    __shared__ double colsum[64 * VEC];           // this block's column sums
    __shared__ double alpha[kFusedThreads];
    __shared__ int last;
    const int t = threadIdx.x, b = blockIdx.x;
    int ncp = 4;
    while (ncp < n_cand) ncp <<= 1;
    if (PROMPT && b >= blocks) {
        // prompt cosine of chunk b - blocks
        const int m = b - blocks;
        const double cs = prompt_cosine(pr.cur_prompt, pr.chunk_prompts + (int64_t)m * pr.emb_dim,
                                        pr.emb_dim, lds);
        if (t == 0) __hip_atomic_store(pr.cosine + m, cs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        const int g = b % groups, rb = b / groups;
        const int c0 = g * group_chunks;
        const int gw = min(group_chunks, chunks - c0) * VEC;   // columns in this group
        colsum_block<BF16, kFusedBatch>(q, nullptr, nullptr, nullptr, n_q, chunks, c0, group_chunks,
                                        row_lanes, rows_per_block, rb, lds, colsum, c0 * VEC);
        __syncthreads();

        // candidate j's dot product with this block's column sums: tpc = 256 / ncp
        // consecutive lanes per candidate (ncp = n_cand rounded up to a power of
        // two, at least 4); lane sub adds columns sub, sub + tpc, ... in order,
        // 8 loads in flight at a time, then a butterfly over the tpc lanes
        const int tpc = kFusedThreads / ncp;
        {
            const int j = t / tpc, sub = t % tpc;
            const int id = j < n_cand ? (cand_in ? cand_in[j] : j) : -1;
            double v = 0.0;
            if (id >= 0 && id < max_pages) {
                const double *pm = page_means + (int64_t)id * hd + (int64_t)c0 * VEC;
                int c = sub;
                for (; c + 7 * tpc < gw; c += 8 * tpc) {
                    double x[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) x[u] = pm[c + u * tpc];
#pragma unroll
                    for (int u = 0; u < 8; ++u) v += colsum[c + u * tpc] * x[u];
                }
                for (; c < gw; c += tpc) v += colsum[c] * pm[c];
            }
            for (int off = tpc >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            if (sub == 0 && j < n_cand)
                __hip_atomic_store(alpha_blk + (int64_t)b * n_cand + j, v, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // this wavefront's stores have reached the coherent level; once every
    // wavefront is past the barrier, the block counts itself done
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t == 0)
        last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               grid_blocks - 1;
    __syncthreads();
    if (!last) return;

    // the last block: alpha_j = block partials of candidate j added in block
    // order (slice sl of the kFusedThreads / ncp slices adds blocks sl,
    // sl + slices, ...; then the slices in order)
    const int slices = kFusedThreads / ncp;
    {
        const int j = t % ncp, sl = t / ncp;
        double v = 0.0;
        if (j < n_cand) {
            const int terms = sl < blocks ? (blocks - 1 - sl) / slices + 1 : 0;
            for (int u0 = 0; u0 < terms; u0 += 16) {
                double x[16];   // up to 16 loads in flight, then added in block order
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    x[u] = u0 + u < terms
                               ? __hip_atomic_load(alpha_blk + (int64_t)(sl + (u0 + u) * slices) * n_cand + j,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                               : 0.0;
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    if (u0 + u < terms) v += x[u];
            }
        }
        alpha[t] = v;   // alpha[sl * ncp + j]
    }
    __syncthreads();
    auto slice_sum = [&](int j) -> double {
        double v = 0.0;
        for (int sl = 0; sl < slices; ++sl) v += alpha[sl * ncp + j];
        return v;
    };
    if constexpr (PROMPT) {
        // the chunks in (cosine desc, id asc) order, the first n_keep kept;
        // candidate j is page j % ppc of the (j / ppc)-th kept chunk
        __shared__ double cosl[kFusedMaxCand];
        __shared__ int kept[kFusedMaxCand];
        for (int m = t; m < pr.n_chunks; m += kFusedThreads)
            cosl[m] = __hip_atomic_load(pr.cosine + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (t < 64) rank_chunks(cosl, pr.n_chunks, pr.n_keep, kept);
        __syncthreads();
        const int ppc = pr.pages_per_chunk, n_kept = pr.n_keep * ppc;
        auto src = [&](int j) -> int { return kept[j / ppc] * ppc + j % ppc; };
        if (pr.out_chunks)
            for (int r = t; r < pr.n_keep; r += kFusedThreads) pr.out_chunks[r] = kept[r];
        if (pr.out_cand)
            for (int j = t; j < n_kept; j += kFusedThreads) pr.out_cand[j] = cand_in[src(j)];
        auto alpha_of = [&](int j) -> double { return slice_sum(src(j)); };
        auto id_of = [&](int j) -> int { return cand_in[src(j)]; };
        finish_select<kFusedThreads, kFusedMaxCand>(alpha_of, id_of, n_kept, max_pages, denom,
                                                    k_p, recent, n_recent, out_idx, out_scores);
    } else {
        auto id_of = [&](int j) -> int { return cand_in ? cand_in[j] : j; };
        finish_select<kFusedThreads, kFusedMaxCand>(slice_sum, id_of, n_cand, max_pages, denom,
                                                    k_p, recent, n_recent, out_idx, out_scores);
    }
    // ready for the next call on this workspace
    if (t == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The two-level one-launch path (kFusedMaxCand < n_cand <= kWideMaxCand, no
// prompt stage).  Block (column group g, row block rb) forms the fp64 column
// sums of its rows of Q over the group's columns and publishes them
// (agent-scope stores); the last row block of group g to finish (its own
// counter) adds the group's row-block sums in row-block order and forms each
// candidate's partial dot product over the group's columns; the last group to
// finish (the final counter) adds the group partials in group order, scales,
// ranks and writes the result, then clears every counter.
template <bool BF16>
__global__ __launch_bounds__(kFusedThreads) void k_select_wide(
    const uint4 *__restrict__ q, int64_t n_q, int chunks, int group_chunks, int groups,
    int row_lanes, int rows_per_block, int row_blocks, const double *__restrict__ page_means,
    int64_t hd, int max_pages, const int32_t *__restrict__ cand_in, int n_cand, double denom,
    int k_p, const int32_t *__restrict__ recent, int n_recent, int *__restrict__ counters,
    double *__restrict__ colpart, double *__restrict__ gpart, int32_t *__restrict__ out_idx,
    double *__restrict__ out_scores) {
    constexpr int VEC = BF16 ? 8 : 4;
    constexpr int NT = kFusedThreads;
    __shared__ double lds[NT * VEC];    // row-lane partials of colsum_block, then a scratch
    __shared__ double colsum[64 * VEC];
    __shared__ double alpha[kWideMaxCand];
    __shared__ int cid[kWideMaxCand];
    __shared__ int flag;
    const int t = threadIdx.x, b = blockIdx.x;
    const int g = b % groups, rb = b / groups;
    const int c0 = g * group_chunks;
    const int gw = min(group_chunks, chunks - c0) * VEC;   // columns in this group
    colsum_block<BF16, kFusedBatch>(q, nullptr, nullptr, nullptr, n_q, chunks, c0, group_chunks,
                                    row_lanes, rows_per_block, rb, lds, colsum, c0 * VEC);
    __syncthreads();
    double *const my_cols = colpart + (int64_t)rb * hd + (int64_t)c0 * VEC;
    for (int c = t; c < gw; c += NT)
        __hip_atomic_store(my_cols + c, colsum[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t == 0)
        flag = __hip_atomic_fetch_add(counters + 1 + g, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == row_blocks - 1;
    __syncthreads();
    if (!flag) return;

    // last row block of group g: column c's sum over the row blocks, split
    // over `splits` lanes (lane s adds row blocks s, s + splits, ... in order,
    // then the splits are added in order)
    const int splits = NT / gw;   // >= 1 (gw <= kWideGroupChunks vectors)
    // the candidate ids, read while the column sums are on their way
    for (int j = t; j < n_cand; j += NT) cid[j] = cand_in ? cand_in[j] : j;
    {
        const int c = t % gw, sp = t / gw;
        double v = 0.0;
        if (sp < splits) {
            const double *col = colpart + (int64_t)c0 * VEC + c;
            const int terms = sp < row_blocks ? (row_blocks - 1 - sp) / splits + 1 : 0;
            for (int u0 = 0; u0 < terms; u0 += 16) {
                double x[16];
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    x[u] = u0 + u < terms
                               ? __hip_atomic_load(col + (int64_t)(sp + (u0 + u) * splits) * hd,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                               : 0.0;
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    if (u0 + u < terms) v += x[u];
            }
            lds[sp * gw + c] = v;
        }
    }
    __syncthreads();
    if (t < gw) {
        double v = 0.0;
        for (int sp = 0; sp < splits; ++sp) v += lds[sp * gw + t];
        colsum[t] = v;   // the group's column sums over all of Q
    }
    __syncthreads();

    // partial dot products over the group's columns: 8 lanes per candidate,
    // 32 candidates per round, kWideRounds rounds' loads in flight together;
    // lane sub adds columns sub, sub + 8, ... in order, then a butterfly over
    // the 8 lanes
    {
        constexpr int U = kWideGroupChunks * VEC / 8;   // columns of a lane per candidate
        const int sub = t & 7, slot = t >> 3;
        for (int j0 = 0; j0 < n_cand; j0 += (NT / 8) * kWideRounds) {
            double x[kWideRounds][U];
#pragma unroll
            for (int r = 0; r < kWideRounds; ++r) {
                const int j = j0 + (NT / 8) * r + slot;
                const int id = j < n_cand ? cid[j] : -1;
                const bool ok = id >= 0 && id < max_pages;
                const double *pm = page_means + (int64_t)(ok ? id : 0) * hd + (int64_t)c0 * VEC;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = sub + 8 * u;
                    x[r][u] = ok && c < gw ? pm[c] : 0.0;
                }
            }
#pragma unroll
            for (int r = 0; r < kWideRounds; ++r) {
                double v = 0.0;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = sub + 8 * u;
                    if (c < gw) v += colsum[c] * x[r][u];
                }
                v += __shfl_xor(v, 4, 64);
                v += __shfl_xor(v, 2, 64);
                v += __shfl_xor(v, 1, 64);
                const int j = j0 + (NT / 8) * r + slot;
                if (sub == 0 && j < n_cand)
                    __hip_atomic_store(gpart + (int64_t)g * n_cand + j, v, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t == 0)
        flag = __hip_atomic_fetch_add(counters, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               groups - 1;
    __syncthreads();
    if (!flag) return;

    // the last group: alpha_j = the group partials of candidate j in group order
    for (int j = t; j < n_cand; j += NT) {
        double v = 0.0;
        for (int g0 = 0; g0 < groups; g0 += 32) {
            double x[32];   // up to 32 loads in flight, then added in group order
#pragma unroll
            for (int u = 0; u < 32; ++u)
                x[u] = g0 + u < groups
                           ? __hip_atomic_load(gpart + (int64_t)(g0 + u) * n_cand + j,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : 0.0;
#pragma unroll
            for (int u = 0; u < 32; ++u)
                if (g0 + u < groups) v += x[u];
        }
        alpha[j] = v;
    }
    __syncthreads();
    auto alpha_of = [&](int j) -> double { return alpha[j]; };
    auto id_of = [&](int j) -> int { return cid[j]; };
    finish_select<NT, kWideMaxCand, kFusedMaxCand>(alpha_of, id_of, n_cand, max_pages, denom, k_p,
                                                   recent, n_recent, out_idx, out_scores);
    // ready for the next call on this workspace
    if (t <= groups) __hip_atomic_store(counters + t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_select(const wa_layout &L, const void *q, int32_t n_q, const double *page_means,
                         const int32_t *cand, int32_t n_cand, const wa_prompt_stage *prompt,
                         const int32_t *recent, int32_t n_recent, int32_t k_p, int32_t *out_idx,
                         double *out_scores, void *ws, hipStream_t s) {
    const int64_t hd = (int64_t)L.n_heads * L.head_dim;
    const int n_chunks = prompt ? prompt->n_chunks : 0;
    const SelectWs w = select_workspace(L.dtype, hd, n_q, n_cand, n_chunks,
                                        prompt ? prompt->pages_per_chunk : 0);
    char *base = (char *)ws;
    if (w.one_launch) {
        const ColSumPlan &p = w.q_plan;
        const double denom = (double)n_q * sqrt((double)L.head_dim);
        OnePrompt pr{};
        int n_scored = n_cand;
        const int32_t *scored = cand;
        if (prompt) {
            pr = OnePrompt{prompt->chunk_prompts, prompt->cur_prompt, prompt->emb_dim, n_chunks,
                           prompt->pages_per_chunk, prompt->n_keep, prompt->out_chunks,
                           prompt->out_cand, (double *)(base + w.cosine)};
            n_scored = n_chunks * prompt->pages_per_chunk;
            scored = prompt->chunk_pages;
        }
        const int blocks = p.groups * p.blocks;
        const int grid = blocks + n_chunks;
        auto launch = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, dim3(grid), dim3(kFusedThreads), 0, s, (const uint4 *)q,
                               (int64_t)n_q, p.chunks, p.group_chunks, p.groups, p.row_lanes,
                               p.rows_per_block, blocks, grid, page_means, hd, L.max_pages, scored,
                               n_scored, denom, k_p, recent, n_recent, (int *)base,
                               (double *)(base + w.alpha_part), out_idx, out_scores, pr);
        };
        if (L.dtype == WA_BF16) {
            if (prompt) launch(k_select_one<true, true>);
            else launch(k_select_one<true, false>);
        } else {
            if (prompt) launch(k_select_one<false, true>);
            else launch(k_select_one<false, false>);
        }
        return hipGetLastError();
    }
    if (w.wide) {
        const ColSumPlan &p = w.q_plan;
        const double denom = (double)n_q * sqrt((double)L.head_dim);
        auto launch = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, dim3(p.groups * p.blocks), dim3(kFusedThreads), 0, s,
                               (const uint4 *)q, (int64_t)n_q, p.chunks, p.group_chunks, p.groups,
                               p.row_lanes, p.rows_per_block, p.blocks, page_means, hd,
                               L.max_pages, cand, n_cand, denom, k_p, recent, n_recent,
                               (int *)base, (double *)(base + w.partial_q),
                               (double *)(base + w.alpha_part), out_idx, out_scores);
        };
        if (L.dtype == WA_BF16) launch(k_select_wide<true>);
        else launch(k_select_wide<false>);
        return hipGetLastError();
    }
    double *partial_q = (double *)(base + w.partial_q);
    double *cosine = prompt ? (double *)(base + w.cosine) : nullptr;
    double *alpha_part = (double *)(base + w.alpha_part);
    int32_t *cand_ws = (int32_t *)(base + w.cand);
    const ColSumPlan &p = w.q_plan;

    const int blocks1 = p.groups * p.blocks + n_chunks;
    const float *cp = prompt ? prompt->chunk_prompts : nullptr;
    const float *cur = prompt ? prompt->cur_prompt : nullptr;
    const int emb = prompt ? prompt->emb_dim : 0;
    if (L.dtype == WA_BF16)
        hipLaunchKernelGGL(k_select_stage1<true>, dim3(blocks1), dim3(p.threads), 0, s,
                           (const uint4 *)q, (int64_t)n_q, p.chunks, p.group_chunks, p.groups,
                           p.row_lanes, p.rows_per_block, p.blocks, partial_q, cp, cur, emb,
                           cosine);
    else
        hipLaunchKernelGGL(k_select_stage1<false>, dim3(blocks1), dim3(p.threads), 0, s,
                           (const uint4 *)q, (int64_t)n_q, p.chunks, p.group_chunks, p.groups,
                           p.row_lanes, p.rows_per_block, p.blocks, partial_q, cp, cur, emb,
                           cosine);
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

    hipLaunchKernelGGL(k_select_stage3, dim3(1), dim3(kStage3Threads), 0, s,
                       (const double *)alpha_part, w.groups, n_cand, (const int32_t *)cand_ws,
                       L.max_pages, sqrt((double)L.head_dim), k_p, recent, n_recent, out_idx,
                       out_scores);
    return hipGetLastError();
}

}  // namespace wa
