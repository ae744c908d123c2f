// HSA sparse branch, block selection (WorldAttention review, "HSA: Dual
// Branches of Linear + Sparse": the retrieved keys are cut into blocks, 128
// keys for the past pages and 64 for the current chunk; a pooled attention
// map picks, per head, the fewest blocks whose cumulative attention mass
// reaches a threshold tau_h; attention then runs on the selected blocks only).
//
// Readings (the page leaves them open): queries are pooled per 256-query
// block, the attention kernel's query tile, so that one block list serves a
// whole workgroup; the map is a softmax over the key blocks of
// (mean query . mean key) * scale, unweighted by block size; tau_h is given
// per head (the page derives it from the head's Gini coefficient, but the
// formula did not survive), and the Gini coefficient of every map row is
// reported.
//
//   k_hsa_pool    fp64 sums of the keys of every key block and of the queries
//                 of every query block (column sums, fixed order).
//   k_hsa_scores  block scores (mean query . mean key) * scale in fp64 for
//                 every (head, query block, key block), 16 x 16 per
//                 workgroup from LDS, so that each key-block mean is read
//                 once per 16 query blocks.
//   k_hsa_select  one workgroup per (head, query block): softmax of its
//                 scores, a bitonic sort into (mass desc, block asc) in the
//                 registers of one wavefront, the Gini coefficient, the
//                 shortest prefix in that order whose running sum reaches
//                 tau_h (at least one block), and the selected blocks' 64-key
//                 tiles in ascending order.
#include <math.h>

#include "colsum.h"
#include "wa_internal.h"

namespace wa {

static constexpr int kHsaInter = WA_HSA_CTX_BLOCK;   // keys per context block
static constexpr int kHsaIntra = WA_HSA_OWN_BLOCK;   // keys per own block
static constexpr int kHsaQBlock = WA_HSA_Q_BLOCK;    // queries per pooled query block
static constexpr int kHsaRowLanes = 4;               // column-sum row lanes
static constexpr int kHsaThreads = 256;
static_assert(WA_MAX_HSA_BLOCKS <= 64 * 32, "the sort holds at most 32 blocks per lane");

HsaShape hsa_shape(int32_t n_heads, int32_t n_q, int32_t n_ctx, int32_t n_own) {
    HsaShape w;
    w.nb_ctx = (n_ctx + kHsaInter - 1) / kHsaInter;
    w.nb_own = (n_own + kHsaIntra - 1) / kHsaIntra;
    w.q_blocks = (n_q + kHsaQBlock - 1) / kHsaQBlock;
    w.items = w.q_blocks * n_heads;
    w.n_tiles = (int32_t)(((int64_t)n_ctx + n_own + 63) / 64);
    return w;
}

static size_t hsa_ksum_bytes(int64_t hd, const HsaShape &w) {
    return align_up((size_t)(w.nb_ctx + w.nb_own) * hd * sizeof(double), 256);
}
static size_t hsa_qsum_bytes(int64_t hd, const HsaShape &w) {
    return align_up((size_t)w.q_blocks * hd * sizeof(double), 256);
}

// key-block sums, query-block sums, scores [items][nb]
size_t hsa_workspace_bytes(int64_t hd, const HsaShape &w) {
    return hsa_ksum_bytes(hd, w) + hsa_qsum_bytes(hd, w) +
           (size_t)w.items * (w.nb_ctx + w.nb_own) * sizeof(double);
}

// blockIdx.x: column group; blockIdx.y + y0: a context key block, an own key
// block or a query block, in that order (y0 = nb_ctx skips the context
// blocks, whose sums an earlier call left in place).  Each writes the column
// sums of its rows.
template <bool BF16>
__global__ __launch_bounds__(kHsaThreads) void k_hsa_pool(
    const uint4 *__restrict__ k_ctx, int n_ctx, const uint4 *__restrict__ k_own, int n_own,
    const uint4 *__restrict__ q, int n_q, int nb_ctx, int nb_own, int chunks, int group_chunks,
    int hd, int y0, double *__restrict__ ksum, double *__restrict__ qsum) {
    __shared__ double lds[kHsaRowLanes * 64 * (BF16 ? 8 : 4)];
    int y = blockIdx.y + y0;
    const uint4 *x;
    int rows, per_block;
    double *out;
    if (y < nb_ctx) {
        x = k_ctx, rows = n_ctx, per_block = kHsaInter, out = ksum;
    } else if ((y -= nb_ctx) < nb_own) {
        x = k_own, rows = n_own, per_block = kHsaIntra, out = ksum + (int64_t)nb_ctx * hd;
    } else {
        y -= nb_own;
        x = q, rows = n_q, per_block = kHsaQBlock, out = qsum;
    }
    colsum_block<BF16>(x, nullptr, nullptr, nullptr, rows, chunks, blockIdx.x * group_chunks,
                       group_chunks, kHsaRowLanes, per_block, y, lds, out + (int64_t)y * hd);
}

// Scores of 16 query blocks x 16 key blocks of one head: blockIdx.x = key
// block group, blockIdx.y = query block group, blockIdx.z = head.  The means
// (sums / counts) go to LDS (2 x 16 rows of head_dim + 1 doubles, sized at
// launch) with coalesced loads; thread t takes query block t / 16 and key
// block t % 16 and sums the products in four interleaved partial sums
// (dimensions c = 4i + r in partial r, in order), added in a fixed order.
// Rows are padded by one double so that the 16 key rows a wavefront reads
// at one dimension fall in different banks.
static constexpr int kScT = 16;
__global__ __launch_bounds__(kHsaThreads) void k_hsa_scores(
    const double *__restrict__ ksum, const double *__restrict__ qsum, int nb_ctx, int nb_own,
    int n_ctx, int n_own, int n_q, int q_blocks, int hd, int head_dim, double scale,
    double *__restrict__ scores) {
    extern __shared__ double sc_lds[];
    const int ld = head_dim + 1;
    double *qm = sc_lds, *km = sc_lds + kScT * ld;
    const int nb = nb_ctx + nb_own;
    const int j0 = blockIdx.x * kScT, b0 = blockIdx.y * kScT, h = blockIdx.z;
    const int t = threadIdx.x;
    // every load in flight at once: thread t takes elements t + 256 u of the
    // 16 x head_dim query and key tiles
    constexpr int kU = kScT * WA_HSA_MAX_HEAD_DIM / kHsaThreads;
    const int n_el = kScT * head_dim;
    double qv[kU], kv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int e = t + kHsaThreads * u;
        const int r = e / head_dim, c = e - r * head_dim;
        qv[u] = (e < n_el && b0 + r < q_blocks)
                    ? qsum[(int64_t)(b0 + r) * hd + (int64_t)h * head_dim + c] : 0.0;
        kv[u] = (e < n_el && j0 + r < nb)
                    ? ksum[(int64_t)(j0 + r) * hd + (int64_t)h * head_dim + c] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int e = t + kHsaThreads * u;
        if (e >= n_el) continue;
        const int r = e / head_dim, c = e - r * head_dim;
        const int b = b0 + r, j = j0 + r;
        if (b < q_blocks) qm[r * ld + c] = qv[u] / (double)min(kHsaQBlock, n_q - kHsaQBlock * b);
        if (j < nb)
            km[r * ld + c] = kv[u] / (double)(j < nb_ctx ? min(kHsaInter, n_ctx - kHsaInter * j)
                                                   : min(kHsaIntra, n_own - kHsaIntra * (j - nb_ctx)));
    }
    __syncthreads();
    const int rb = t / kScT, rj = t % kScT;
    const int b = b0 + rb, j = j0 + rj;
    if (b >= q_blocks || j >= nb) return;
    const double *qr = qm + rb * ld, *kr = km + rj * ld;
    double p[4] = {0.0, 0.0, 0.0, 0.0};
    int c = 0;
#pragma unroll 2
    for (; c + 3 < head_dim; c += 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] += qr[c + r] * kr[c + r];
    }
    for (int r = 0; c < head_dim; ++c, ++r) p[r] += qr[c] * kr[c];
    scores[((int64_t)h * q_blocks + b) * nb + j] = ((p[0] + p[1]) + (p[2] + p[3])) * scale;
}

// Workgroup reductions and scans in a fixed order: within each wavefront by
// lane shuffles, then over the four wavefronts in wavefront order through
// LDS (`red`: kHsaThreads / 64 slots).  Every thread gets the result.
static constexpr int kHsaWaves = kHsaThreads / 64;
__device__ double hsa_sum(double v, double *red) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = red[0];
    for (int w = 1; w < kHsaWaves; ++w) r += red[w];
    __syncthreads();
    return r;
}
__device__ double hsa_max(double v, double *red) {
    for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = red[0];
    for (int w = 1; w < kHsaWaves; ++w) r = fmax(r, red[w]);
    __syncthreads();
    return r;
}
// Exclusive prefix over the thread index (T = int or double).
template <typename T>
__device__ T hsa_exclusive_scan(T v, T *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    T x = v;
    for (int o = 1; o < 64; o <<= 1) {
        const T y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) red[wave] = x;
    __syncthreads();
    T before = 0;
    for (int w = 0; w < wave; ++w) before += red[w];
    __syncthreads();
    return before + x - v;
}

// Tiles of key block j: a context block holds tiles 2j and 2j+1, or only 2j
// when the context ends 64 keys into it; own block j is tile n_ctx / 64 + j.
__device__ __forceinline__ int hsa_block_tiles(int j, int nb_ctx, int n_ctx) {
    return j < nb_ctx ? (n_ctx - kHsaInter * j >= kHsaInter ? 2 : 1) : 1;
}


// Bitonic sort of 64 R (mass, id) pairs held by one wavefront, element
// x = lane R + e in register e of lane `lane`, into the order hsa_before
// (element 0 first; ids distinct).  Stage k merges runs of k; pass jj
// compares x with x ^ jj.  Passes with jj >= R exchange across lanes
// (lane ^ jj / R, same register: every exchange of the pass is issued
// before the first is used); the others compare two registers of one lane.
// The comparisons are written without short-circuit operators so that they
// compile to predicate logic rather than branches.
__device__ __forceinline__ bool hsa_first(double ma, int ia, double mb, int ib) {
    return (ma > mb) | ((ma == mb) & (ia < ib));
}
template <int R>
__device__ __forceinline__ void hsa_wave_sort(double (&m)[R], int (&id)[R], int lane) {
    for (int k = 2; k <= 64 * R; k <<= 1) {
        for (int jj = k >> 1; jj >= R; jj >>= 1) {
            const int ld = jj / R;
            const bool lower = (lane & ld) == 0;
            double om[R];
            int oi[R];
#pragma unroll
            for (int e = 0; e < R; ++e) {
                om[e] = __shfl_xor(m[e], ld);
                oi[e] = __shfl_xor(id[e], ld);
            }
#pragma unroll
            for (int e = 0; e < R; ++e) {
                const bool fwd = ((lane * R + e) & k) == 0;
                // the lower element of a forward pair keeps the first of the
                // two, the upper one the second; reversed pairs the opposite
                const bool take = hsa_first(om[e], oi[e], m[e], id[e]) ^ (lower != fwd);
                m[e] = take ? om[e] : m[e];
                id[e] = take ? oi[e] : id[e];
            }
        }
#pragma unroll
        for (int jb = R / 2; jb >= 1; jb >>= 1) {
            if (jb >= k) continue;
#pragma unroll
            for (int e = 0; e < R; ++e) {
                const int f = e ^ jb;
                if (f < e) continue;
                const bool fwd = ((lane * R + e) & k) == 0;
                const bool swap = hsa_first(m[f], id[f], m[e], id[e]) ^ !fwd;
                const double me = m[e], mf = m[f];
                const int ie = id[e], jf = id[f];
                m[e] = swap ? mf : me;
                m[f] = swap ? me : mf;
                id[e] = swap ? jf : ie;
                id[f] = swap ? ie : jf;
            }
        }
    }
}

// One workgroup per item.  All threads: the softmax of the item's scores
// (k_hsa_scores) into LDS.  Wavefront 0: the sort into (mass desc, block
// asc) in registers (nb2 = 64 R >= nb slots, padding sorts last), then in
// that order the Gini coefficient
//     G = sum_i sum_j |p_i - p_j| / (2 nb sum p) = sum_k (nb - 1 - 2k) p_(k) / (nb sum p)
// and the running sums S_k = p_(0) + ... + p_(k), non-decreasing, so that the
// shortest prefix reaching tau has m = min(nb, 1 + #{k : S_k < tau}) blocks;
// it flags them.  All threads: the flagged blocks' tiles in block order.
template <int R>
__global__ __launch_bounds__(kHsaThreads) void k_hsa_select(
    const double *__restrict__ scores, int nb_ctx, int nb_own, int n_ctx, int q_blocks,
    const double *__restrict__ tau, int n_tiles, int32_t *__restrict__ tiles,
    int32_t *__restrict__ count, double *__restrict__ gini_out) {
    __shared__ double mass[64 * R];
    __shared__ int flag[64 * R];
    __shared__ double red[kHsaWaves];
    __shared__ int ired[kHsaWaves];
    const int t = threadIdx.x, lane = t & 63;
    const int item = blockIdx.x;
    const int h = item / q_blocks;
    const int nb = nb_ctx + nb_own;
    const double *row = scores + (int64_t)item * nb;

    double mx = -INFINITY;
    for (int j = t; j < nb; j += kHsaThreads) {
        const double v = row[j];
        mass[j] = v;
        mx = fmax(mx, v);
    }
    mx = hsa_max(mx, red);
    double part = 0.0;
    for (int j = t; j < nb; j += kHsaThreads) {
        const double e = exp(mass[j] - mx);
        mass[j] = e;
        part += e;
    }
    const double s = hsa_sum(part, red);
    for (int j = t; j < nb; j += kHsaThreads) {
        mass[j] /= s;
        flag[j] = 0;
    }
    __syncthreads();

    if (t < 64) {
        double m[R];
        int id[R];
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const int x = lane * R + e;
            m[e] = x < nb ? mass[x] : -1.0;   // padding: below every mass, ids nb ...
            id[e] = x;
        }
        hsa_wave_sort<R>(m, id, lane);
        double g = 0.0, ps = 0.0, loc = 0.0;
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const int x = lane * R + e;
            if (x < nb) {
                g += (double)(nb - 1 - 2 * x) * m[e];
                ps += m[e];
                loc += m[e];
            }
        }
        for (int o = 32; o > 0; o >>= 1) {
            g += __shfl_xor(g, o);
            ps += __shfl_xor(ps, o);
        }
        // exclusive prefix of the lanes' sums, then the running sums
        double x_in = loc;
        for (int o = 1; o < 64; o <<= 1) {
            const double y = __shfl_up(x_in, o);
            if (lane >= o) x_in += y;
        }
        double run = x_in - loc;
        const double th = tau[h];
        int below = 0;
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const int x = lane * R + e;
            if (x < nb) {
                run += m[e];
                below += run < th ? 1 : 0;
            }
        }
        for (int o = 32; o > 0; o >>= 1) below += __shfl_xor(below, o);
        const int n_sel = below + 1 < nb ? below + 1 : nb;
#pragma unroll
        for (int e = 0; e < R; ++e)
            if (lane * R + e < n_sel) flag[id[e]] = 1;
        if (gini_out && lane == 0) gini_out[item] = g / ((double)nb * ps);
    }
    __syncthreads();

    // the flagged blocks' tiles, block order: thread t owns blocks
    // [t per, t per + per)
    const int per = (nb + kHsaThreads - 1) / kHsaThreads;
    const int j0 = min(nb, t * per), j1 = min(nb, j0 + per);
    int mine = 0;
    for (int j = j0; j < j1; ++j)
        if (flag[j]) mine += hsa_block_tiles(j, nb_ctx, n_ctx);
    int at = hsa_exclusive_scan(mine, ired);
    if (t == kHsaThreads - 1) count[item] = at + mine;
    int32_t *list = tiles + (int64_t)item * n_tiles;
    const int t_ctx = n_ctx / 64;
    for (int j = j0; j < j1; ++j) {
        if (!flag[j]) continue;
        if (j < nb_ctx) {
            list[at++] = 2 * j;
            if (hsa_block_tiles(j, nb_ctx, n_ctx) == 2) list[at++] = 2 * j + 1;
        } else {
            list[at++] = t_ctx + (j - nb_ctx);
        }
    }
}

hipError_t launch_hsa_select(const wa_layout &L, const void *q, int32_t n_q, const void *k_ctx,
                             int32_t n_ctx, const void *k_own, int32_t n_own, double scale,
                             const double *tau, int32_t *tiles, int32_t *count, double *gini,
                             bool ctx_sums_ready, void *ws, hipStream_t s) {
    const int64_t hd = (int64_t)L.n_heads * L.head_dim;
    const HsaShape w = hsa_shape(L.n_heads, n_q, n_ctx, n_own);
    double *ksum = (double *)ws;
    double *qsum = (double *)((char *)ws + hsa_ksum_bytes(hd, w));
    double *scores = (double *)((char *)ws + hsa_ksum_bytes(hd, w) + hsa_qsum_bytes(hd, w));
    const int vec = 16 / elem_bytes(L.dtype);
    const int chunks = (int)(hd / vec);
    const int group_chunks = chunks < 64 ? chunks : 64;
    const int groups = (chunks + group_chunks - 1) / group_chunks;
    const int y0 = ctx_sums_ready ? w.nb_ctx : 0;
    const dim3 grid((unsigned)groups, (unsigned)(w.nb_ctx + w.nb_own + w.q_blocks - y0));
    if (L.dtype == WA_BF16)
        hipLaunchKernelGGL(k_hsa_pool<true>, grid, dim3(kHsaThreads), 0, s, (const uint4 *)k_ctx,
                           n_ctx, (const uint4 *)k_own, n_own, (const uint4 *)q, n_q, w.nb_ctx,
                           w.nb_own, chunks, group_chunks, (int)hd, y0, ksum, qsum);
    else
        hipLaunchKernelGGL(k_hsa_pool<false>, grid, dim3(kHsaThreads), 0, s, (const uint4 *)k_ctx,
                           n_ctx, (const uint4 *)k_own, n_own, (const uint4 *)q, n_q, w.nb_ctx,
                           w.nb_own, chunks, group_chunks, (int)hd, y0, ksum, qsum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nb = w.nb_ctx + w.nb_own;
    hipLaunchKernelGGL(k_hsa_scores,
                       dim3((unsigned)((nb + kScT - 1) / kScT),
                            (unsigned)((w.q_blocks + kScT - 1) / kScT), (unsigned)L.n_heads),
                       dim3(kHsaThreads), (size_t)2 * kScT * (L.head_dim + 1) * sizeof(double), s,
                       ksum, qsum, w.nb_ctx, w.nb_own, n_ctx, n_own, n_q,
                       w.q_blocks, (int)hd, L.head_dim, scale, scores);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    int nb2 = 64;
    while (nb2 < nb) nb2 <<= 1;
#define WA_HSA_SELECT(R)                                                                          \
    hipLaunchKernelGGL(k_hsa_select<R>, dim3((unsigned)w.items), dim3(kHsaThreads), 0, s, scores, \
                       w.nb_ctx, w.nb_own, n_ctx, w.q_blocks, tau, w.n_tiles, tiles, count, gini)
    switch (nb2 / 64) {
        case 1: WA_HSA_SELECT(1); break;
        case 2: WA_HSA_SELECT(2); break;
        case 4: WA_HSA_SELECT(4); break;
        case 8: WA_HSA_SELECT(8); break;
        case 16: WA_HSA_SELECT(16); break;
        default: WA_HSA_SELECT(32); break;
    }
#undef WA_HSA_SELECT
    return hipGetLastError();
}

}  // namespace wa
