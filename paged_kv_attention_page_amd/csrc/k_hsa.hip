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
//   k_hsa_select  one workgroup per (head, query block): block scores in fp64,
//                 softmax, a bitonic sort by (mass desc, block asc), the Gini
//                 coefficient from the sorted masses, the shortest prefix
//                 whose running sum (in sorted order, sequential) reaches
//                 tau_h, at least one block, and the selected blocks' 64-key
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
static_assert(WA_MAX_HSA_BLOCKS % kHsaThreads == 0, "scan ownership");

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

size_t hsa_workspace_bytes(int64_t hd, const HsaShape &w) {
    return hsa_ksum_bytes(hd, w) + (size_t)w.q_blocks * hd * sizeof(double);
}

// blockIdx.x: column group; blockIdx.y: a context key block, an own key block
// or a query block, in that order.  Each writes the column sums of its rows.
template <bool BF16>
__global__ __launch_bounds__(kHsaThreads) void k_hsa_pool(
    const uint4 *__restrict__ k_ctx, int n_ctx, const uint4 *__restrict__ k_own, int n_own,
    const uint4 *__restrict__ q, int n_q, int nb_ctx, int nb_own, int chunks, int group_chunks,
    int hd, double *__restrict__ ksum, double *__restrict__ qsum) {
    __shared__ double lds[kHsaRowLanes * 64 * (BF16 ? 8 : 4)];
    int y = blockIdx.y;
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

// Fixed-order sum / max over the workgroup (tree over the thread index).
__device__ double hsa_tree(double v, double *red, bool is_max) {
    const int t = threadIdx.x;
    red[t] = v;
    __syncthreads();
    for (int n = kHsaThreads >> 1; n > 0; n >>= 1) {
        if (t < n) red[t] = is_max ? fmax(red[t], red[t + n]) : red[t] + red[t + n];
        __syncthreads();
    }
    const double r = red[0];
    __syncthreads();
    return r;
}

// Exclusive prefix sum over the workgroup of one int per thread.
__device__ int hsa_exclusive_scan(int v, int *sc) {
    const int t = threadIdx.x;
    sc[t] = v;
    __syncthreads();
    for (int d = 1; d < kHsaThreads; d <<= 1) {
        const int add = t >= d ? sc[t - d] : 0;
        __syncthreads();
        sc[t] += add;
        __syncthreads();
    }
    const int r = sc[t] - v;
    __syncthreads();
    return r;
}

// (mass desc, block asc): a before b
__device__ __forceinline__ bool hsa_before(double ma, int ia, double mb, int ib) {
    return ma > mb || (ma == mb && ia < ib);
}

__global__ __launch_bounds__(kHsaThreads) void k_hsa_select(
    const double *__restrict__ ksum, const double *__restrict__ qsum, int nb_ctx, int nb_own,
    int n_ctx, int n_own, int n_q, int q_blocks, int hd, int head_dim, double scale,
    const double *__restrict__ tau, int n_tiles, int32_t *__restrict__ tiles,
    int32_t *__restrict__ count, double *__restrict__ gini_out) {
    __shared__ double qbar[WA_HSA_MAX_HEAD_DIM];
    __shared__ double mass[WA_MAX_HSA_BLOCKS];
    __shared__ int ids[WA_MAX_HSA_BLOCKS];
    __shared__ int ntl[WA_MAX_HSA_BLOCKS];
    __shared__ double red[kHsaThreads];
    __shared__ int sc[kHsaThreads];
    __shared__ int n_sel;
    const int t = threadIdx.x;
    const int item = blockIdx.x;
    const int h = item / q_blocks, qb = item % q_blocks;
    const int nb = nb_ctx + nb_own;
    const int nq_b = min(kHsaQBlock, n_q - qb * kHsaQBlock);
    for (int c = t; c < head_dim; c += kHsaThreads)
        qbar[c] = qsum[(int64_t)qb * hd + (int64_t)h * head_dim + c] / (double)nq_b;
    __syncthreads();

    // block scores: (mean query . mean key) * scale, dimensions in order
    double mx = -INFINITY;
    for (int j = t; j < nb; j += kHsaThreads) {
        const int cnt = j < nb_ctx ? min(kHsaInter, n_ctx - kHsaInter * j)
                                   : min(kHsaIntra, n_own - kHsaIntra * (j - nb_ctx));
        const double *ks = ksum + (int64_t)j * hd + (int64_t)h * head_dim;
        double dot = 0.0;
        for (int c = 0; c < head_dim; ++c) dot += qbar[c] * (ks[c] / (double)cnt);
        mass[j] = dot * scale;
        mx = fmax(mx, dot * scale);
    }
    mx = hsa_tree(mx, red, true);
    double part = 0.0;
    for (int j = t; j < nb; j += kHsaThreads) {
        const double e = exp(mass[j] - mx);
        mass[j] = e;
        part += e;
    }
    const double s = hsa_tree(part, red, false);
    // normalise, and pad to a power of two with entries that sort last
    int nb2 = 1;
    while (nb2 < nb) nb2 <<= 1;
    for (int j = t; j < nb2; j += kHsaThreads) {
        if (j < nb) {
            mass[j] /= s;
            ids[j] = j;
        } else {
            mass[j] = -1.0;
            ids[j] = 0x7fffffff;
        }
    }
    __syncthreads();

    // bitonic sort into (mass desc, block asc); pairs of one pass are disjoint
    for (int k = 2; k <= nb2; k <<= 1)
        for (int jj = k >> 1; jj > 0; jj >>= 1) {
            for (int i = t; i < nb2; i += kHsaThreads) {
                const int l = i ^ jj;
                if (l <= i) continue;
                const bool fwd = (i & k) == 0;   // this run ends up in the target order
                const bool swap = fwd ? hsa_before(mass[l], ids[l], mass[i], ids[i])
                                      : hsa_before(mass[i], ids[i], mass[l], ids[l]);
                if (swap) {
                    const double tm = mass[i];
                    mass[i] = mass[l];
                    mass[l] = tm;
                    const int ti = ids[i];
                    ids[i] = ids[l];
                    ids[l] = ti;
                }
            }
            __syncthreads();
        }

    // Gini coefficient: with the masses in decreasing order p_0 >= p_1 >= ...,
    // sum_i sum_j |p_i - p_j| = 2 sum_k (n - 1 - 2k) p_k
    double gpart = 0.0, ppart = 0.0;
    for (int k = t; k < nb; k += kHsaThreads) {
        gpart += (double)(nb - 1 - 2 * k) * mass[k];
        ppart += mass[k];
    }
    const double gsum = hsa_tree(gpart, red, false);
    const double psum = hsa_tree(ppart, red, false);

    // the shortest prefix whose running sum reaches tau_h: one thread, in
    // sorted order, eight values loaded at a time
    if (t == 0) {
        const double th = tau[h];
        double run = 0.0;
        int m = nb;
        for (int k0 = 0; k0 < nb && m == nb; k0 += 8) {
            double v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = mass[k0 + u < nb ? k0 + u : 0];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (m == nb && k0 + u < nb) {
                    run += v[u];
                    if (run >= th) m = k0 + u + 1;
                }
        }
        n_sel = m;
        if (gini_out) gini_out[item] = gsum / ((double)nb * psum);
    }
    __syncthreads();

    // tiles per block (0 when not selected): a context block holds tiles 2j
    // and 2j+1, or only 2j when the context ends 64 keys into it; an own
    // block holds one tile
    for (int j = t; j < nb; j += kHsaThreads) ntl[j] = 0;
    __syncthreads();
    for (int k = t; k < n_sel; k += kHsaThreads) {
        const int j = ids[k];
        ntl[j] = j < nb_ctx ? (n_ctx - kHsaInter * j >= kHsaInter ? 2 : 1) : 1;
    }
    __syncthreads();
    // thread t owns blocks [t * per, (t + 1) * per): prefix over the owners,
    // then each writes its blocks' tiles at their offsets, in block order
    const int per = (nb + kHsaThreads - 1) / kHsaThreads;
    const int j0 = min(nb, t * per), j1 = min(nb, j0 + per);
    int mine = 0;
    for (int j = j0; j < j1; ++j) mine += ntl[j];
    int at = hsa_exclusive_scan(mine, sc);
    if (t == kHsaThreads - 1) count[item] = at + mine;
    int32_t *list = tiles + (int64_t)item * n_tiles;
    const int t_ctx = n_ctx / 64;
    for (int j = j0; j < j1; ++j) {
        const int c = ntl[j];
        if (c == 0) continue;
        if (j < nb_ctx) {
            list[at] = 2 * j;
            if (c == 2) list[at + 1] = 2 * j + 1;
        } else {
            list[at] = t_ctx + (j - nb_ctx);
        }
        at += c;
    }
}

hipError_t launch_hsa_select(const wa_layout &L, const void *q, int32_t n_q, const void *k_ctx,
                             int32_t n_ctx, const void *k_own, int32_t n_own, double scale,
                             const double *tau, int32_t *tiles, int32_t *count, double *gini,
                             void *ws, hipStream_t s) {
    const int64_t hd = (int64_t)L.n_heads * L.head_dim;
    const HsaShape w = hsa_shape(L.n_heads, n_q, n_ctx, n_own);
    double *ksum = (double *)ws;
    double *qsum = (double *)((char *)ws + hsa_ksum_bytes(hd, w));
    const int vec = 16 / elem_bytes(L.dtype);
    const int chunks = (int)(hd / vec);
    const int group_chunks = chunks < 64 ? chunks : 64;
    const int groups = (chunks + group_chunks - 1) / group_chunks;
    const dim3 grid((unsigned)groups, (unsigned)(w.nb_ctx + w.nb_own + w.q_blocks));
    if (L.dtype == WA_BF16)
        hipLaunchKernelGGL(k_hsa_pool<true>, grid, dim3(kHsaThreads), 0, s, (const uint4 *)k_ctx,
                           n_ctx, (const uint4 *)k_own, n_own, (const uint4 *)q, n_q, w.nb_ctx,
                           w.nb_own, chunks, group_chunks, (int)hd, ksum, qsum);
    else
        hipLaunchKernelGGL(k_hsa_pool<false>, grid, dim3(kHsaThreads), 0, s, (const uint4 *)k_ctx,
                           n_ctx, (const uint4 *)k_own, n_own, (const uint4 *)q, n_q, w.nb_ctx,
                           w.nb_own, chunks, group_chunks, (int)hd, ksum, qsum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_hsa_select, dim3((unsigned)w.items), dim3(kHsaThreads), 0, s, ksum, qsum,
                       w.nb_ctx, w.nb_own, n_ctx, n_own, n_q, w.q_blocks, (int)hd, L.head_dim,
                       scale, tau, w.n_tiles, tiles, count, gini);
    return hipGetLastError();
}

}  // namespace wa
