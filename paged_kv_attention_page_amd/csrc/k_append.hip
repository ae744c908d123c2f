// Append one page to the pool and record its mean key (WorldAttention
// review, "HKV: Page-Level Multi-Tier Memory": each page is summarised by the
// mean of its keys; Inferix summary, section 3.4, Step 4: the cache grows
// after a block's last denoising step).
//
// Pass 1 (k_append_sum): one HBM pass over the page.  Every block copies its
// row range of K (and V) into the pool slot and forms fp64 partial column
// sums of K.  Pass 2 (k_colsum_finish): adds the block partials in a fixed
// order (16 lanes per column) and divides by the row count.  Bound: HBM bandwidth; the algorithmic
// traffic is 2 x (K + V page bytes) plus 8 bytes per mean element written.
#include "colsum.h"
#include "wa_internal.h"

namespace wa {

ColSumPlan colsum_plan(int32_t dtype, int64_t hd, int64_t rows, int rows_per_lane,
                       int max_group_chunks) {
    ColSumPlan p;
    p.vec = 16 / elem_bytes(dtype);
    p.chunks = (int)(hd / p.vec);
    p.group_chunks = p.chunks < max_group_chunks ? p.chunks : max_group_chunks;
    p.groups = (p.chunks + p.group_chunks - 1) / p.group_chunks;
    p.row_lanes = 256 / p.group_chunks;
    p.threads = p.group_chunks * p.row_lanes;
    p.threads = (p.threads + 63) / 64 * 64;
    p.rows_per_block = p.row_lanes * rows_per_lane;
    p.blocks = (int)((rows + p.rows_per_block - 1) / p.rows_per_block);
    if (p.blocks < 1) p.blocks = 1;
    return p;
}

// Groups of 32 sixteen-byte vectors (8 row lanes x 8 rows = 64 rows per
// block): measured 33.2 us per Wan-shaped page against 34.5 us with groups of
// 64 vectors and 32 rows (and 33.7-37.2 us for 8 or 16 vectors per group).
static ColSumPlan append_plan(int32_t dtype, int64_t hd, int64_t page_tokens) {
    return colsum_plan(dtype, hd, page_tokens, 8, 32);
}

size_t append_workspace_bytes(int32_t dtype, int64_t hd, int64_t page_tokens) {
    const ColSumPlan p = append_plan(dtype, hd, page_tokens);
    return (size_t)p.blocks * (size_t)hd * sizeof(double);
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_append_sum(
    const uint4 *__restrict__ k_src, uint4 *__restrict__ k_dst, const uint4 *__restrict__ v_src,
    uint4 *__restrict__ v_dst, int64_t rows, int chunks, int group_chunks, int row_lanes,
    int rows_per_block, double *__restrict__ partial) {
    __shared__ double lds[256 * (BF16 ? 8 : 4)];
    constexpr int VEC = BF16 ? 8 : 4;
    colsum_block<BF16>(k_src, k_dst, v_src, v_dst, rows, chunks, blockIdx.x * group_chunks,
                       group_chunks, row_lanes, rows_per_block, blockIdx.y, lds,
                       partial + (int64_t)blockIdx.y * chunks * VEC);
}

// out[col] = (sum of the block partials of col, fixed order) / rows; one
// block of 1024 threads per 64 columns
__global__ __launch_bounds__(1024) void k_colsum_finish(const double *__restrict__ partial,
                                                        int blocks, int hd, int64_t rows,
                                                        double *__restrict__ out) {
    __shared__ double lds[16 * 64];
    const int c0 = blockIdx.x * 64;
    const double tot = reduce_partials_64(partial, blocks, hd, c0, lds);
    if (threadIdx.x < 64 && c0 + (int)threadIdx.x < hd) out[c0 + threadIdx.x] = tot / (double)rows;
}

hipError_t launch_append(const wa_layout &L, const void *k_src, const void *v_src, void *k_pool,
                         void *v_pool, int32_t slot, double *page_means, void *ws,
                         hipStream_t s) {
    const int64_t hd = (int64_t)L.n_heads * L.head_dim;
    const int64_t page_elems = (int64_t)L.page_tokens * hd;
    const int eb = elem_bytes(L.dtype);
    char *k_slot = (char *)k_pool + (int64_t)slot * page_elems * eb;
    char *v_slot = v_pool ? (char *)v_pool + (int64_t)slot * page_elems * eb : nullptr;
    // a source that already is the slot needs no copy (the mean-only mode)
    uint4 *k_dst = (k_src == k_slot) ? nullptr : (uint4 *)k_slot;
    const uint4 *v_read = (v_src && v_src != v_slot && v_slot) ? (const uint4 *)v_src : nullptr;
    uint4 *v_dst = v_read ? (uint4 *)v_slot : nullptr;

    const ColSumPlan p = append_plan(L.dtype, hd, L.page_tokens);
    double *partial = (double *)ws;
    const dim3 grid((unsigned)p.groups, (unsigned)p.blocks);
    if (L.dtype == WA_BF16)
        hipLaunchKernelGGL(k_append_sum<true>, grid, dim3(p.threads), 0, s, (const uint4 *)k_src,
                           k_dst, v_read, v_dst, (int64_t)L.page_tokens, p.chunks, p.group_chunks,
                           p.row_lanes, p.rows_per_block, partial);
    else
        hipLaunchKernelGGL(k_append_sum<false>, grid, dim3(p.threads), 0, s, (const uint4 *)k_src,
                           k_dst, v_read, v_dst, (int64_t)L.page_tokens, p.chunks, p.group_chunks,
                           p.row_lanes, p.rows_per_block, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_colsum_finish, dim3((unsigned)((hd + 63) / 64)), dim3(1024), 0, s,
                       (const double *)partial, p.blocks, (int)hd, (int64_t)L.page_tokens,
                       page_means + (int64_t)slot * hd);
    return hipGetLastError();
}

}  // namespace wa
