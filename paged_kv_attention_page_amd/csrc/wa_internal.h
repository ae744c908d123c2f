// Internal declarations shared by the host entry points (wa_api.cpp) and the
// kernel sources.  Not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/wa.h"

namespace wa {

inline int elem_bytes(int32_t dtype) { return dtype == WA_F32 ? 4 : 2; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// column sums (page mean key, chunk mean query)
//
// A column-sum launch is a 2-D grid: blockIdx.x picks a group of up to 64
// 16-byte column vectors, blockIdx.y a range of rows.  Each block writes one
// fp64 partial sum per column of its group for its row range (partial layout
// [row_blocks][hd]); a second kernel adds the partials of a column in a fixed
// order.  `vec` = elements per 16-byte vector, `chunks` = hd / vec vectors per
// row, `group_chunks` = vectors per block, `row_lanes` = rows read at once.
struct ColSumPlan {
    int vec;
    int chunks;
    int group_chunks;
    int groups;
    int row_lanes;
    int threads;
    int rows_per_block;
    int blocks;   // row blocks
};
// Column groups of at most max_group_chunks 16-byte vectors (64 fills a
// 256-thread block with 4 row lanes).
ColSumPlan colsum_plan(int32_t dtype, int64_t hd, int64_t rows, int rows_per_lane,
                       int max_group_chunks = 64);

// ---------------------------------------------------------------------------
// workspace layouts

size_t append_workspace_bytes(int32_t dtype, int64_t hd, int64_t page_tokens);

// Bytes [0, 256) hold the one-launch paths' completion counters (zero between
// calls).  One-launch path: alpha_part is [groups * row blocks][n_cand]; two-level
// path: partial_q is [row blocks][hd] column sums, alpha_part [groups][n_cand].
struct SelectWs {
    bool one_launch;    // few candidates (with a prompt stage: few pages in all the chunks): one kernel
    bool wide;          // up to 256 candidates, no prompt stage: one kernel, two-level hand-off
    size_t partial_q;   // [q_blocks][hd] double
    size_t cosine;      // [n_chunks] double (prompt stage)
    size_t alpha_part;  // [groups][n_cand] double
    size_t cand;        // [n_cand] int32
    size_t total;
    ColSumPlan q_plan;
    int groups;
};
SelectWs select_workspace(int32_t dtype, int64_t hd, int32_t n_q, int32_t n_cand,
                          int32_t n_chunks, int32_t pages_per_chunk);
// Device address of this device's fixed selection workspace (the `scratch`
// array of k_select.hip, WA_SELECT_NOALLOC_MAX_WORKSPACE bytes), looked up
// once per device; allocates nothing.
hipError_t select_scratch(void **out);

// ---------------------------------------------------------------------------
// launchers (return hipSuccess or the launch error)

hipError_t launch_append(const wa_layout &L, const void *k_src, const void *v_src, void *k_pool,
                         void *v_pool, int32_t slot, double *page_means, void *ws,
                         hipStream_t s);

// recent / n_recent: the sliding window (range access); its ids come first in
// out_idx and are excluded from the ranked (selective) part, which fills
// out_idx[n_recent .. n_recent + k_p).  n_recent = 0: the plain page stage.
hipError_t launch_select(const wa_layout &L, const void *q, int32_t n_q, const double *page_means,
                         const int32_t *cand, int32_t n_cand, const wa_prompt_stage *prompt,
                         const int32_t *recent, int32_t n_recent, int32_t k_p, int32_t *out_idx,
                         double *out_scores, void *ws, hipStream_t s);

hipError_t launch_gather(const wa_layout &L, const void *k_pool, const void *v_pool,
                         const int32_t *idx, int32_t k_p, void *k_ctx, void *v_ctx,
                         hipStream_t s);

// Where the context keys come from: idx == nullptr means k_ctx / v_ctx are
// contiguous [n_ctx][H][d] buffers; otherwise they are the pools
// [max_pages][page_tokens][H][d] and context key n is token n % page_tokens
// of page idx[n / page_tokens] (n_ctx = k_p * page_tokens).
struct PagedCtx {
    const int32_t *idx = nullptr;   // device [k_p]
    int32_t page_tokens = 0;
    int32_t max_pages = 0;
};

hipError_t launch_attention_f32(int32_t n_heads, int32_t head_dim, const float *q, int32_t n_q,
                                const float *k_ctx, const float *v_ctx, int32_t n_ctx,
                                const float *k_own, const float *v_own, int32_t n_own,
                                float scale, float *out, float *lse, const PagedCtx &pg,
                                hipStream_t s);

// bf16 attention launch plan: one block per (query block, head) item, or
// (split) one block per CU, each taking an equal run of the items' key tiles,
// followed by a merge of the items shared by several blocks.
struct AttnPlan {
    int split;
    int grid;
    int items;
    int n_tiles;
    int head_tiles;     // split: first-phase tiles per item
    int slots;          // split: partial slots per item
    int64_t total;
    size_t workspace;   // bytes of partial results (0 unless split)
};
AttnPlan attention_plan(int32_t n_heads, int32_t n_q, int32_t n_keys, int cu_count);

// Sparse branch: per (query block, head) item, the ascending 64-key tiles of
// [ctx ++ own] to attend over (tiles[item][0 .. count[item])).  tiles == null:
// every tile (dense attention).
// The launch plans on the device (whether to split the lists over all CUs);
// workspace: sparse_workspace_bytes(items, cu_count) bytes.
struct SparseCtx {
    const int32_t *tiles = nullptr;   // device [items][n_tiles]
    const int32_t *count = nullptr;   // device [items]
    int cu_count = 0;
};
size_t sparse_workspace_bytes(int items, int cu_count);

hipError_t launch_attention_bf16(int32_t n_heads, const uint16_t *q, int32_t n_q,
                                 const uint16_t *k_ctx, const uint16_t *v_ctx, int32_t n_ctx,
                                 const uint16_t *k_own, const uint16_t *v_own, int32_t n_own,
                                 float scale, int32_t out_dtype, void *out, float *lse,
                                 const AttnPlan &plan, void *workspace, const PagedCtx &pg,
                                 hipStream_t s, const SparseCtx &sp = SparseCtx{});

// merge of two attentions over disjoint key sets (fp32 outputs and lse)
hipError_t launch_merge_attention(int32_t n_heads, int32_t head_dim, int32_t n_q,
                                  const float *out_a, const float *lse_a, const float *out_b,
                                  const float *lse_b, int32_t out_dtype, void *out, float *lse,
                                  hipStream_t s);

// ---------------------------------------------------------------------------
// sparse branch block selection

struct HsaShape {
    int32_t nb_ctx;     // context key blocks
    int32_t nb_own;     // own key blocks
    int32_t q_blocks;   // pooled query blocks
    int32_t items;      // q_blocks * n_heads, item = head * q_blocks + query block
    int32_t n_tiles;    // 64-key tiles of [ctx ++ own] (row stride of the tile lists)
};
HsaShape hsa_shape(int32_t n_heads, int32_t n_q, int32_t n_ctx, int32_t n_own);
// key block sums [nb_ctx + nb_own][hd], then query block sums [q_blocks][hd] (fp64)
size_t hsa_workspace_bytes(int64_t hd, const HsaShape &w);

hipError_t launch_hsa_select(const wa_layout &L, const void *q, int32_t n_q, const void *k_ctx,
                             int32_t n_ctx, const void *k_own, int32_t n_own, double scale,
                             const double *tau, int32_t *tiles, int32_t *count, double *gini,
                             bool ctx_sums_ready, void *ws, hipStream_t s);

}  // namespace wa
