// Host entry points of libwa.so: argument validation, then kernel launches
// on the caller's stream.  Validation runs before any HIP call, so every
// error path can be exercised without a GPU.  Semantics and error rules of
// each entry point are stated in include/wa.h.
#include <math.h>

#include "wa_internal.h"

using namespace wa;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Checks shared by all calls.  need_pool: page_tokens and max_pages matter.
wa_status check_layout(const wa_layout *L, bool need_pool) {
    if (!L) return WA_ERR_INVALID_ARG;
    if (L->n_heads < 1 || L->head_dim < 1) return WA_ERR_INVALID_ARG;
    if (L->dtype != WA_F32 && L->dtype != WA_BF16) return WA_ERR_UNSUPPORTED;
    if (need_pool && (L->page_tokens < 1 || L->max_pages < 1)) return WA_ERR_INVALID_ARG;
    const int64_t hd = (int64_t)L->n_heads * L->head_dim;
    if (hd > WA_MAX_ROW_ELEMS) return WA_ERR_UNSUPPORTED;
    if ((hd * elem_bytes(L->dtype)) % 16 != 0) return WA_ERR_UNSUPPORTED;
    return WA_OK;
}

wa_status from_hip(hipError_t e) { return e == hipSuccess ? WA_OK : WA_ERR_HIP; }

wa_status check_prompt(const wa_layout *L, const wa_prompt_stage *P, const int32_t *cand,
                       int32_t n_cand) {
    if (!P) return WA_OK;
    if (cand) return WA_ERR_INVALID_ARG;
    if (!P->chunk_prompts || !P->cur_prompt || !P->chunk_pages) return WA_ERR_INVALID_ARG;
    if (!aligned16(P->chunk_prompts) || !aligned16(P->cur_prompt) || !aligned16(P->chunk_pages))
        return WA_ERR_INVALID_ARG;
    if (P->n_chunks < 1 || P->emb_dim < 1 || P->pages_per_chunk < 1 || P->n_keep < 1 ||
        P->n_keep > P->n_chunks)
        return WA_ERR_INVALID_ARG;
    if (P->n_chunks > WA_MAX_CANDIDATES) return WA_ERR_UNSUPPORTED;
    if ((int64_t)P->n_keep * P->pages_per_chunk != n_cand) return WA_ERR_INVALID_ARG;
    (void)L;
    return WA_OK;
}

}  // namespace

extern "C" {

size_t wa_append_workspace_bytes(const wa_layout *L) {
    if (check_layout(L, true) != WA_OK) return 0;
    return append_workspace_bytes(L->dtype, (int64_t)L->n_heads * L->head_dim, L->page_tokens);
}

wa_status wa_append_page(const wa_layout *L, const void *k_src, const void *v_src, void *k_pool,
                         void *v_pool, int32_t slot, double *page_means, void *workspace,
                         size_t workspace_bytes, void *stream) {
    wa_status st = check_layout(L, true);
    if (st != WA_OK) return st;
    if (!k_src || !k_pool || !page_means || !workspace) return WA_ERR_INVALID_ARG;
    if (v_src && !v_pool) return WA_ERR_INVALID_ARG;
    if (slot < 0 || slot >= L->max_pages) return WA_ERR_INVALID_ARG;
    if (!aligned16(k_src) || !aligned16(k_pool) || !aligned16(page_means) || !aligned16(workspace) ||
        (v_src && !aligned16(v_src)) || (v_pool && !aligned16(v_pool)))
        return WA_ERR_INVALID_ARG;
    if (workspace_bytes < wa_append_workspace_bytes(L)) return WA_ERR_INVALID_ARG;
    return from_hip(launch_append(*L, k_src, v_src, k_pool, v_pool, slot, page_means, workspace,
                                  (hipStream_t)stream));
}

size_t wa_select_workspace_bytes(const wa_layout *L, int32_t n_q, int32_t n_cand,
                                 const wa_prompt_stage *prompt) {
    if (check_layout(L, true) != WA_OK || n_q < 1 || n_cand < 1) return 0;
    if (n_cand > WA_MAX_CANDIDATES) return 0;
    const int32_t n_chunks = prompt ? prompt->n_chunks : 0;
    if (n_chunks < 0 || n_chunks > WA_MAX_CANDIDATES) return 0;
    if (prompt && (n_chunks < 1 || prompt->pages_per_chunk < 1 || prompt->n_keep < 1 ||
                   prompt->n_keep > n_chunks ||
                   (int64_t)prompt->n_keep * prompt->pages_per_chunk != n_cand))
        return 0;
    return select_workspace(L->dtype, (int64_t)L->n_heads * L->head_dim, n_q, n_cand, n_chunks,
                            prompt ? prompt->pages_per_chunk : 0)
        .total;
}

namespace {

// Argument checks of a selection, everything but the workspace.
wa_status select_check(const wa_layout *L, const void *q, int32_t n_q, const double *page_means,
                       const int32_t *cand, int32_t n_cand, const wa_prompt_stage *prompt,
                       const int32_t *recent, int32_t n_recent, int32_t k_p, int32_t *out_idx,
                       double *out_scores) {
    wa_status st = check_layout(L, true);
    if (st != WA_OK) return st;
    if (!q || !page_means || !out_idx) return WA_ERR_INVALID_ARG;
    if (n_q < 1 || n_cand < 1 || k_p < 0 || k_p > n_cand) return WA_ERR_INVALID_ARG;
    if (n_recent < 0 || n_recent + k_p < 1 || (n_recent > 0 && !recent)) return WA_ERR_INVALID_ARG;
    if (n_cand > WA_MAX_CANDIDATES || n_recent > WA_MAX_WINDOW) return WA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(page_means) || !aligned16(out_idx) ||
        (cand && !aligned16(cand)) || (out_scores && !aligned16(out_scores)) ||
        ((uintptr_t)recent & 3u))
        return WA_ERR_INVALID_ARG;
    return check_prompt(L, prompt, cand, n_cand);
}

// Shared by wa_select_pages (no window) and wa_select_window.
wa_status select_impl(const wa_layout *L, const void *q, int32_t n_q, const double *page_means,
                      const int32_t *cand, int32_t n_cand, const wa_prompt_stage *prompt,
                      const int32_t *recent, int32_t n_recent, int32_t k_p, int32_t *out_idx,
                      double *out_scores, void *workspace, size_t workspace_bytes,
                      void *stream) {
    wa_status st = check_layout(L, true);
    if (st != WA_OK) return st;
    if (!q || !page_means || !out_idx || !workspace) return WA_ERR_INVALID_ARG;
    if (n_q < 1 || n_cand < 1 || k_p < 0 || k_p > n_cand) return WA_ERR_INVALID_ARG;
    if (n_recent < 0 || n_recent + k_p < 1 || (n_recent > 0 && !recent)) return WA_ERR_INVALID_ARG;
    if (n_cand > WA_MAX_CANDIDATES || n_recent > WA_MAX_WINDOW) return WA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(page_means) || !aligned16(out_idx) || !aligned16(workspace) ||
        (cand && !aligned16(cand)) || (out_scores && !aligned16(out_scores)) ||
        ((uintptr_t)recent & 3u))
        return WA_ERR_INVALID_ARG;
    st = check_prompt(L, prompt, cand, n_cand);
    if (st != WA_OK) return st;
    if (workspace_bytes < wa_select_workspace_bytes(L, n_q, n_cand, prompt))
        return WA_ERR_INVALID_ARG;
    return from_hip(launch_select(*L, q, n_q, page_means, cand, n_cand, prompt, recent, n_recent,
                                  k_p, out_idx, out_scores, workspace, (hipStream_t)stream));
}

}  // namespace

wa_status wa_select_pages(const wa_layout *L, const void *q, int32_t n_q, const double *page_means,
                          const int32_t *cand, int32_t n_cand, const wa_prompt_stage *prompt,
                          int32_t k_p, int32_t *out_idx, double *out_scores, void *workspace,
                          size_t workspace_bytes, void *stream) {
    if (k_p < 1) return WA_ERR_INVALID_ARG;
    return select_impl(L, q, n_q, page_means, cand, n_cand, prompt, nullptr, 0, k_p, out_idx,
                       out_scores, workspace, workspace_bytes, stream);
}

wa_status wa_select_pages_noalloc(const wa_layout *L, const void *q, int32_t n_q,
                                  const double *page_means, const int32_t *cand, int32_t n_cand,
                                  const wa_prompt_stage *prompt, int32_t k_p, int32_t *out_idx,
                                  double *out_scores, void *stream) {
    if (k_p < 1) return WA_ERR_INVALID_ARG;
    wa_status st = select_check(L, q, n_q, page_means, cand, n_cand, prompt, nullptr, 0, k_p,
                                out_idx, out_scores);
    if (st != WA_OK) return st;
    const size_t need = wa_select_workspace_bytes(L, n_q, n_cand, prompt);
    if (need == 0) return WA_ERR_INVALID_ARG;
    if (need > WA_SELECT_NOALLOC_MAX_WORKSPACE) return WA_ERR_UNSUPPORTED;
    void *ws = nullptr;
    if (select_scratch(&ws) != hipSuccess) return WA_ERR_HIP;
    return select_impl(L, q, n_q, page_means, cand, n_cand, prompt, nullptr, 0, k_p, out_idx,
                       out_scores, ws, need, stream);
}

wa_status wa_select_window(const wa_layout *L, const void *q, int32_t n_q,
                           const double *page_means, const int32_t *cand, int32_t n_cand,
                           const wa_prompt_stage *prompt, const int32_t *recent,
                           int32_t n_recent, int32_t k_p, int32_t *out_idx, double *out_scores,
                           void *workspace, size_t workspace_bytes, void *stream) {
    return select_impl(L, q, n_q, page_means, cand, n_cand, prompt, recent, n_recent, k_p,
                       out_idx, out_scores, workspace, workspace_bytes, stream);
}

wa_status wa_gather(const wa_layout *L, const void *k_pool, const void *v_pool, const int32_t *idx,
                    int32_t k_p, void *k_ctx, void *v_ctx, void *stream) {
    wa_status st = check_layout(L, true);
    if (st != WA_OK) return st;
    if (!k_pool || !idx || !k_ctx) return WA_ERR_INVALID_ARG;
    if ((v_pool == nullptr) != (v_ctx == nullptr)) return WA_ERR_INVALID_ARG;
    if (k_p < 1) return WA_ERR_INVALID_ARG;
    if (k_p > 65535) return WA_ERR_UNSUPPORTED;
    if (!aligned16(k_pool) || !aligned16(k_ctx) || (v_pool && !aligned16(v_pool)) ||
        (v_ctx && !aligned16(v_ctx)) || ((uintptr_t)idx & 3u))
        return WA_ERR_INVALID_ARG;
    return from_hip(launch_gather(*L, k_pool, v_pool, idx, k_p, k_ctx, v_ctx, (hipStream_t)stream));
}

// CUs of the current device; 256 (MI355X) when no device can be queried, so
// that the workspace size can be asked for without a GPU.
static int current_cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        return 256;
    return n;
}

size_t wa_attention_workspace_bytes(const wa_layout *L, int32_t n_q, int32_t n_ctx,
                                    int32_t n_own) {
    if (check_layout(L, false) != WA_OK || L->dtype != WA_BF16) return 0;
    if (n_q < 1 || n_ctx < 0 || n_own < 0 || (int64_t)n_ctx + n_own < 1) return 0;
    if ((int64_t)n_ctx + n_own > 0x7fffffff - 256) return 0;
    return attention_plan(L->n_heads, n_q, n_ctx + n_own, current_cu_count()).workspace;
}

namespace {

// Shared by wa_block_attention and wa_paged_attention: the layout is already
// checked, and pg says where the n_ctx context keys come from.
wa_status attention(const wa_layout *L, const void *q, int32_t n_q, const void *k_ctx,
                    const void *v_ctx, int32_t n_ctx, const void *k_own, const void *v_own,
                    int32_t n_own, float softmax_scale, int32_t out_dtype, void *out, float *lse,
                    void *workspace, size_t ws_bytes, const PagedCtx &pg, void *stream,
                    const SparseCtx &sp = SparseCtx{}) {
    if (!q || !out) return WA_ERR_INVALID_ARG;
    if (n_q < 1 || n_ctx < 0 || n_own < 0 || (int64_t)n_ctx + n_own < 1) return WA_ERR_INVALID_ARG;
    if ((int64_t)n_ctx + n_own > 0x7fffffff - 256) return WA_ERR_UNSUPPORTED;
    if (n_ctx > 0 && (!k_ctx || !v_ctx)) return WA_ERR_INVALID_ARG;
    if (n_own > 0 && (!k_own || !v_own)) return WA_ERR_INVALID_ARG;
    if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return WA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out) || (n_ctx > 0 && (!aligned16(k_ctx) || !aligned16(v_ctx))) ||
        (n_own > 0 && (!aligned16(k_own) || !aligned16(v_own))) || ((uintptr_t)lse & 3u))
        return WA_ERR_INVALID_ARG;
    if (sp.tiles) {   // sparse branch: bf16 only, tile lists bounded
        if (L->dtype != WA_BF16) return WA_ERR_UNSUPPORTED;
        const int64_t n_tiles = ((int64_t)n_ctx + n_own + 63) / 64;
        if (n_tiles > WA_MAX_SPARSE_TILES) return WA_ERR_UNSUPPORTED;
        if ((int64_t)(n_q + 255) / 256 * L->n_heads * n_tiles > 0x7fffffff) return WA_ERR_UNSUPPORTED;
    }
    if (L->dtype == WA_F32) {
        if (L->head_dim != 64 && L->head_dim != 128) return WA_ERR_UNSUPPORTED;
        if (out_dtype != WA_F32) return WA_ERR_UNSUPPORTED;
        return from_hip(launch_attention_f32(L->n_heads, L->head_dim, (const float *)q, n_q,
                                             (const float *)k_ctx, (const float *)v_ctx, n_ctx,
                                             (const float *)k_own, (const float *)v_own, n_own,
                                             softmax_scale, (float *)out, lse, pg,
                                             (hipStream_t)stream));
    }
    if (L->head_dim != 128) return WA_ERR_UNSUPPORTED;
    if (out_dtype != WA_F32 && out_dtype != WA_BF16) return WA_ERR_UNSUPPORTED;
    const AttnPlan plan = attention_plan(L->n_heads, n_q, n_ctx + n_own, current_cu_count());
    if (sp.tiles) {
        if (!workspace || !aligned16(workspace) ||
            ws_bytes < sparse_workspace_bytes(plan.items, sp.cu_count))
            return WA_ERR_INVALID_ARG;
    } else if (plan.workspace > 0 && (!workspace || ws_bytes < plan.workspace || !aligned16(workspace)))
        return WA_ERR_INVALID_ARG;
    return from_hip(launch_attention_bf16(L->n_heads, (const uint16_t *)q, n_q,
                                          (const uint16_t *)k_ctx, (const uint16_t *)v_ctx, n_ctx,
                                          (const uint16_t *)k_own, (const uint16_t *)v_own, n_own,
                                          softmax_scale, out_dtype, out, lse, plan, workspace, pg,
                                          (hipStream_t)stream, sp));
}

}  // namespace

wa_status wa_block_attention(const wa_layout *L, const void *q, int32_t n_q, const void *k_ctx,
                             const void *v_ctx, int32_t n_ctx, const void *k_own,
                             const void *v_own, int32_t n_own, float softmax_scale,
                             int32_t out_dtype, void *out, float *lse, void *workspace,
                             size_t ws_bytes, void *stream) {
    const wa_status st = check_layout(L, false);
    if (st != WA_OK) return st;
    return attention(L, q, n_q, k_ctx, v_ctx, n_ctx, k_own, v_own, n_own, softmax_scale,
                     out_dtype, out, lse, workspace, ws_bytes, PagedCtx{}, stream);
}

wa_status wa_paged_attention(const wa_layout *L, const void *q, int32_t n_q, const void *k_pool,
                             const void *v_pool, const int32_t *idx, int32_t k_p,
                             const void *k_own, const void *v_own, int32_t n_own,
                             float softmax_scale, int32_t out_dtype, void *out, float *lse,
                             void *workspace, size_t ws_bytes, void *stream) {
    const wa_status st = check_layout(L, true);
    if (st != WA_OK) return st;
    if (!k_pool || !v_pool || !idx) return WA_ERR_INVALID_ARG;
    if (k_p < 1) return WA_ERR_INVALID_ARG;
    if ((int64_t)k_p * L->page_tokens > 0x7fffffff - 256) return WA_ERR_UNSUPPORTED;
    if ((uintptr_t)idx & 3u) return WA_ERR_INVALID_ARG;
    PagedCtx pg;
    pg.idx = idx;
    pg.page_tokens = L->page_tokens;
    pg.max_pages = L->max_pages;
    return attention(L, q, n_q, k_pool, v_pool, k_p * L->page_tokens, k_own, v_own, n_own,
                     softmax_scale, out_dtype, out, lse, workspace, ws_bytes, pg, stream);
}

size_t wa_hsa_workspace_bytes(const wa_layout *L, int32_t n_q, int32_t n_ctx, int32_t n_own) {
    if (check_layout(L, false) != WA_OK) return 0;
    if (n_q < 1 || n_ctx < 0 || n_own < 0 || (int64_t)n_ctx + n_own < 1) return 0;
    if (n_ctx % 64 != 0 || L->head_dim > WA_HSA_MAX_HEAD_DIM) return 0;
    const HsaShape w = hsa_shape(L->n_heads, n_q, n_ctx, n_own);
    if (w.nb_ctx + w.nb_own > WA_MAX_HSA_BLOCKS) return 0;
    if ((int64_t)w.nb_ctx + w.nb_own + w.q_blocks > 65535) return 0;
    return hsa_workspace_bytes((int64_t)L->n_heads * L->head_dim, w);
}

wa_status wa_hsa_select(const wa_layout *L, const void *q, int32_t n_q, const void *k_ctx,
                        int32_t n_ctx, const void *k_own, int32_t n_own, double scale,
                        const double *tau, int32_t *sel_tiles, int32_t *sel_count, double *gini,
                        int32_t ctx_sums_ready, void *workspace, size_t ws_bytes, void *stream) {
    const wa_status st = check_layout(L, false);
    if (st != WA_OK) return st;
    if (!q || !tau || !sel_tiles || !sel_count || !workspace) return WA_ERR_INVALID_ARG;
    if (n_q < 1 || n_ctx < 0 || n_own < 0 || (int64_t)n_ctx + n_own < 1) return WA_ERR_INVALID_ARG;
    if ((n_ctx > 0 && !k_ctx) || (n_own > 0 && !k_own)) return WA_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.0)) return WA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(workspace) || (n_ctx > 0 && !aligned16(k_ctx)) ||
        (n_own > 0 && !aligned16(k_own)) || ((uintptr_t)tau & 7u) || ((uintptr_t)gini & 7u) ||
        ((uintptr_t)sel_tiles & 3u) || ((uintptr_t)sel_count & 3u))
        return WA_ERR_INVALID_ARG;
    if (n_ctx % 64 != 0 || L->head_dim > WA_HSA_MAX_HEAD_DIM) return WA_ERR_UNSUPPORTED;
    const HsaShape w = hsa_shape(L->n_heads, n_q, n_ctx, n_own);
    if (w.nb_ctx + w.nb_own > WA_MAX_HSA_BLOCKS) return WA_ERR_UNSUPPORTED;
    if ((int64_t)w.nb_ctx + w.nb_own + w.q_blocks > 65535) return WA_ERR_UNSUPPORTED;
    if (ws_bytes < hsa_workspace_bytes((int64_t)L->n_heads * L->head_dim, w))
        return WA_ERR_INVALID_ARG;
    return from_hip(launch_hsa_select(*L, q, n_q, k_ctx, n_ctx, k_own, n_own, scale, tau,
                                      sel_tiles, sel_count, gini, ctx_sums_ready != 0 && n_ctx > 0,
                                      workspace, (hipStream_t)stream));
}

size_t wa_sparse_workspace_bytes(const wa_layout *L, int32_t n_q, int32_t n_ctx,
                                 int32_t n_own) {
    if (check_layout(L, false) != WA_OK || L->dtype != WA_BF16) return 0;
    if (n_q < 1 || n_ctx < 0 || n_own < 0 || (int64_t)n_ctx + n_own < 1) return 0;
    const int64_t n_tiles = ((int64_t)n_ctx + n_own + 63) / 64;
    if (n_tiles > WA_MAX_SPARSE_TILES) return 0;
    const int64_t items = (int64_t)(n_q + 255) / 256 * L->n_heads;
    if (items * n_tiles > 0x7fffffff) return 0;
    return sparse_workspace_bytes((int)items, current_cu_count());
}

wa_status wa_sparse_attention(const wa_layout *L, const void *q, int32_t n_q, const void *k_ctx,
                              const void *v_ctx, int32_t n_ctx, const void *k_own,
                              const void *v_own, int32_t n_own, float softmax_scale,
                              const int32_t *sel_tiles, const int32_t *sel_count,
                              int32_t out_dtype, void *out, float *lse, void *workspace,
                              size_t ws_bytes, void *stream) {
    const wa_status st = check_layout(L, false);
    if (st != WA_OK) return st;
    if (!sel_tiles || !sel_count) return WA_ERR_INVALID_ARG;
    if (((uintptr_t)sel_tiles & 3u) || ((uintptr_t)sel_count & 3u)) return WA_ERR_INVALID_ARG;
    SparseCtx sp;
    sp.tiles = sel_tiles;
    sp.count = sel_count;
    sp.cu_count = current_cu_count();
    return attention(L, q, n_q, k_ctx, v_ctx, n_ctx, k_own, v_own, n_own, softmax_scale,
                     out_dtype, out, lse, workspace, ws_bytes, PagedCtx{}, stream, sp);
}

wa_status wa_merge_attention(const wa_layout *L, int32_t n_q, const float *out_a,
                             const float *lse_a, const float *out_b, const float *lse_b,
                             int32_t out_dtype, void *out, float *lse, void *stream) {
    const wa_status st = check_layout(L, false);
    if (st != WA_OK) return st;
    if (!out_a || !lse_a || !out_b || !lse_b || !out) return WA_ERR_INVALID_ARG;
    if (n_q < 1) return WA_ERR_INVALID_ARG;
    if (!aligned16(out_a) || !aligned16(out_b) || !aligned16(out) || ((uintptr_t)lse_a & 3u) ||
        ((uintptr_t)lse_b & 3u) || ((uintptr_t)lse & 3u))
        return WA_ERR_INVALID_ARG;
    if (out_dtype != WA_F32 && out_dtype != WA_BF16) return WA_ERR_UNSUPPORTED;
    if (L->head_dim % 4 != 0) return WA_ERR_UNSUPPORTED;
    return from_hip(launch_merge_attention(L->n_heads, L->head_dim, n_q, out_a, lse_a, out_b,
                                           lse_b, out_dtype, out, lse, (hipStream_t)stream));
}

namespace {

// Token rows [row0, row0 + n_rows) of one page of K (and V) (the whole page:
// 0, page_tokens) between a pinned host pool and an HBM pool slot, on the
// caller's stream (the copy engines move it; no kernel runs).
wa_status page_copy(const wa_layout *L, bool to_device, const void *host_k, const void *host_v,
                    int32_t host_pages, int32_t host_slot, const void *k_pool, const void *v_pool,
                    int32_t slot, int32_t row0, int32_t n_rows, void *stream) {
    const wa_status st = check_layout(L, true);
    if (st != WA_OK) return st;
    if (!host_k || !k_pool) return WA_ERR_INVALID_ARG;
    if ((host_v == nullptr) != (v_pool == nullptr)) return WA_ERR_INVALID_ARG;
    if (host_pages < 1 || host_slot < 0 || host_slot >= host_pages) return WA_ERR_INVALID_ARG;
    if (slot < 0 || slot >= L->max_pages) return WA_ERR_INVALID_ARG;
    if (row0 < 0 || n_rows < 1 || (int64_t)row0 + n_rows > L->page_tokens) return WA_ERR_INVALID_ARG;
    if (!aligned16(host_k) || !aligned16(k_pool) || (host_v && !aligned16(host_v)) ||
        (v_pool && !aligned16(v_pool)))
        return WA_ERR_INVALID_ARG;
    // the host pool must be pinned host memory (hipHostMalloc): pageable
    // memory would turn the asynchronous copy into a staged, blocking one
    for (const void *h : {host_k, host_v}) {
        if (!h) continue;
        hipPointerAttribute_t attr;
        if (hipPointerGetAttributes(&attr, h) != hipSuccess) {
            (void)hipGetLastError();
            return WA_ERR_INVALID_ARG;
        }
        if (attr.type != hipMemoryTypeHost) return WA_ERR_INVALID_ARG;
    }
    const size_t row_bytes = (size_t)L->n_heads * L->head_dim * elem_bytes(L->dtype);
    const size_t page_bytes = (size_t)L->page_tokens * row_bytes;
    const size_t first = (size_t)row0 * row_bytes, bytes = (size_t)n_rows * row_bytes;
    const hipMemcpyKind kind = to_device ? hipMemcpyHostToDevice : hipMemcpyDeviceToHost;
    const char *hk = (const char *)host_k + (size_t)host_slot * page_bytes + first;
    const char *dk = (const char *)k_pool + (size_t)slot * page_bytes + first;
    hipError_t e = to_device ? hipMemcpyAsync((void *)dk, hk, bytes, kind, (hipStream_t)stream)
                             : hipMemcpyAsync((void *)hk, dk, bytes, kind, (hipStream_t)stream);
    if (e != hipSuccess || !host_v) return from_hip(e);
    const char *hv = (const char *)host_v + (size_t)host_slot * page_bytes + first;
    const char *dv = (const char *)v_pool + (size_t)slot * page_bytes + first;
    e = to_device ? hipMemcpyAsync((void *)dv, hv, bytes, kind, (hipStream_t)stream)
                  : hipMemcpyAsync((void *)hv, dv, bytes, kind, (hipStream_t)stream);
    return from_hip(e);
}

}  // namespace

wa_status wa_page_in(const wa_layout *L, const void *host_k, const void *host_v,
                     int32_t host_pages, int32_t host_slot, void *k_pool, void *v_pool,
                     int32_t slot, void *stream) {
    return page_copy(L, true, host_k, host_v, host_pages, host_slot, k_pool, v_pool, slot, 0,
                     L ? L->page_tokens : 0, stream);
}

wa_status wa_page_in_rows(const wa_layout *L, const void *host_k, const void *host_v,
                          int32_t host_pages, int32_t host_slot, void *k_pool, void *v_pool,
                          int32_t slot, int32_t row0, int32_t n_rows, void *stream) {
    return page_copy(L, true, host_k, host_v, host_pages, host_slot, k_pool, v_pool, slot, row0,
                     n_rows, stream);
}

wa_status wa_page_out(const wa_layout *L, const void *k_pool, const void *v_pool, int32_t slot,
                      void *host_k, void *host_v, int32_t host_pages, int32_t host_slot,
                      void *stream) {
    return page_copy(L, false, host_k, host_v, host_pages, host_slot, k_pool, v_pool, slot, 0,
                     L ? L->page_tokens : 0, stream);
}

const char *wa_status_string(wa_status s) {
    switch (s) {
        case WA_OK: return "ok";
        case WA_ERR_INVALID_ARG: return "invalid argument";
        case WA_ERR_UNSUPPORTED: return "unsupported layout or argument";
        case WA_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

}  // extern "C"
