/*
 * wa.h -- C ABI of the paged-KV retrieval attention library (libwa.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The library runs the attention step of block-diffusion video generation
 * over a paged KV cache, in four calls:
 *
 *   wa_append_page     copy one page of K/V into the pool and record its
 *                      mean key;
 *   wa_select_pages    score the chunk's mean query against the page mean
 *                      keys and keep the top-K_p pages (optionally after a
 *                      prompt stage that picks the candidate chunks);
 *   wa_select_window   the most recent pages plus the top-K_p of the rest;
 *   wa_gather          copy the kept pages into one contiguous K/V buffer;
 *   wa_block_attention unmasked softmax attention of the chunk's queries over
 *                      the gathered pages followed by the chunk's own K/V;
 *   wa_paged_attention the same attention reading the kept pages in place
 *                      from the pool (no gathered copy);
 *   wa_hsa_select      the sparse branch's block selection: per head and
 *                      query block, the fewest key blocks that hold a given
 *                      share of a pooled attention map;
 *   wa_sparse_attention attention over those blocks only;
 *   wa_page_in/out     move a page between a pinned host tier and HBM;
 *   wa_page_in_rows    page-in of a range of a page's token rows;
 *   wa_merge_attention combine attentions over two disjoint key sets.
 *
 * Sources (page title, section):
 *   WorldAttention review, "WorldAttention: An Efficient Attention
 *   Architecture for Interactive Video World Models" (jaehun.me):
 *     - "HKV: Page-Level Multi-Tier Memory": a page is 8 latent frames of
 *       1,560 tokens; the prompt stage ranks past chunks by cosine
 *       similarity of prompt embeddings; the page stage ranks pages by
 *       alpha = mean(Q)^T mean(K_page) / sqrt(d_k) and keeps K_p = 4;
 *     - "Core Idea", item 3: retrieved pages are reorganised into one
 *       contiguous buffer.
 *   Inferix summary, "Inferix: A Block-Diffusion based Next-Generation
 *   Inference Engine for World Simulation", section 3.4, "The
 *   Block-Diffusion Generation Pipeline", Step 3: a block's queries attend
 *   over [cached K ++ own K] and [cached V ++ own V] with one softmax and no
 *   mask inside the block; Step 4: the cache grows only after the block's
 *   last denoising step.
 *
 * Conventions shared by every call
 *   - Memory: every array argument is DEVICE memory owned by the caller,
 *     except the wa_layout / wa_prompt_stage structs themselves, which are
 *     host memory read during the call only.  The library allocates and frees
 *     nothing and keeps no global state, with one exception: the fixed
 *     per-device workspace of wa_select_pages_noalloc (see there).  Calls
 *     are reentrant, except that wa_select_pages_noalloc calls overlapping
 *     on one GPU share that workspace.
 *   - Layout: token-major and dense.  A K, V, Q or output array of T tokens
 *     is [T][n_heads][head_dim]; the pool is [max_pages][page_tokens][n_heads]
 *     [head_dim]; page_means is [max_pages][n_heads][head_dim] double.
 *   - Element type: layout.dtype (WA_F32 = float, WA_BF16 = bfloat16) for
 *     pages, queries and own K/V.  Means, scores and the selection are fp64.
 *   - Alignment: every device pointer is 16-byte aligned, and one token row
 *     (n_heads * head_dim elements) is a multiple of 16 bytes.
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream).  Every
 *     call only enqueues work on it and returns; no call synchronises the
 *     host, and page indices never travel to the host.  Buffers must stay
 *     valid until the stream has finished the work.
 *   - Errors: argument errors are found on the host before anything is
 *     enqueued and return WA_ERR_INVALID_ARG or WA_ERR_UNSUPPORTED; a failed
 *     launch returns WA_ERR_HIP.  Nothing aborts or throws.  Device data
 *     (candidate ids, page indices) are checked on the device: an id outside
 *     [0, max_pages) is never dereferenced (see each call).
 */
#ifndef WA_H
#define WA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t wa_status;
#define WA_OK 0
#define WA_ERR_INVALID_ARG (-1)
#define WA_ERR_UNSUPPORTED (-2)
#define WA_ERR_HIP (-3)

/* element types */
#define WA_F32 0
#define WA_BF16 1

/* Largest n_heads * head_dim the kernels accept (WA_ERR_UNSUPPORTED above). */
#define WA_MAX_ROW_ELEMS 4096
/* Largest candidate count of one selection (WA_ERR_UNSUPPORTED above). */
#define WA_MAX_CANDIDATES 4096
/* Most pages a sliding window (wa_select_window) may hold. */
#define WA_MAX_WINDOW 64
/* Sparse branch (wa_hsa_select, wa_sparse_attention): keys per context
 * block, keys per own block, queries per pooled query block, and limits. */
#define WA_HSA_CTX_BLOCK 128
#define WA_HSA_OWN_BLOCK 64
#define WA_HSA_Q_BLOCK 256
#define WA_MAX_HSA_BLOCKS 2048   /* key blocks of one selection */
#define WA_HSA_MAX_HEAD_DIM 128  /* head_dim of a selection (64 and 128 tested, bf16 and fp32) */
#define WA_MAX_SPARSE_TILES 4096 /* 64-key tiles of one sparse attention */

typedef struct wa_layout {
    int32_t n_heads;     /* H >= 1 */
    int32_t head_dim;    /* d >= 1 (attention: 64 or 128 for WA_F32, 128 for WA_BF16) */
    int32_t page_tokens; /* P_t >= 1 tokens per page (8 frames x 1,560 = 12,480 in the pages) */
    int32_t max_pages;   /* pool slots >= 1 */
    int32_t dtype;       /* WA_F32 or WA_BF16 */
} wa_layout;

/*
 * Prompt stage (WorldAttention review, "HKV: Page-Level Multi-Tier Memory",
 * stage 1, with several kept chunks as in the Tab. 8 ablation): rank the
 * past chunks by cos(cur_prompt, chunk_prompts[m]) descending, ties to the
 * lower chunk id; keep the first n_keep; the candidate pages are their pages,
 * chunk by chunk in rank order, page by page in chunk_pages order.
 */
typedef struct wa_prompt_stage {
    const float *chunk_prompts;  /* device [n_chunks][emb_dim] */
    const float *cur_prompt;     /* device [emb_dim] */
    const int32_t *chunk_pages;  /* device [n_chunks][pages_per_chunk] pool slots */
    int32_t n_chunks;            /* 1 ... WA_MAX_CANDIDATES */
    int32_t emb_dim;             /* >= 1 */
    int32_t pages_per_chunk;     /* >= 1 */
    int32_t n_keep;              /* 1 ... n_chunks */
    int32_t *out_chunks;         /* device [n_keep] kept chunk ids in rank order, or NULL */
    int32_t *out_cand;           /* device [n_keep * pages_per_chunk] candidate pages, or NULL */
} wa_prompt_stage;

/*
 * Bytes of device workspace wa_append_page needs for this layout (0 if the
 * layout is invalid).  Contents need no initialisation.
 */
size_t wa_append_workspace_bytes(const wa_layout *layout);

/*
 * Append one page (WorldAttention review, "HKV: Page-Level Multi-Tier
 * Memory": a page's keys are summarised by their mean; Inferix summary,
 * section 3.4, Step 4: pages enter the cache after the block is final).
 *
 *   k_pool[slot] = k_src, v_pool[slot] = v_src               (byte copies)
 *   page_means[slot][h][c] = (sum_t k_src[t][h][c]) / page_tokens   (fp64)
 *
 * k_src, v_src: [page_tokens][H][d].  If k_src (v_src) is the address of
 * pool slot `slot` itself, that copy is skipped ("mean-only": the producer
 * wrote the page in place).  v_src may be NULL: V is then left untouched.
 * Any other overlap of source and pool is undefined.  The sum is
 * accumulated in fp64 in a fixed order, so repeated calls are bitwise equal.
 * workspace: device, >= wa_append_workspace_bytes(layout) bytes.
 * Errors: NULL layout / k_src / k_pool / page_means / workspace, v_src
 * without v_pool, slot outside [0, max_pages), misaligned pointers,
 * workspace too small -> WA_ERR_INVALID_ARG; unsupported layout ->
 * WA_ERR_UNSUPPORTED.
 */
wa_status wa_append_page(const wa_layout *layout, const void *k_src, const void *v_src,
                         void *k_pool, void *v_pool, int32_t slot, double *page_means,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace wa_select_pages needs (0 if the arguments are
 * invalid).  prompt may be NULL.  The workspace must be zero-filled before
 * its first use (its first 256 bytes hold completion counters); every call leaves it
 * zero-filled where that matters again, so one workspace serves any number
 * of calls ordered on one stream.  Calls that overlap on one workspace race.
 */
size_t wa_select_workspace_bytes(const wa_layout *layout, int32_t n_q, int32_t n_cand,
                                 const wa_prompt_stage *prompt);

/*
 * Page stage (WorldAttention review, "HKV: Page-Level Multi-Tier Memory",
 * stage 2), all in fp64:
 *   qbar[h][c]  = (sum_i q[i][h][c]) / n_q
 *   alpha_j     = (sum_h sum_c qbar[h][c] * page_means[cand[j]][h][c]) / sqrt(d)
 *   out_idx[r]  = the candidate ranked r-th by (alpha desc, page id asc), r < k_p.
 * One score per page, shared by all heads.
 *
 * q: [n_q][H][d].  cand: device [n_cand] pool slots; NULL means slots
 * 0 ... n_cand-1.  prompt: NULL, or a prompt stage that produces the
 * candidates (then cand must be NULL and n_cand = n_keep * pages_per_chunk).
 * out_idx: device [k_p] int32.  out_scores: device [n_cand] double (alpha in
 * candidate order), or NULL.  A candidate id outside [0, max_pages) is never
 * read: it scores -inf and ranks last; ranks that only such ids could fill
 * get -1.  Duplicate ids are distinct candidates.  workspace: device, >=
 * wa_select_workspace_bytes(...) bytes, zero-filled before its first use
 * (see wa_select_workspace_bytes).
 * Errors: NULL layout / q / page_means / out_idx / workspace, n_q < 1,
 * n_cand < 1, k_p < 1 or k_p > n_cand, inconsistent prompt stage, misaligned
 * pointers, workspace too small -> WA_ERR_INVALID_ARG; n_cand or n_chunks > WA_MAX_CANDIDATES,
 * unsupported layout -> WA_ERR_UNSUPPORTED.
 */
wa_status wa_select_pages(const wa_layout *layout, const void *q, int32_t n_q,
                          const double *page_means, const int32_t *cand, int32_t n_cand,
                          const wa_prompt_stage *prompt, int32_t k_p, int32_t *out_idx,
                          double *out_scores, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * wa_select_pages without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The selection's workspace is a fixed
 * array inside the library's device image, one per GPU the library runs on,
 * held until the process ends; the call allocates nothing (its first call on
 * a device looks the array's address up).  Same arguments, results and
 * errors as wa_select_pages, plus: a selection whose workspace
 * (wa_select_workspace_bytes) exceeds WA_SELECT_NOALLOC_MAX_WORKSPACE ->
 * WA_ERR_UNSUPPORTED.  All calls on one GPU share the array, so calls that
 * overlap on one GPU (concurrent streams, threads) race; calls ordered on
 * one stream do not.  The call launches kernels only (no memset or copy), so
 * it can be captured in a HIP graph; make one call on each device before
 * capturing, so that the address look-up runs outside the capture.
 */
#define WA_SELECT_NOALLOC_MAX_WORKSPACE (8u << 20)
wa_status wa_select_pages_noalloc(const wa_layout *layout, const void *q, int32_t n_q,
                                  const double *page_means, const int32_t *cand, int32_t n_cand,
                                  const wa_prompt_stage *prompt, int32_t k_p, int32_t *out_idx,
                                  double *out_scores, void *stream);

/*
 * Sliding window plus selective fetch (Inferix summary, "Dual access
 * patterns": a range of the most recent blocks attended densely, and
 * specific distant blocks fetched by index for long-range context; the
 * WorldAttention review's Tab. 7 compares retrieval against keeping the
 * recent pages):
 *   out_idx[0 .. n_recent)            = recent[0 .. n_recent)   (range access)
 *   out_idx[n_recent .. n_recent+k_p) = the k_p candidates ranked first by
 *                                       (alpha desc, page id asc) among those
 *                                       whose id is not in recent
 * with alpha as in wa_select_pages.  recent: device [n_recent] pool slots
 * (the caller's most recent pages, in the order wanted in the output).
 * k_p may be 0 (window only) and n_recent 0 (wa_select_pages).  out_idx:
 * device [n_recent + k_p].  out_scores reports alpha for every candidate,
 * window pages included.  Other arguments, workspace (wa_select_workspace_
 * bytes) and errors as wa_select_pages, plus: n_recent < 0, n_recent + k_p
 * < 1, recent NULL with n_recent > 0 -> WA_ERR_INVALID_ARG; n_recent >
 * WA_MAX_WINDOW -> WA_ERR_UNSUPPORTED.
 */
wa_status wa_select_window(const wa_layout *layout, const void *q, int32_t n_q,
                           const double *page_means, const int32_t *cand, int32_t n_cand,
                           const wa_prompt_stage *prompt, const int32_t *recent,
                           int32_t n_recent, int32_t k_p, int32_t *out_idx, double *out_scores,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Gather (WorldAttention review, "Core Idea", item 3: the retrieved pages are
 * reorganised into one contiguous buffer):
 *   k_ctx[r * page_tokens + t] = k_pool[idx[r]][t]    for r < k_p, t < page_tokens
 * and the same for V; byte copies, pages in the order of idx.
 *
 * idx: device [k_p] int32, read on the device (no host synchronisation).
 * k_ctx, v_ctx: [k_p * page_tokens][H][d].  v_pool and v_ctx may both be
 * NULL (K only).  A rank whose idx is outside [0, max_pages) is left
 * unwritten.  The pool and the destination must not overlap.
 * Errors: NULL layout / k_pool / idx / k_ctx, only one of v_pool / v_ctx NULL,
 * k_p < 1, misaligned pointers -> WA_ERR_INVALID_ARG; k_p > 65535,
 * unsupported layout -> WA_ERR_UNSUPPORTED.
 */
wa_status wa_gather(const wa_layout *layout, const void *k_pool, const void *v_pool,
                    const int32_t *idx, int32_t k_p, void *k_ctx, void *v_ctx, void *stream);

/*
 * Block attention (Inferix summary, section 3.4, Step 3; the einsum post on
 * nakranivaibhav.github.io, "Where the mental model stops": scores are the
 * contraction over d, softmax and the value weighting follow it).  For head
 * h and query row i, with keys n running over the n_ctx rows of k_ctx and
 * then the n_own rows of k_own (values likewise):
 *   s_n   = (q[i][h] . k_n[h]) * softmax_scale
 *   out[i][h] = sum_n exp(s_n) v_n[h] / sum_n exp(s_n)
 *   lse[h][i] = log(sum_n exp(s_n))                 (natural log)
 * One softmax over both segments, no mask of any kind.
 *
 * q, out: [n_q][H][d]; k_ctx, v_ctx: [n_ctx][H][d]; k_own, v_own: [n_own][H][d].
 * Precision (WA_BF16): the queries and keys enter the matrix-core products
 * exactly as given (bf16 x bf16 products, fp32 accumulation); the softmax
 * scale is applied to each fp32 score by one fused multiply-add (together
 * with log2(e) and the running maximum) before the exponential, so a score
 * carries only fp32 rounding.  The probabilities are rounded to bf16 before
 * the value product (fp32 accumulation), and the row sum is taken from the
 * same rounded probabilities.  WA_F32 inputs are computed in fp32
 * throughout.
 * out_dtype: WA_F32, or WA_BF16 when layout.dtype is WA_BF16.
 * lse: device [H][n_q] float, or NULL.  n_ctx or n_own may be 0 (the
 * matching pointers may then be NULL).  out must not overlap any input.
 * page_tokens and max_pages of the layout are not used.
 * workspace: device memory of at least wa_attention_workspace_bytes() bytes
 * for the same arguments (16-byte aligned; may be NULL when that is 0),
 * owned by the caller; it holds partial results of a launch that splits the
 * key range of some (query block, head) items over several blocks so that
 * every CU has work, and must not be shared by calls in flight at once.
 * Errors: NULL layout / q / out, NULL pointers of a non-empty segment,
 * n_q < 1, n_ctx < 0, n_own < 0, n_ctx + n_own < 1, softmax_scale not finite
 * and > 0, misaligned pointers (lse: 4-byte aligned), workspace missing,
 * misaligned or too small -> WA_ERR_INVALID_ARG; head_dim or out_dtype not
 * supported for the dtype, n_ctx + n_own > 2^31 - 257 -> WA_ERR_UNSUPPORTED.
 */
wa_status wa_block_attention(const wa_layout *layout, const void *q, int32_t n_q,
                             const void *k_ctx, const void *v_ctx, int32_t n_ctx,
                             const void *k_own, const void *v_own, int32_t n_own,
                             float softmax_scale, int32_t out_dtype, void *out, float *lse,
                             void *workspace, size_t ws_bytes, void *stream);

/* Bytes of workspace wa_block_attention needs for these arguments on the
 * current device (0 for WA_F32 layouts and for launches that do not split;
 * 0 for arguments wa_block_attention would reject).  A pure function of the
 * arguments and the device's compute-unit count; launches nothing. */
size_t wa_attention_workspace_bytes(const wa_layout *layout, int32_t n_q, int32_t n_ctx,
                                    int32_t n_own);

/*
 * Paged block attention: the same result as wa_gather into k_ctx / v_ctx
 * followed by wa_block_attention over them, without the copy.  The context
 * keys are read in place from the pool pages idx[0 .. k_p-1] (key n is token
 * n % page_tokens of page idx[n / page_tokens], n < k_p * page_tokens), then
 * the n_own keys of k_own / v_own; one softmax, no mask.  The WorldAttention
 * review (its Tab. 9, in "Strengths") finds that rebuilding and copying the
 * retrieved KV into a contiguous buffer is the largest share of the sparse
 * path's time; reading the pages where they lie removes that copy, for every
 * denoising step.
 *
 * k_pool, v_pool: [max_pages][page_tokens][H][d] (16-byte aligned).
 * idx: device [k_p] int32 pool slots, read on the device; every entry must be
 * in [0, max_pages) (an entry outside is clamped into the pool so that no
 * access leaves it, and the result is then unspecified).  Other arguments,
 * precision, workspace (wa_attention_workspace_bytes with n_ctx =
 * k_p * page_tokens) and errors as wa_block_attention, plus: NULL k_pool /
 * v_pool / idx, idx not 4-byte aligned, k_p < 1, page_tokens or max_pages < 1
 * -> WA_ERR_INVALID_ARG; k_p * page_tokens > 2^31 - 257 -> WA_ERR_UNSUPPORTED.
 * The fast path reads whole 64-key tiles from one page and needs
 * page_tokens % 64 == 0 (bf16); other page sizes take a slower per-row path.
 */
wa_status wa_paged_attention(const wa_layout *layout, const void *q, int32_t n_q,
                             const void *k_pool, const void *v_pool, const int32_t *idx,
                             int32_t k_p, const void *k_own, const void *v_own, int32_t n_own,
                             float softmax_scale, int32_t out_dtype, void *out, float *lse,
                             void *workspace, size_t ws_bytes, void *stream);

/*
 * Bytes of device workspace wa_hsa_select needs (0 if the arguments are
 * invalid).  Contents need no initialisation.
 */
size_t wa_hsa_workspace_bytes(const wa_layout *layout, int32_t n_q, int32_t n_ctx,
                              int32_t n_own);

/*
 * Sparse branch, block selection (WorldAttention review, "HSA: Dual Branches
 * of Linear + Sparse": keys in blocks of 128 for the retrieved pages and 64
 * for the current chunk; a pooled attention map picks, per head, the fewest
 * blocks whose cumulative attention mass reaches tau_h, whose sparsity the
 * page measures with the Gini coefficient).  Key blocks, in [ctx ++ own]
 * order: context keys [128 j, 128 j + 128) (the last may hold 64), then own
 * keys [64 j, 64 j + 64) (the last may be shorter).  Query block b = queries
 * [256 b, 256 b + 256).  For head h and query block b, in fp64:
 *   qbar[c]   = mean over the block's queries of q[i][h][c]
 *   kbar_j[c] = mean over block j's keys of k[n][h][c]
 *   p_j       = softmax_j((qbar . kbar_j) * scale)
 *   G         = sum_i sum_j |p_i - p_j| / (2 nb sum_j p_j)       (Gini)
 *   selected  = the first m blocks in (p desc, block asc) order, m the least
 *               count whose running sum (in that order) is >= tau[h], m >= 1
 *               (all blocks when the sum never reaches tau[h]).
 * Output per item = h * q_blocks + b (q_blocks = ceil(n_q / 256)):
 *   sel_count[item]                     tiles selected
 *   sel_tiles[item * n_tiles + 0 ..)    the selected blocks' 64-key tiles of
 *                                       [ctx ++ own], ascending (context
 *                                       block j: tiles 2j, 2j+1; own block j:
 *                                       tile n_ctx / 64 + j)
 *   gini[item]                          G (if gini is not NULL)
 * with n_tiles = ceil((n_ctx + n_own) / 64): exactly the lists
 * wa_sparse_attention reads.
 *
 * q: [n_q][H][d]; k_ctx: [n_ctx][H][d]; k_own: [n_own][H][d] (layout.dtype;
 * V is not read).  tau: device [H] double.  sel_tiles: device int32
 * [q_blocks * H][n_tiles]; sel_count: device int32 [q_blocks * H]; gini:
 * device double [q_blocks * H] or NULL.  scale: the score scale (the
 * attention's softmax_scale).  ctx_sums_ready: 0 pools every block;
 * nonzero takes the context key blocks' sums already in the workspace as
 * they are (the own and query blocks are always pooled): they must have been
 * left there by an earlier call with this workspace, the same layout and
 * n_ctx, and the same k_ctx contents.  The context does not change over a
 * chunk's denoising steps (Inferix summary, section 3.4, Step 3), so the
 * chunk's first step pools it and the later steps reuse it.  The library
 * cannot check this; other sums give other selections.  With n_ctx = 0 the
 * flag is ignored.  workspace: device,
 * >= wa_hsa_workspace_bytes bytes, 16-byte aligned; calls in flight at once
 * need separate workspaces.
 * Errors: NULL layout / q / tau / sel_tiles / sel_count / workspace, NULL
 * pointer of a non-empty segment, n_q < 1, n_ctx < 0, n_own < 0,
 * n_ctx + n_own < 1, scale not finite and > 0, misaligned pointers,
 * workspace too small -> WA_ERR_INVALID_ARG; n_ctx not a multiple of 64,
 * head_dim > WA_HSA_MAX_HEAD_DIM, more than WA_MAX_HSA_BLOCKS key blocks,
 * unsupported layout -> WA_ERR_UNSUPPORTED.
 */
wa_status wa_hsa_select(const wa_layout *layout, const void *q, int32_t n_q, const void *k_ctx,
                        int32_t n_ctx, const void *k_own, int32_t n_own, double scale,
                        const double *tau, int32_t *sel_tiles, int32_t *sel_count, double *gini,
                        int32_t ctx_sums_ready, void *workspace, size_t ws_bytes, void *stream);

/*
 * Sparse branch, attention over the selected blocks (WorldAttention review,
 * "HSA: Dual Branches of Linear + Sparse"): for head h and query row i of
 * query block b = i / 256, item = h * q_blocks + b, the keys n run over the
 * 64-key tiles sel_tiles[item * n_tiles + 0 .. sel_count[item]) of
 * [ctx ++ own] (tile t = keys [64 t, 64 t + 64), cut at n_ctx + n_own), in
 * list order:
 *   out[i][h] = sum_n exp(s_n) v_n[h] / sum_n exp(s_n),  lse[h][i] = log(sum_n exp(s_n))
 * with s_n as in wa_block_attention: one softmax, no mask.  Over the full list
 * 0 .. n_tiles-1 this is wa_block_attention.
 *
 * sel_tiles / sel_count: as written by wa_hsa_select, or any lists with
 * 1 <= count <= n_tiles and strictly ascending entries in [0, n_tiles)
 * (a count or an entry outside its range is clamped so that every access
 * stays inside the keys, and the result is then unspecified).  Other
 * arguments as wa_block_attention; layout.dtype must be WA_BF16 and head_dim
 * 128.  The counts stay on the device: a first kernel lays the lists end to
 * end and, when they are uneven enough that one workgroup per item would
 * leave CUs idle, the lists are cut into equal runs over all CUs and the
 * pieces merged (otherwise the result is bit for bit that of
 * wa_block_attention over the same tiles laid end to end).
 * workspace: device, >= wa_sparse_workspace_bytes bytes, 16-byte aligned,
 * not shared by calls in flight at once.
 * Errors: as wa_block_attention, plus NULL or misaligned sel_tiles /
 * sel_count, workspace missing or too small -> WA_ERR_INVALID_ARG; a WA_F32
 * layout, more than WA_MAX_SPARSE_TILES tiles, more than 2^31 - 1 list
 * entries in all -> WA_ERR_UNSUPPORTED.
 */
wa_status wa_sparse_attention(const wa_layout *layout, const void *q, int32_t n_q,
                              const void *k_ctx, const void *v_ctx, int32_t n_ctx,
                              const void *k_own, const void *v_own, int32_t n_own,
                              float softmax_scale, const int32_t *sel_tiles,
                              const int32_t *sel_count, int32_t out_dtype, void *out,
                              float *lse, void *workspace, size_t ws_bytes, void *stream);

/* Bytes of workspace wa_sparse_attention needs for these arguments on the
 * current device (0 for arguments it would reject): the launch plan, the
 * running list offsets and partial results of (query blocks x heads + CUs)
 * pieces.  Launches nothing. */
size_t wa_sparse_workspace_bytes(const wa_layout *layout, int32_t n_q, int32_t n_ctx,
                                 int32_t n_own);

/*
 * Host-memory page tier (WorldAttention review, "HKV: Page-Level Multi-Tier
 * Memory": tier L1 (HBM) holds the retrieved pages, tier L2 (host DRAM) the
 * pages the current chunk does not use; Inferix summary, "KV Cache Manager",
 * offloading to main memory: a block fetched by index is loaded back into GPU
 * memory before the attention).  The caller keeps the page table (which
 * logical page is in which HBM slot or host slot) and the policy; these calls
 * move pages between tiers.
 *
 * wa_page_in:  k_pool[slot] = host_k[host_slot] (and V), host -> HBM;
 * wa_page_out: host_k[host_slot] = k_pool[slot] (and V), HBM -> host.
 * host_k, host_v: PINNED host memory from hipHostMalloc, [host_pages]
 * [page_tokens][H][d] in layout.dtype, owned by the caller; pageable memory is
 * rejected.  host_v and v_pool may both be NULL (K only).  The copies are
 * queued on `stream` for the copy engines (no kernel runs, nothing is
 * allocated) and run asynchronously: the caller orders them against the
 * attention that reads the slot with stream order or events, and must keep
 * the host pool unchanged until a page-in has finished.  Page means are not
 * touched (they stay in HBM for every page, so selection sees every tier).
 * Errors: NULL layout / host_k / k_pool, only one of host_v / v_pool NULL,
 * host_slot outside [0, host_pages), slot outside [0, max_pages), misaligned
 * pointers, a host pool that is not pinned host memory -> WA_ERR_INVALID_ARG;
 * a failed copy -> WA_ERR_HIP.
 */
wa_status wa_page_in(const wa_layout *layout, const void *host_k, const void *host_v,
                     int32_t host_pages, int32_t host_slot, void *k_pool, void *v_pool,
                     int32_t slot, void *stream);
wa_status wa_page_out(const wa_layout *layout, const void *k_pool, const void *v_pool,
                      int32_t slot, void *host_k, void *host_v, int32_t host_pages,
                      int32_t host_slot, void *stream);

/*
 * A page-in in parts (same tier passages as wa_page_in): token rows
 * [row0, row0 + n_rows) of host page host_slot go to the same rows of pool
 * slot `slot` (K, and V when given):
 *   k_pool[slot][row0 + r] = host_k[host_slot][row0 + r],  0 <= r < n_rows.
 * A page's rows are contiguous, so attention over the rows already copied
 * (wa_block_attention on that row range of the slot, with wa_merge_attention
 * combining the parts) can run while the rest of the page is copied; after
 * the last part, the attention over the page is exact up to the merge's
 * rounding.  Same arguments, conventions and errors as wa_page_in, plus:
 * row0 < 0, n_rows < 1, row0 + n_rows > page_tokens -> WA_ERR_INVALID_ARG.
 */
wa_status wa_page_in_rows(const wa_layout *layout, const void *host_k, const void *host_v,
                          int32_t host_pages, int32_t host_slot, void *k_pool, void *v_pool,
                          int32_t slot, int32_t row0, int32_t n_rows, void *stream);

/*
 * Merge of two attentions of the same queries over disjoint key sets A and B
 * (Inferix summary, "Ring Attention": partial attention over one chunk of keys
 * at a time, accumulated; here A = the pages resident in HBM, B = the pages
 * brought in from host memory, so that the attention over A runs while B is
 * copied).  For head h and query i, with lse_X = log sum_{n in X} exp(s_n):
 *   lse[h][i] = log(exp(lse_A) + exp(lse_B))
 *   out[i][h] = exp(lse_A - lse) out_A[i][h] + exp(lse_B - lse) out_B[i][h]
 * which is the attention over A u B (wa_block_attention's definition).
 * out_a, out_b: fp32 [n_q][H][d] (attention outputs with WA_F32 out_dtype);
 * lse_a, lse_b: fp32 [H][n_q], at least one of each pair finite; out:
 * [n_q][H][d] in out_dtype (WA_F32 or WA_BF16); lse: [H][n_q] or NULL.  out
 * may be out_a when out_dtype is WA_F32; no other overlap.  head_dim must be
 * a multiple of 4.
 * Errors: NULL layout / out_a / lse_a / out_b / lse_b / out, n_q < 1,
 * misaligned pointers -> WA_ERR_INVALID_ARG; out_dtype, head_dim % 4 != 0 ->
 * WA_ERR_UNSUPPORTED.
 */
wa_status wa_merge_attention(const wa_layout *layout, int32_t n_q, const float *out_a,
                             const float *lse_a, const float *out_b, const float *lse_b,
                             int32_t out_dtype, void *out, float *lse, void *stream);

/* Static text describing a status code. */
const char *wa_status_string(wa_status status);

#ifdef __cplusplus
}
#endif

#endif /* WA_H */
