/*
 * wa_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow fp64 CPU reference for the paged-KV block-attention path.
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * may load it; the HIP library never does, and the two share no code.
 *
 * Every input element is widened exactly to double (fp32 directly, bf16 by
 * placing its 16 bits on top of a float).  Everything after that is fp64.
 *
 * Sources (page title, section):
 *  [WA-HKV]  "WorldAttention: An Efficient Attention Architecture for
 *            Interactive Video World Models" (jaehun.me review), section
 *            "HKV: Page-Level Multi-Tier Memory": pages of 8 frames x 1,560
 *            tokens; prompt stage = top chunk by cosine similarity of prompt
 *            embeddings; page stage = top-K_p pages by
 *            alpha = mean(Q)^T mean(K_page) / sqrt(d_k), K_p = 4.
 *  [WA-CORE] same page, "Core Idea" item 3: the retrieved pages are
 *            reorganised into one contiguous buffer.
 *  [WA-T8]   same page, "Secret Weapon" paragraph on Tab. 8: several
 *            candidate chunks may be kept by the prompt stage.
 *  [INF-S3]  "Inferix: A Block-Diffusion based Next-Generation Inference
 *            Engine for World Simulation", section 3.4, "The Block-Diffusion
 *            Generation Pipeline", Step 3: the attention of a block's queries
 *            over [cached K ++ own K], [cached V ++ own V], with no mask
 *            inside the block.
 *  [EINSUM]  nakranivaibhav.github.io, the einsum post, "Where the mental
 *            model stops": scores are the contraction bhqd,bhkd->bhqk;
 *            softmax and the weighting of values are separate steps.
 *
 * Readings where the pages are silent are listed beside each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define WAO_F32 0
#define WAO_BF16 1

/* Widen element i of an fp32 or bf16 array to double, exactly. */
static double elem(const void *base, int dtype, int64_t i)
{
    float f;
    if (dtype == WAO_F32)
        return (double)((const float *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * Column mean of a token-major [rows][n_heads][head_dim] array:
 * out[h*head_dim + c] = (sum over t of x[t][h][c]) / rows.
 * [WA-HKV] uses it twice: the mean key of a page and the mean query of the
 * current chunk.
 */
void wao_column_mean(const void *x, int dtype, int64_t rows, int64_t hd, double *out)
{
    /* each column is summed in row order t = 0, 1, ..., rows-1 */
    for (int64_t col = 0; col < hd; ++col)
        out[col] = 0.0;
    for (int64_t t = 0; t < rows; ++t)
        for (int64_t col = 0; col < hd; ++col)
            out[col] += elem(x, dtype, t * hd + col);
    for (int64_t col = 0; col < hd; ++col)
        out[col] = out[col] / (double)rows;
}

/*
 * Page stage score [WA-HKV]: alpha_j = sum_{h,c} qbar[h,c] * kbar_j[h,c] / sqrt(d_k)
 * for every candidate page id cand[j].  Reading: one score per page shared by
 * all heads (qbar and kbar are the per-head means laid end to end), and d_k
 * is the head dimension.
 */
void wao_page_scores(const double *qbar, const double *page_means, int64_t hd,
                     int head_dim, const int32_t *cand, int n_cand, double *alpha)
{
    for (int j = 0; j < n_cand; ++j) {
        const double *kbar = page_means + (int64_t)cand[j] * hd;
        double s = 0.0;
        for (int64_t col = 0; col < hd; ++col)
            s += qbar[col] * kbar[col];
        alpha[j] = s / sqrt((double)head_dim);
    }
}

/* (score desc, id asc): nonzero when (sa, ia) ranks before (sb, ib). */
static int ranks_before(double sa, int32_t ia, double sb, int32_t ib)
{
    return sa > sb || (sa == sb && ia < ib);
}

/*
 * Top-k by score [WA-HKV]: out[r] = the id ranked r-th under (score
 * descending, id ascending), r < k.  Plain selection: k passes, each taking
 * the best item not yet taken.  Reading: the pages give no tie rule; the
 * lower id wins, and the output is in rank order.
 */
void wao_top_k(const double *score, const int32_t *ids, int n, int k, int32_t *out)
{
    char *taken = (char *)calloc((size_t)n, 1);
    for (int r = 0; r < k; ++r) {
        int best = -1;
        for (int j = 0; j < n; ++j) {
            if (taken[j])
                continue;
            if (best < 0 || ranks_before(score[j], ids[j], score[best], ids[best]))
                best = j;
        }
        taken[best] = 1;
        out[r] = ids[best];
    }
    free(taken);
}

/*
 * Prompt stage [WA-HKV]: cos_m = <p, p_m> / (|p| |p_m|) between the current
 * prompt embedding p and each past chunk's embedding p_m (fp32 inputs).
 */
void wao_prompt_cosine(const float *chunk_prompts, const float *cur, int n_chunks,
                       int emb_dim, double *cos_out)
{
    double pp = 0.0;
    for (int e = 0; e < emb_dim; ++e)
        pp += (double)cur[e] * (double)cur[e];
    for (int m = 0; m < n_chunks; ++m) {
        const float *pm = chunk_prompts + (int64_t)m * emb_dim;
        double dot = 0.0, nn = 0.0;
        for (int e = 0; e < emb_dim; ++e) {
            dot += (double)cur[e] * (double)pm[e];
            nn += (double)pm[e] * (double)pm[e];
        }
        /* Reading: an embedding of zero norm has no direction, so its cosine
         * is -inf (that chunk ranks last; ties go to the lower chunk id). */
        cos_out[m] = (pp > 0.0 && nn > 0.0) ? dot / (sqrt(pp) * sqrt(nn)) : -INFINITY;
    }
}

/*
 * Candidate pages of the prompt stage [WA-HKV, WA-T8]: the n_keep chunks
 * ranked first by (cosine desc, chunk id asc); their pages, chunk by chunk
 * in rank order and page by page in the map's order.  Reading: "the top-1
 * chunk and its neighbours" is the n_keep best chunks by the same cosine.
 */
void wao_prompt_candidates(const double *cos_m, int n_chunks, const int32_t *chunk_pages,
                           int pages_per_chunk, int n_keep, int32_t *chunks_out,
                           int32_t *cand_out)
{
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_chunks);
    for (int m = 0; m < n_chunks; ++m)
        ids[m] = m;
    wao_top_k(cos_m, ids, n_chunks, n_keep, chunks_out);
    for (int r = 0; r < n_keep; ++r)
        for (int p = 0; p < pages_per_chunk; ++p)
            cand_out[r * pages_per_chunk + p] =
                chunk_pages[(int64_t)chunks_out[r] * pages_per_chunk + p];
    free(ids);
}

/*
 * Gather [WA-CORE]: rank r of the output is a byte copy of pool page idx[r].
 * Reading: pages are laid out in the order of idx (score order).
 */
void wao_gather(const void *pool, int64_t page_bytes, const int32_t *idx, int k_p, void *out)
{
    for (int r = 0; r < k_p; ++r)
        memcpy((char *)out + (int64_t)r * page_bytes,
               (const char *)pool + (int64_t)idx[r] * page_bytes, (size_t)page_bytes);
}

/*
 * Block attention [INF-S3, EINSUM].  For head h and query row i the keys are
 * the rows of k_ctx followed by the rows of k_own (concatenation along the
 * sequence), with the values in the same order:
 *   s_n = (q_i . k_n) * scale
 *   o_i = sum_n softmax(s)_n v_n,   lse_i = log sum_n exp(s_n).
 * No mask of any kind.  The softmax is evaluated as exp(s_n - max s) / sum,
 * which is the same function, kept in range.
 *
 * rows: the query rows to compute (n_rows of them); out is
 * [n_rows][n_heads][head_dim], lse is [n_heads][n_rows] (may be NULL).
 * Rows and heads are independent, so they are spread over threads.
 */
void wao_attention(const void *q, const void *k_ctx, const void *v_ctx, int64_t n_ctx,
                   const void *k_own, const void *v_own, int64_t n_own, int n_heads,
                   int head_dim, int dtype, double scale, const int64_t *rows,
                   int64_t n_rows, double *out, double *lse, int n_threads)
{
    const int64_t hd = (int64_t)n_heads * head_dim;
    const int64_t n_keys = n_ctx + n_own;
    const int64_t n_tasks = n_rows * n_heads;
#pragma omp parallel num_threads(n_threads > 0 ? n_threads : 1)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
        double *qi = (double *)malloc(sizeof(double) * (size_t)head_dim);
        double *acc = (double *)malloc(sizeof(double) * (size_t)head_dim);
#pragma omp for schedule(dynamic, 4)
        for (int64_t task = 0; task < n_tasks; ++task) {
            const int64_t r = task / n_heads;
            const int h = (int)(task % n_heads);
            const int64_t i = rows[r];
            for (int c = 0; c < head_dim; ++c)
                qi[c] = elem(q, dtype, i * hd + (int64_t)h * head_dim + c);
            /* scores over the concatenated key sequence */
            double m = -INFINITY;
            for (int64_t n = 0; n < n_keys; ++n) {
                const void *kb = n < n_ctx ? k_ctx : k_own;
                const int64_t row = n < n_ctx ? n : n - n_ctx;
                double dot = 0.0;
                for (int c = 0; c < head_dim; ++c)
                    dot += qi[c] * elem(kb, dtype, row * hd + (int64_t)h * head_dim + c);
                s[n] = dot * scale;
                if (s[n] > m)
                    m = s[n];
            }
            double l = 0.0;
            for (int64_t n = 0; n < n_keys; ++n) {
                s[n] = exp(s[n] - m);
                l += s[n];
            }
            for (int c = 0; c < head_dim; ++c)
                acc[c] = 0.0;
            for (int64_t n = 0; n < n_keys; ++n) {
                const void *vb = n < n_ctx ? v_ctx : v_own;
                const int64_t row = n < n_ctx ? n : n - n_ctx;
                for (int c = 0; c < head_dim; ++c)
                    acc[c] += s[n] * elem(vb, dtype, row * hd + (int64_t)h * head_dim + c);
            }
            for (int c = 0; c < head_dim; ++c)
                out[r * hd + (int64_t)h * head_dim + c] = acc[c] / l;
            if (lse)
                lse[(int64_t)h * n_rows + r] = m + log(l);
        }
        free(s);
        free(qi);
        free(acc);
    }
}
