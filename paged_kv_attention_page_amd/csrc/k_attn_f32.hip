// fp32 block attention (Inferix summary, section 3.4, Step 3): each query of
// the chunk attends over the gathered pages (or, paged, the selected pool
// pages read in place) followed by the chunk's own K/V, one softmax, no mask.  Used for fp32 layouts (head_dim 64 or 128), where
// exactness matters more than speed; plain FMA arithmetic, no matrix cores.
//
// Block = 64 queries of one head; 4 threads per query, each owning d/4 of
// the head dimensions.  K/V tiles of 32 keys are staged in LDS.  Per tile:
// scores (partial dot + two quad shuffles), tile max, one rescale of the
// running output, then the probability-weighted value sum.  exp2 with
// scale*log2(e) folded into the scores.
#include <math.h>

#include "wa_internal.h"

namespace wa {

static constexpr int kF32Queries = 64;
static constexpr int kF32Keys = 32;

template <int D>
__global__ __launch_bounds__(256) void k_attn_f32(const float *__restrict__ q, int n_q,
                                                  const float *__restrict__ k_ctx,
                                                  const float *__restrict__ v_ctx, int n_ctx,
                                                  const float *__restrict__ k_own,
                                                  const float *__restrict__ v_own, int n_own,
                                                  int n_heads, float c, float *__restrict__ out,
                                                  float *__restrict__ lse,
                                                  const int32_t *__restrict__ idx, int page_tokens,
                                                  int max_pages) {
    constexpr int DQ = D / 4;   // dims per thread
    __shared__ float ks[kF32Keys][D];
    __shared__ float vs[kF32Keys][D];
    const int h = blockIdx.y;
    const int t = threadIdx.x;
    const int qi = blockIdx.x * kF32Queries + (t >> 2);
    const int sub = t & 3;
    const int64_t hd = (int64_t)n_heads * D;
    const int n_keys = n_ctx + n_own;

    float qv[DQ], o[DQ];
#pragma unroll
    for (int e = 0; e < DQ; ++e) {
        qv[e] = qi < n_q ? q[(int64_t)qi * hd + h * D + sub * DQ + e] * c : 0.f;
        o[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    for (int k0 = 0; k0 < n_keys; k0 += kF32Keys) {
        __syncthreads();
        // stage the tile: kF32Keys * D floats of K and of V, 16 bytes at a time
        for (int i = t; i < kF32Keys * D / 4; i += blockDim.x) {
            const int row = i / (D / 4), cv = i % (D / 4);
            const int n = k0 + row;
            float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
            if (n < n_keys) {
                // context row n: row n of the gathered buffer, or (paged) token
                // n % page_tokens of pool page idx[n / page_tokens], the id
                // clamped into the pool (memory safety only)
                int64_t row = n;
                if (idx && n < n_ctx) {
                    const int r = n / page_tokens;
                    int id = idx[r];
                    id = id < 0 ? 0 : (id >= max_pages ? max_pages - 1 : id);
                    row = (int64_t)id * page_tokens + (n - r * page_tokens);
                }
                const float *kb = n < n_ctx ? k_ctx + row * hd : k_own + (int64_t)(n - n_ctx) * hd;
                const float *vb = n < n_ctx ? v_ctx + row * hd : v_own + (int64_t)(n - n_ctx) * hd;
                kk = *(const float4 *)(kb + h * D + cv * 4);
                vv = *(const float4 *)(vb + h * D + cv * 4);
            }
            *(float4 *)&ks[row][cv * 4] = kk;
            *(float4 *)&vs[row][cv * 4] = vv;
        }
        __syncthreads();
        float s[kF32Keys];
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < kF32Keys; ++j) {
            float p = 0.f;
#pragma unroll
            for (int e = 0; e < DQ; ++e) p = fmaf(qv[e], ks[j][sub * DQ + e], p);
            p += __shfl_xor(p, 1, 64);
            p += __shfl_xor(p, 2, 64);
            s[j] = (k0 + j < n_keys) ? p : -INFINITY;
            mt = fmaxf(mt, s[j]);
        }
        const float m_new = fmaxf(m, mt);
        const float corr = exp2f(m - m_new);   // 0 on the first tile
        l *= corr;
#pragma unroll
        for (int e = 0; e < DQ; ++e) o[e] *= corr;
#pragma unroll
        for (int j = 0; j < kF32Keys; ++j) {
            const float p = exp2f(s[j] - m_new);
            l += p;
#pragma unroll
            for (int e = 0; e < DQ; ++e) o[e] = fmaf(p, vs[j][sub * DQ + e], o[e]);
        }
        m = m_new;
    }
    if (qi < n_q) {
        const float inv = 1.f / l;
#pragma unroll
        for (int e = 0; e < DQ; ++e) out[(int64_t)qi * hd + h * D + sub * DQ + e] = o[e] * inv;
        // natural-log sum of exp of the unscaled-by-log2e scores
        if (lse && sub == 0) lse[(int64_t)h * n_q + qi] = (m + log2f(l)) * 0.69314718055994531f;
    }
}

hipError_t launch_attention_f32(int32_t n_heads, int32_t head_dim, const float *q, int32_t n_q,
                                const float *k_ctx, const float *v_ctx, int32_t n_ctx,
                                const float *k_own, const float *v_own, int32_t n_own,
                                float scale, float *out, float *lse, const PagedCtx &pg,
                                hipStream_t s) {
    const float c = scale * 1.4426950408889634f;
    const dim3 grid((unsigned)((n_q + kF32Queries - 1) / kF32Queries), (unsigned)n_heads);
    if (head_dim == 64)
        hipLaunchKernelGGL(k_attn_f32<64>, grid, dim3(256), 0, s, q, n_q, k_ctx, v_ctx, n_ctx,
                           k_own, v_own, n_own, n_heads, c, out, lse, pg.idx, pg.page_tokens,
                           pg.max_pages);
    else
        hipLaunchKernelGGL(k_attn_f32<128>, grid, dim3(256), 0, s, q, n_q, k_ctx, v_ctx, n_ctx,
                           k_own, v_own, n_own, n_heads, c, out, lse, pg.idx, pg.page_tokens,
                           pg.max_pages);
    return hipGetLastError();
}

}  // namespace wa
