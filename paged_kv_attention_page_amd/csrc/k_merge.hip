// Merge of two attentions of the same queries over disjoint key sets A and B
// (Inferix summary, "Ring Attention": each step attends the local queries to
// one chunk of keys and values and the partial results are accumulated;
// here the two parts are the pages resident in HBM and the pages being
// brought in from host memory, WorldAttention review, "HKV: Page-Level
// Multi-Tier Memory", tiers L1 and L2).
//
// With lse_X = log sum_{n in X} exp(s_n) and out_X the softmax-weighted mean
// of the values over X, attention over A u B is
//   lse = log(exp(lse_A) + exp(lse_B)),
//   out = exp(lse_A - lse) out_A + exp(lse_B - lse) out_B,
// evaluated against m = max(lse_A, lse_B) so that no exponential overflows.
// HBM-bound: one thread per 16-byte vector of the fp32 inputs.
#include <math.h>

#include "wa_internal.h"

namespace wa {

static constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void k_merge_attention(
    const float4 *__restrict__ out_a, const float *__restrict__ lse_a,
    const float4 *__restrict__ out_b, const float *__restrict__ lse_b, int64_t n_vec, int n_q,
    int n_heads, int vec_per_head, int out_bf16, void *__restrict__ out, float *__restrict__ lse) {
    const int64_t v = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
    if (v >= n_vec) return;
    const int64_t per_row = (int64_t)n_heads * vec_per_head;
    const int64_t i = v / per_row;
    const int h = (int)((v - i * per_row) / vec_per_head);
    const float la = lse_a[(int64_t)h * n_q + i], lb = lse_b[(int64_t)h * n_q + i];
    const float m = fmaxf(la, lb);
    const float wa = expf(la - m), wb = expf(lb - m);
    const float inv = 1.f / (wa + wb);
    const float4 a = out_a[v], b = out_b[v];
    const float x0 = (wa * a.x + wb * b.x) * inv, x1 = (wa * a.y + wb * b.y) * inv;
    const float x2 = (wa * a.z + wb * b.z) * inv, x3 = (wa * a.w + wb * b.w) * inv;
    if (out_bf16) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 o = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
        ((bf16x4 *)out)[v] = o;
    } else {
        ((float4 *)out)[v] = make_float4(x0, x1, x2, x3);
    }
    if (lse && (v - i * per_row) % vec_per_head == 0)
        lse[(int64_t)h * n_q + i] = m + logf(wa + wb);
}

hipError_t launch_merge_attention(int32_t n_heads, int32_t head_dim, int32_t n_q,
                                  const float *out_a, const float *lse_a, const float *out_b,
                                  const float *lse_b, int32_t out_dtype, void *out, float *lse,
                                  hipStream_t s) {
    const int vec_per_head = head_dim / 4;
    const int64_t n_vec = (int64_t)n_q * n_heads * vec_per_head;
    const unsigned blocks = (unsigned)((n_vec + kMergeThreads - 1) / kMergeThreads);
    hipLaunchKernelGGL(k_merge_attention, dim3(blocks), dim3(kMergeThreads), 0, s,
                       (const float4 *)out_a, lse_a, (const float4 *)out_b, lse_b, n_vec, n_q,
                       n_heads, vec_per_head, out_dtype == WA_BF16 ? 1 : 0, out, lse);
    return hipGetLastError();
}

}  // namespace wa
