// bf16 block attention on the CDNA4 matrix cores (Inferix summary, section
// 3.4, Step 3: the block's queries attend over [cached K ++ own K],
// [cached V ++ own V], one softmax, no mask; the einsum post on
// nakranivaibhav.github.io, "Where the mental model stops": Q K^T and P V are
// the only contractions, softmax sits between them).
//
// Design (gfx950, head_dim 128):
//  * Block = 4 wavefronts x 64 queries = 256 queries of one head.  Blocks are
//    renumbered so that consecutive (head, query-block) tiles land on the
//    same XCD: the blocks of one head then stream the same K/V through one
//    L2.
//  * K/V tiles of 64 keys are staged through LDS, double buffered (64 KB):
//    K as [key][d] and V transposed to [d][key], both with XOR-swizzled
//    16-byte chunks so the matrix-core operand reads are conflict free.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (fp32 accumulation): a lane
//    then holds 32 keys of ONE query, so the running max / sum of a query
//    live in one lane (plus one cross-half exchange), and rescaling the
//    output is a per-lane multiply.
//  * P = exp2(S * scale*log2(e) - m) in fp32, rounded to bf16 and fed as the
//    B operand of O^T += V^T P^T straight from the S^T accumulator layout;
//    the V^T tile stores keys in the matching permuted order.
//  * The output is only rescaled when some lane's max grew.
#include <math.h>

#include "wa_internal.h"

namespace wa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

static constexpr int kD = 128;        // head dim
static constexpr int kBM = 256;       // queries per block
static constexpr int kBN = 64;        // keys per tile
static constexpr int kThreads = 256;  // 4 wavefronts

// element offsets inside one LDS tile
__device__ __forceinline__ int k_off(int key, int chunk) {
    return key * kD + ((chunk ^ (key & 15)) << 3);
}
__device__ __forceinline__ int vt_off(int dv, int chunk) {
    return dv * kBN + ((chunk ^ ((dv >> 1) & 7)) << 3);
}

__device__ __forceinline__ int xcd_remap(int bid, int n) {
    const int q = n >> 3, r = n & 7;
    const int x = bid & 7, i = bid >> 3;
    return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

struct AttnArgs {
    const uint16_t *q;
    const uint16_t *k_ctx;
    const uint16_t *v_ctx;
    const uint16_t *k_own;
    const uint16_t *v_own;
    int n_q, n_ctx, n_own, n_heads, q_blocks;
    float c;        // softmax_scale * log2(e)
    int out_bf16;
    void *out;
    float *lse;
};

struct Smem {
    uint16_t k[2][kBN * kD];
    uint16_t vt[2][kD * kBN];
};

__device__ __forceinline__ const uint16_t *seq_row(const uint16_t *ctx, const uint16_t *own,
                                                   int n, int n_ctx, int64_t hd) {
    return n < n_ctx ? ctx + (int64_t)n * hd : own + (int64_t)(n - n_ctx) * hd;
}

// S^T for 32 keys (rows 32*kb ... of the LDS tile) against the wave's 64
// queries: s[qb] holds keys x queries 32qb ... 32qb+31.
template <bool MASKED>
__device__ __forceinline__ void subtile_scores(const uint16_t *ks, const bf16x8 (&qf)[2][8],
                                               f32x16 (&s)[2], int kb, int lr, int hb,
                                               int key0, int n_keys) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[qb][i] = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        const bf16x8 ak = *(const bf16x8 *)&ks[k_off(32 * kb + lr, 2 * st + hb)];
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[0][st], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[1][st], s[1], 0, 0, 0);
    }
    if (MASKED) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * hb + (i & 3);
            if (key >= n_keys) {
                s[0][i] = -INFINITY;
                s[1][i] = -INFINITY;
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_attn_bf16(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) Smem sm;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, lr = lane & 31, hb = lane >> 5;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int h = logical / a.q_blocks;
    const int q0 = (logical % a.q_blocks) * kBM + wave * 64;
    const int64_t hd = (int64_t)a.n_heads * kD;
    const int n_keys = a.n_ctx + a.n_own;
    const int n_tiles = (n_keys + kBN - 1) / kBN;
    const bool ragged = (n_keys % kBN) != 0;

    // this wave's 64 queries as B operands: qf[qb][st] = Q[q0+32qb+lr][16st+8hb ..+7]
    bf16x8 qf[2][8];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int row = q0 + 32 * qb + lr;
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            if (row < a.n_q)
                qf[qb][st] = *(const bf16x8 *)(a.q + (int64_t)row * hd + h * kD + 16 * st + 8 * hb);
            else
                qf[qb][st] = (bf16x8)(__bf16)0.f;
        }
    }

    f32x16 o[4][2];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[b][qb][i] = 0.f;
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

    // loader mapping: K rows (tid>>4)+16i, chunk tid&15; V keys 4*(tid>>4)+j, chunk tid&15
    const int lc = tid & 15, lg = tid >> 4;
    uint4 kreg[4], vreg[4];
    auto load_tile = [&](int key0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = key0 + lg + 16 * i;
            kreg[i] = n < n_keys
                          ? *(const uint4 *)(seq_row(a.k_ctx, a.k_own, n, a.n_ctx, hd) + h * kD + 8 * lc)
                          : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = key0 + 4 * lg + j;
            vreg[j] = n < n_keys
                          ? *(const uint4 *)(seq_row(a.v_ctx, a.v_own, n, a.n_ctx, hd) + h * kD + 8 * lc)
                          : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *(uint4 *)&sm.k[buf][k_off(lg + 16 * i, lc)] = kreg[i];
        // V: keys 4lg..4lg+3 x dims 8lc..8lc+7, transposed into [dim][key]
        const int g16 = lg >> 2, w = lg & 3;
        const int pos = (w >> 1) | ((w & 1) << 1);
        const int unit = g16 * 4 + pos;           // 8-byte unit in the 64-key row
        const int chunk = unit >> 1, half = unit & 1;
        const uint32_t v0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
        const uint32_t v1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
        const uint32_t v2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
        const uint32_t v3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int wi = e >> 1;
            uint32_t w0, w1;
            if (e & 1) {
                w0 = (v0[wi] >> 16) | (v1[wi] & 0xffff0000u);
                w1 = (v2[wi] >> 16) | (v3[wi] & 0xffff0000u);
            } else {
                w0 = (v0[wi] & 0xffffu) | (v1[wi] << 16);
                w1 = (v2[wi] & 0xffffu) | (v3[wi] << 16);
            }
            *(uint2 *)&sm.vt[buf][vt_off(8 * lc + e, chunk) + 4 * half] = make_uint2(w0, w1);
        }
    };

    // softmax of one 32-key sub-tile and its P V^T product
    auto softmax_pv = [&](int buf, int kb, f32x16 (&s)[2]) {
        bf16x8 pb[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float mt = s[qb][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[qb][i]);
            mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
            const float m_new = fmaxf(m[qb], mt);
            if (__any(m_new > m[qb])) {
                const float corr = __builtin_amdgcn_exp2f((m[qb] - m_new) * a.c);
                l[qb] *= corr;
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[b][qb][i] *= corr;
                m[qb] = m_new;
            }
            const float mc = m[qb] * a.c;
            float ls = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[qb][i], a.c, -mc));
                s[qb][i] = p;
                ls += p;
            }
            l[qb] += ls;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int t = 0; t < 8; ++t) pb[qb][jj][t] = (__bf16)s[qb][8 * jj + t];
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int j = 2 * kb + jj;
                const bf16x8 av = *(const bf16x8 *)&sm.vt[buf][vt_off(32 * b + lr, 2 * j + hb)];
                o[b][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[0][jj], o[b][0], 0, 0, 0);
                o[b][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[1][jj], o[b][1], 0, 0, 0);
            }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        const bool more = t + 1 < n_tiles;
        if (more) load_tile((t + 1) * kBN);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 s[2];
            if (ragged && t == n_tiles - 1)
                subtile_scores<true>(sm.k[buf], qf, s, kb, lr, hb, t * kBN, n_keys);
            else
                subtile_scores<false>(sm.k[buf], qf, s, kb, lr, hb, t * kBN, n_keys);
            softmax_pv(buf, kb, s);
        }
        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }

    // epilogue: O^T[dv][q] / l, lanes l and l^32 hold the two halves of l
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float lt = l[qb] + __shfl_xor(l[qb], 32, 64);
        const float inv = 1.f / lt;
        const int row = q0 + 32 * qb + lr;
        if (row < a.n_q) {
            const int64_t base = (int64_t)row * hd + h * kD;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int dv = 32 * b + 8 * g + 4 * hb;
                    const float x0 = o[b][qb][4 * g] * inv, x1 = o[b][qb][4 * g + 1] * inv;
                    const float x2 = o[b][qb][4 * g + 2] * inv, x3 = o[b][qb][4 * g + 3] * inv;
                    if (a.out_bf16) {
                        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                        bf16x4 v = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
                        *(bf16x4 *)((uint16_t *)a.out + base + dv) = v;
                    } else {
                        *(float4 *)((float *)a.out + base + dv) = make_float4(x0, x1, x2, x3);
                    }
                }
            if (a.lse && hb == 0)
                a.lse[(int64_t)h * a.n_q + row] = (m[qb] * a.c + __log2f(lt)) * 0.69314718055994531f;
        }
    }
}

hipError_t launch_attention_bf16(int32_t n_heads, const uint16_t *q, int32_t n_q,
                                 const uint16_t *k_ctx, const uint16_t *v_ctx, int32_t n_ctx,
                                 const uint16_t *k_own, const uint16_t *v_own, int32_t n_own,
                                 float scale, int32_t out_dtype, void *out, float *lse,
                                 hipStream_t s) {
    AttnArgs a;
    a.q = q;
    a.k_ctx = k_ctx;
    a.v_ctx = v_ctx;
    a.k_own = k_own;
    a.v_own = v_own;
    a.n_q = n_q;
    a.n_ctx = n_ctx;
    a.n_own = n_own;
    a.n_heads = n_heads;
    a.q_blocks = (n_q + kBM - 1) / kBM;
    a.c = scale * 1.4426950408889634f;
    a.out_bf16 = out_dtype == WA_BF16;
    a.out = out;
    a.lse = lse;
    const unsigned grid = (unsigned)(a.q_blocks * n_heads);
    hipLaunchKernelGGL(k_attn_bf16, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace wa
