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
//  * K/V tiles of 64 keys go from global memory straight into LDS with
//    global_load_lds_dwordx4 (no register staging), in a ring of kStages
//    tiles; the loads of tile t+kStages-1 are in flight while tile t is
//    computed.  Both tiles are row-major [key][d] with XOR-swizzled 16-byte
//    chunks; the swizzle is applied on the global side of the copy.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (fp32 accumulation) on 32-key
//    sub-tiles: a lane then holds 16 keys of ONE query per query block, so a
//    query's running max / sum live in one lane pair (one permlane32 swap)
//    and rescaling the output is a per-lane multiply.
//  * O^T += V^T P^T: P comes straight from the S^T accumulator layout
//    (exp2 of S * scale*log2(e) - m, rounded to bf16); V^T operands are read
//    with ds_read_b64_tr_b16, whose 16-lane 4x16 -> 16x4 transpose turns the
//    row-major V tile into the key-contiguous operand, in the key order that
//    matches P.
//  * Software pipeline per wave: the Q K^T products of the next sub-tile are
//    issued before the exponentials of the current one, so matrix-core and
//    vector work overlap; the output is only rescaled when a query's max
//    grows by more than 2^8 in the exp2 domain (exact either way: the final
//    division uses the same reference max).
#include <math.h>

#include "wa_internal.h"

namespace wa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define WA_LDS __attribute__((address_space(3)))

static constexpr int kD = 128;        // head dim
static constexpr int kBM = 256;       // queries per block
static constexpr int kBN = 64;        // keys per tile
static constexpr int kThreads = 256;  // 4 wavefronts
static constexpr int kStages = 3;     // LDS ring depth (tiles)
static constexpr int kTileElems = kBN * kD;
static constexpr float kRescaleLog2 = 8.f;   // rescale when the max grows by > 2^8

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

// One 16-byte-per-lane DMA from global memory into LDS: lane i's 16 bytes
// land at lds_base + 16 i.  Issued through inline assembly so that the
// compiler does not insert its own (conservative) waits for the copy before
// unrelated LDS reads; the kernel waits for the copies itself (vmcnt) before
// the barrier that publishes a tile.  Nothing else in the kernel uses m0.
__device__ __forceinline__ void dma16(const void *gptr, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(gptr)
                 : "memory", "m0");
}
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_vm8() { asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); }

__device__ __forceinline__ unsigned lds_addr(const void *p) {
    return (unsigned)(uintptr_t)(const WA_LDS void *)p;
}

__device__ __forceinline__ float xhalf_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One LDS variable per ring stage: every access below names its stage at
// compile time, so the compiler can tell the stage being refilled by DMA from
// the stages being read, and does not wait for the refill before reading.
__shared__ __attribute__((aligned(1024))) uint16_t lds_k0[kTileElems];
__shared__ __attribute__((aligned(1024))) uint16_t lds_k1[kTileElems];
__shared__ __attribute__((aligned(1024))) uint16_t lds_k2[kTileElems];
__shared__ __attribute__((aligned(1024))) uint16_t lds_v0[kTileElems];
__shared__ __attribute__((aligned(1024))) uint16_t lds_v1[kTileElems];
__shared__ __attribute__((aligned(1024))) uint16_t lds_v2[kTileElems];

template <int S>
struct StageTag {
    static constexpr int value = S;
};

template <int S>
__device__ __forceinline__ uint16_t *kst() {
    static_assert(S >= 0 && S < kStages, "stage");
    if constexpr (S == 0) return lds_k0;
    else if constexpr (S == 1) return lds_k1;
    else return lds_k2;
}
template <int S>
__device__ __forceinline__ uint16_t *vst() {
    if constexpr (S == 0) return lds_v0;
    else if constexpr (S == 1) return lds_v1;
    else return lds_v2;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_attn_bf16(AttnArgs a) {

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, lr = lane & 31, hb = lane >> 5;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int h = logical / a.q_blocks;
    const int q0 = (logical % a.q_blocks) * kBM + wave * 64;
    const int64_t hd = (int64_t)a.n_heads * kD;
    const int n_keys = a.n_ctx + a.n_own;
    const int n_tiles = (n_keys + kBN - 1) / kBN;
    const bool ragged = (n_keys % kBN) != 0;
    const float c = a.c;
    const float thr = kRescaleLog2 / c;   // raw-score growth that forces a rescale

    // ---- tile loads: wave w copies rows 16w ... 16w+15 of the K and V tiles,
    // 4 rows (1 KB) per instruction; lane -> (row 16w+4i+lane/16, slot lane%16)
    const int ld_row0 = 16 * wave + (lane >> 4);
    const int ld_slot = lane & 15;
    const unsigned ld_base = __builtin_amdgcn_readfirstlane(16 * wave * kD * 2);
    auto issue_tile = [&](int t, uint16_t *ks, uint16_t *vs) __attribute__((always_inline)) {
        const int key0 = t * kBN;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = ld_row0 + 4 * i;
            int n = key0 + row;
            n = n < n_keys ? n : n_keys - 1;           // rows past the end repeat the last key
            const bool in_ctx = n < a.n_ctx;
            const int64_t off = (int64_t)(in_ctx ? n : n - a.n_ctx) * hd + h * kD;
            const uint16_t *kr = (in_ctx ? a.k_ctx : a.k_own) + off;
            const uint16_t *vr = (in_ctx ? a.v_ctx : a.v_own) + off;
            const int kchunk = ld_slot ^ (row & 15);
            const int vchunk = ld_slot ^ (4 * (row & 3));
            dma16(kr + 8 * kchunk, lds_addr(ks) + ld_base + 4 * i * kD * 2);
            dma16(vr + 8 * vchunk, lds_addr(vs) + ld_base + 4 * i * kD * 2);
        }
    };

    // ---- this wave's 64 queries as B operands: qf[qb][st] = Q[q0+32qb+lr][16st+8hb ..+7]
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

    // ---- S^T of 32 keys (sub-tile `sub` of tile stage `stage`) against the 64 queries
    // per-lane byte offsets of the K operand reads (one per 16-wide d step)
    int kofs[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) kofs[st] = 2 * (lr * kD + (((2 * st + hb) ^ (lr & 15)) << 3));
    auto qk = [&](const uint16_t *kt, int sub, f32x16 (&s)[2]) __attribute__((always_inline)) {
        const WA_LDS char *kb = (const WA_LDS char *)kt + sub * 32 * kD * 2;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[qb][i] = 0.f;
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const bf16x8 ak = *(const WA_LDS bf16x8 *)(kb + kofs[st]);
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[0][st], s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[1][st], s[1], 0, 0, 0);
        }
    };

    // ---- running max of one sub-tile; rescale the output when it grew enough
    auto row_max = [&](f32x16 (&s)[2], int key0, bool masked) __attribute__((always_inline)) {
        if (masked) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = key0 + 8 * (i >> 2) + 4 * hb + (i & 3);
                if (key >= n_keys) {
                    s[0][i] = -INFINITY;
                    s[1][i] = -INFINITY;
                }
            }
        }
        float mt[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float x = s[qb][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) x = fmaxf(x, s[qb][i]);
            mt[qb] = xhalf_max(x);
        }
        const bool grow = mt[0] > m[0] + thr || mt[1] > m[1] + thr;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const float mn = fmaxf(m[qb], mt[qb]);
                const float corr = __builtin_amdgcn_exp2f((m[qb] - mn) * c);
                l[qb] *= corr;
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[b][qb][i] *= corr;
                m[qb] = mn;
            }
        }
    };

    // ---- P = exp2(S c - m c) as bf16 B operands; l accumulates the bf16 values
    auto softmax = [&](f32x16 (&s)[2], bf16x8 (&pb)[2][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float mc = m[qb] * c;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    pb[qb][jj][t] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[qb][8 * jj + t], c, -mc));
            float ls = l[qb];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int t = 0; t < 8; t += 2) {
                    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                    const bf16x2 pair = {pb[qb][jj][t], pb[qb][jj][t + 1]};
                    const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
                    ls = __builtin_amdgcn_fdot2_f32_bf16(pair, one, ls, false);
                }
            l[qb] = ls;
        }
    };

    // ---- O^T += V^T P^T for sub-tile `sub`.  V^T operand of dv block b, k-step
    // jj: lane group g = lane/16 supplies keys 4hb + u/4 (+16jj, +8 for the
    // upper half) and dims 32b + 16(g&1) + 4(u%4) .. +3 of the row-major tile;
    // the transpose read hands lane 16g+i dims 32b+16(g&1)+i over those keys.
    int vofs[4];
    {
        const int u = lane & 15, g = lane >> 4;
        const int r = 4 * hb + (u >> 2);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int cidx = 4 * b + 2 * (g & 1) + ((u & 3) >> 1);
            vofs[b] = r * (kD * 2) + ((cidx ^ (4 * (r & 3))) << 4) + 8 * (u & 1);
        }
    }
    auto pv = [&](const uint16_t *vtile, int sub, const bf16x8 (&pb)[2][2]) __attribute__((always_inline)) {
        const WA_LDS char *vt = (const WA_LDS char *)vtile + sub * 32 * kD * 2;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                i16x4 half[2];
#pragma unroll
                for (int th = 0; th < 2; ++th)
                    half[th] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (WA_LDS i16x4 *)(vt + (16 * jj + 8 * th) * kD * 2 + vofs[b]));
                bf16x8 av;
                __builtin_memcpy(&av, half, sizeof(av));
                o[b][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[0][jj], o[b][0], 0, 0, 0);
                o[b][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[1][jj], o[b][1], 0, 0, 0);
            }
        }
    };

    // ---- prologue: tiles 0 and 1 in flight, wait for tile 0
    issue_tile(0, kst<0>(), vst<0>());
    if (n_tiles > 1) {
        issue_tile(1, kst<1>(), vst<1>());
        wait_vm8();
    } else {
        wait_vm0();
    }
    __syncthreads();

    f32x16 sa[2], sb[2];
    bf16x8 pa[2][2], pbk[2][2];
    qk(kst<0>(), 0, sa);

    // One tile; stage S holds tile t, stage S+1 tile t+1, stage S+2 is refilled
    // with tile t+2.  Returns false after the last tile.
    auto tile = [&](int t, auto stage_tag) __attribute__((always_inline)) -> bool {
        constexpr int S = decltype(stage_tag)::value;
        constexpr int S1 = (S + 1) % kStages, S2 = (S + 2) % kStages;
        const bool last = t == n_tiles - 1;
        const bool mask = ragged && last;
        // sub-tile 0 softmax, overlapped with the sub-tile 1 products
        row_max(sa, t * kBN, mask);
        qk(kst<S>(), 1, sb);
        softmax(sa, pa);
        pv(vst<S>(), 0, pa);
        row_max(sb, t * kBN + 32, mask);
        if (!last) {
            // tile t+1 (the only load in flight) must be in LDS for every wave;
            // every wave is past its reads of tile t-1, whose stage is refilled
            wait_vm0();
            __syncthreads();
            if (t + 2 < n_tiles) issue_tile(t + 2, kst<S2>(), vst<S2>());
            qk(kst<S1>(), 0, sa);
        }
        softmax(sb, pbk);
        pv(vst<S>(), 1, pbk);
        return !last;
    };
    for (int t = 0;; t += 3) {
        if (!tile(t, StageTag<0>{})) break;
        if (!tile(t + 1, StageTag<1>{})) break;
        if (!tile(t + 2, StageTag<2>{})) break;
    }

    // ---- epilogue: O^T[dv][q] / l; lanes l and l^32 hold halves of l
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float lt = xhalf_sum(l[qb]);
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
                a.lse[(int64_t)h * a.n_q + row] = (m[qb] * c + __log2f(lt)) * 0.69314718055994531f;
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
