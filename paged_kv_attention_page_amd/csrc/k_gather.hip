// Gather the selected pages into one contiguous K/V buffer (WorldAttention
// review, "Core Idea", item 3, and the Tab. 9 share of time spent on KV
// reconstruction and contiguous copying, in "Strengths").
//
//   k_ctx[r * page_tokens + t] = k_pool[idx[r]][t]   (and V), r < k_p
//
// Pure HBM stream: each byte is read once and written once.  Grid: x = span
// of one page, y = rank r, z = tensor (K, V).  A block copies a contiguous
// 32 KB span of 16-byte vectors of page idx[r], four vectors in flight per thread,
// with non-temporal loads and stores (the data is not reused by this
// kernel).  idx is read on the device; a rank whose page id is outside
// [0, max_pages) is skipped.
#include "wa_internal.h"

namespace wa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

static constexpr int kGatherThreads = 256;
static constexpr int kGatherUnroll = 4;
// vectors per block: 32 KB, so a 38 MB page spreads over ~1,200 blocks (a
// sweep of 2-16 vectors in flight per thread and 16-256 KB per block measured
// this shape fastest, 6.1 TB/s against 5.2 TB/s at 128 KB per block)
static constexpr int64_t kGatherSpan = (int64_t)kGatherThreads * kGatherUnroll * 2;

__global__ __launch_bounds__(kGatherThreads) void k_gather(
    const u32x4 *__restrict__ k_pool, const u32x4 *__restrict__ v_pool,
    const int32_t *__restrict__ idx, int max_pages, int64_t page_vecs,
    u32x4 *__restrict__ k_ctx, u32x4 *__restrict__ v_ctx) {
    const int r = blockIdx.y;
    const int page = idx[r];
    if (page < 0 || page >= max_pages) return;
    const u32x4 *src = (blockIdx.z == 0 ? k_pool : v_pool) + (int64_t)page * page_vecs;
    u32x4 *dst = (blockIdx.z == 0 ? k_ctx : v_ctx) + (int64_t)r * page_vecs;
    const int64_t begin = (int64_t)blockIdx.x * kGatherSpan;
    const int64_t end = min(page_vecs, begin + kGatherSpan);
    constexpr int64_t step = (int64_t)kGatherThreads * kGatherUnroll;
    int64_t i = begin + threadIdx.x;
    for (; i + (kGatherUnroll - 1) * kGatherThreads < end; i += step) {
        u32x4 v[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u)
            v[u] = __builtin_nontemporal_load(src + i + u * kGatherThreads);
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u)
            __builtin_nontemporal_store(v[u], dst + i + u * kGatherThreads);
    }
    for (; i < end; i += kGatherThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

hipError_t launch_gather(const wa_layout &L, const void *k_pool, const void *v_pool,
                         const int32_t *idx, int32_t k_p, void *k_ctx, void *v_ctx,
                         hipStream_t s) {
    const int64_t page_bytes =
        (int64_t)L.page_tokens * L.n_heads * L.head_dim * elem_bytes(L.dtype);
    const int64_t page_vecs = page_bytes / 16;
    const int64_t bx = (page_vecs + kGatherSpan - 1) / kGatherSpan;
    const int tensors = v_pool ? 2 : 1;
    hipLaunchKernelGGL(k_gather, dim3((unsigned)bx, (unsigned)k_p, (unsigned)tensors),
                       dim3(kGatherThreads), 0, s, (const u32x4 *)k_pool, (const u32x4 *)v_pool,
                       idx, L.max_pages, page_vecs, (u32x4 *)k_ctx, (u32x4 *)v_ctx);
    return hipGetLastError();
}

}  // namespace wa
