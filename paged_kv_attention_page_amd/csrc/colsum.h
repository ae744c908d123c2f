// Column sums of a token-major [rows][hd] array, in fp64, with a fixed
// summation order.  Used for the page mean key (append) and the chunk mean
// query (select): WorldAttention review, "HKV: Page-Level Multi-Tier Memory",
// page stage.
//
// Work split: block b owns rows [b*rows_per_block, ...).  Thread t owns the
// 16-byte column vector c = t % chunks and the rows r == t / chunks (mod
// row_lanes) of the block's range, accumulating in registers (row order).
// The row_lanes partials of a column are then added in lane order through
// LDS, and one fp64 partial per (block, column) goes to the workspace.  A
// second kernel adds the block partials in a fixed order
// (reduce_partials_64).  The inputs are bf16
// or fp32 values, so in practice every fp64 sum here is exact; the fixed
// order makes repeated calls bitwise equal regardless.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wa {

// Streaming (non-temporal) 16-byte loads and stores: the rows are touched
// once here, and a copy measured 25 % faster with the non-temporal hint.
typedef unsigned cs_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load(const uint4 *p) {
    const cs_u32x4 v = __builtin_nontemporal_load((const cs_u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void stream_store(uint4 *p, uint4 v) {
    const cs_u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (cs_u32x4 *)p);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Add the elements of one 16-byte vector to acc[] (8 bf16 or 4 fp32 values).
template <bool BF16>
__device__ __forceinline__ void accumulate_vec(double *acc, uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (BF16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[2 * j] += (double)bf16lo(w[j]);
            acc[2 * j + 1] += (double)bf16hi(w[j]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += (double)__uint_as_float(w[j]);
    }
}

// One block's share of the column sums: vectors [c0, c0 + group_chunks) of
// the rows [r0, r1), optionally copying the rows of up to two arrays (K and V
// of a page) to their destinations on the way.
//   x      [rows][chunks] 16-byte vectors, summed (and copied to x_dst if set)
//   y      [rows][chunks] vectors copied to y_dst (not summed), or null
//   lds    row_lanes * group_chunks * VEC doubles of shared memory
//   part   this row block's partial row ([hd] doubles); the block writes the
//          columns of its group.  part_col0: the column part[0] stands for (0
//          for a whole row; the group's first column when part holds only the
//          group's columns, e.g. in shared memory)
// Thread t owns vector c0 + t % group_chunks and rows r0 + t / group_chunks,
// stepping by row_lanes, and accumulates in row order; the row_lanes partials
// of a column are then added in lane order.  BATCH rows of each thread are
// in flight together.
template <bool BF16, int BATCH = 4>
__device__ __forceinline__ void colsum_block(const uint4 *__restrict__ x, uint4 *__restrict__ x_dst,
                                             const uint4 *__restrict__ y, uint4 *__restrict__ y_dst,
                                             int64_t rows, int chunks, int c0, int group_chunks,
                                             int row_lanes, int rows_per_block, int row_block,
                                             double *lds, double *__restrict__ part,
                                             int part_col0 = 0) {
    constexpr int VEC = BF16 ? 8 : 4;
    const int t = threadIdx.x;
    const int gw = min(group_chunks, chunks - c0) * VEC;   // columns in this group
    const int64_t r0 = (int64_t)row_block * rows_per_block;
    const int64_t r1 = min(rows, r0 + rows_per_block);
    double acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0;

    const int cl = t % group_chunks;
    const int lane = t / group_chunks;
    if (lane < row_lanes && c0 + cl < chunks) {
        const int c = c0 + cl;
        int64_t r = r0 + lane;
        for (; r + (BATCH - 1) * row_lanes < r1; r += BATCH * row_lanes) {
            uint4 xv[BATCH], yv[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) xv[u] = stream_load(x + (r + u * row_lanes) * chunks + c);
            if (y) {
#pragma unroll
                for (int u = 0; u < BATCH; ++u)
                    yv[u] = stream_load(y + (r + u * row_lanes) * chunks + c);
            }
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                if (x_dst) stream_store(x_dst + (r + u * row_lanes) * chunks + c, xv[u]);
                if (y) stream_store(y_dst + (r + u * row_lanes) * chunks + c, yv[u]);
                accumulate_vec<BF16>(acc, xv[u]);
            }
        }
        for (; r < r1; r += row_lanes) {
            const uint4 xv = stream_load(x + r * chunks + c);
            if (x_dst) stream_store(x_dst + r * chunks + c, xv);
            if (y) stream_store(y_dst + r * chunks + c, stream_load(y + r * chunks + c));
            accumulate_vec<BF16>(acc, xv);
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) lds[lane * gw + cl * VEC + e] = acc[e];
    }
    __syncthreads();
    for (int col = t; col < gw; col += blockDim.x) {
        double s = 0.0;
        for (int ln = 0; ln < row_lanes; ++ln) s += lds[ln * gw + col];
        part[c0 * VEC - part_col0 + col] = s;
    }
}

// Sum the block partials partial[b][col] (b < blocks, row stride hd) for the
// 64 columns c0 ... c0+63, with a block of 1024 threads: lane r = t/64 adds
// blocks r, r+16, r+32, ... in that order, then the 16 lane sums are added in
// lane order.  The order is fixed, so results are bitwise reproducible.
// `lds` holds 16 * 64 doubles.  Returns the column sum in threads t < 64.
__device__ __forceinline__ double reduce_partials_64(const double *__restrict__ partial, int blocks,
                                                     int hd, int c0, double *lds) {
    const int c = threadIdx.x & 63, r = threadIdx.x >> 6;
    const int col = c0 + c;
    double s = 0.0;
    if (col < hd) {
        const double *p = partial + col;
        int b = r;
        for (; b + 48 < blocks; b += 64) {
            const double v0 = p[(int64_t)b * hd], v1 = p[(int64_t)(b + 16) * hd];
            const double v2 = p[(int64_t)(b + 32) * hd], v3 = p[(int64_t)(b + 48) * hd];
            s += v0;
            s += v1;
            s += v2;
            s += v3;
        }
        for (; b < blocks; b += 16) s += p[(int64_t)b * hd];
    }
    lds[r * 64 + c] = s;
    __syncthreads();
    double tot = 0.0;
    if (r == 0)
        for (int k = 0; k < 16; ++k) tot += lds[k * 64 + c];
    return tot;
}

}  // namespace wa
