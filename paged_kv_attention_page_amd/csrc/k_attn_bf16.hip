// bf16 block attention on the CDNA4 matrix cores (Inferix summary, section
// 3.4, Step 3: the block's queries attend over [cached K ++ own K],
// [cached V ++ own V], one softmax, no mask; the einsum post on
// nakranivaibhav.github.io, "Where the mental model stops": Q K^T and P V are
// the only contractions, softmax sits between them).
//
// Design (gfx950, head_dim 128):
//  * Block = 8 wavefronts x 32 queries = 256 queries of one head, two
//    wavefronts per SIMD: one wavefront's matrix-core work overlaps the
//    other's softmax (a single wavefront issues a vector instruction only
//    every ~8 cycles, too slow to hide the exponentials behind its own
//    products).  Blocks are renumbered so that consecutive (head, query-block)
//    tiles land on the same XCD: the blocks of one head then stream the same
//    K/V through one L2.
//  * K/V tiles of 64 keys go from global memory straight into LDS with
//    global_load_lds_dwordx4 (no register staging), in a ring of kStages
//    tiles; the loads of tile t+kStages-1 are in flight while tile t is
//    computed.  Both tiles are row-major [key][d] with XOR-swizzled 16-byte
//    chunks; the swizzle is applied on the global side of the copy.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (fp32 accumulation) on 32-key
//    sub-tiles: a lane then holds 16 keys of ONE query, so a query's running
//    max / sum live in one lane pair (one permlane32 swap) and rescaling the
//    output is a per-lane multiply.
//  * O^T += V^T P^T: P comes straight from the S^T accumulator layout
//    (p = exp2(S * c - m) with c = scale * log2(e), one fused multiply-add
//    per score on the exact bf16 products, rounded to bf16); V^T operands
//    are read
//    with ds_read_b64_tr_b16, whose 16-lane 4x16 -> 16x4 transpose turns the
//    row-major V tile into the key-contiguous operand, in the key order that
//    matches P.
//  * Software pipeline per wave: the Q K^T products of the next sub-tile are
//    interleaved with the exponentials of the current one, and the P V
//    products with the operand reads of the next region, so matrix-core and
//    vector work overlap (the instruction order inside a region is left to the
//    compiler: with two wavefronts per SIMD, the other wavefront fills the
//    gaps); all operands and accumulators live in VGPRs.
//  * Lazy rescaling without a running maximum: probabilities are taken against
//    a reference max that moves only when a row's probabilities of one
//    sub-tile sum past 2^8; then O and l are rescaled and that sub-tile is
//    recomputed (exact either way: the final division uses the same reference).
#include <math.h>

#include "wa_internal.h"

namespace wa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define WA_LDS __attribute__((address_space(3)))

static constexpr int kD = 128;            // head dim
static constexpr int kWaves = 8;          // wavefronts per block
static constexpr int kWQ = 32;            // queries per wavefront
static constexpr int kBM = kWaves * kWQ;  // queries per block
static constexpr int kBN = 64;            // keys per tile
static constexpr int kThreads = 64 * kWaves;
static constexpr int kStages = 4;         // LDS ring depth (tiles)
static constexpr int kTileElems = kBN * kD;
static constexpr int kRowsPerWave = kBN / kWaves;   // tile rows each wavefront copies
static constexpr int kCopies = kRowsPerWave / 4;    // 1 KB copies per tensor per wavefront
// The matrix cores multiply the exact bf16 queries and keys (fp32
// accumulation, each chain of score products starts from zero), and the
// softmax runs in base-2 units: p = 2^(s c - m) with c = softmax_scale *
// log2(e), the scaling fused into one multiply-add per score before the
// exponential, so the only roundings of a score are those of the fp32
// accumulation and of that multiply-add.  (Scaling the queries by c in bf16
// before the products saves the multiply-add but rounds every q * c to 8
// bits, which moves the log-sum-exp by up to 2^-8 scale sum_d |q_d k_d|.)
// The probabilities of a sub-tile are taken against a reference max m (base-2
// units: c times the row max of the segment's first sub-tile) that only moves
// when a row's new probabilities sum past 2^8 (some score more than 8 above
// m, or an overflow): O and l are then rescaled and the sub-tile's
// probabilities recomputed.  The result is exact either way, since O and l
// always share the reference max, and no per-sub-tile maximum is needed.
static constexpr float kSumLimit = 256.f;
// LDS operands are read this many matrix products ahead of their use (of the
// 8 per region); 6 fits 256 registers without spills in every mode.
static constexpr int kPrefetch = 6;
// Debug build (WA_DEBUG_POISON): the whole K/V ring is filled with NaN when
// a block starts, and every stage is filled with NaN again by the
// wavefronts that refill it, after the barrier that ends its last reads and
// before its copies are issued.  A read of a stage whose tile has not landed
// (a missing wait), of a stage nothing was copied into, or of a stage's
// previous tile then carries NaN into the products; results that stay finite
// and equal to the regular build's show that no such value reaches an output.
#ifdef WA_DEBUG_POISON
static constexpr bool kPoison = true;
#else
static constexpr bool kPoison = false;
#endif
static constexpr int kMaxSplitBlocks = 256;  // blocks of a split launch (partial slots)
static constexpr int kMinSplitTiles = 16;    // fewest tiles per block worth a split
static constexpr int kMaxBlocksPerItem = 32; // split blocks per (query block, head) item
static constexpr int kMaxSlots = 64;         // pieces of one item a split may leave

// Workgroups are dispatched to the 8 XCDs round robin (block b on XCD b % 8),
// so XCD x runs n / 8 blocks, one more when x < n % 8.  Logical block
// numbers are handed out in contiguous ranges per XCD, the XCDs taken in an
// order that alternates those with one block more and those without: with
// 228 items of 19 query blocks per head, every second range boundary then
// falls on a head boundary, and only 4 of the 12 heads have their K/V read
// through two L2s (7 with the XCDs in plain order).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    const int q = n >> 3, r = n & 7;
    const int x = bid & 7, i = bid >> 3;
    const int m = r < 8 - r ? r : 8 - r;
    int start = 0;
    for (int k = 0; k < 8; ++k) {
        const int xk = k < 2 * m ? ((k & 1) ? r + (k >> 1) : (k >> 1))
                                 : (r > 8 - r ? k - m : r + k - m);
        if (xk == x) break;
        start += q + (xk < r ? 1 : 0);
    }
    return start + i;
}

struct AttnArgs {
    const uint16_t *q;
    const uint16_t *k_ctx;
    const uint16_t *v_ctx;
    const uint16_t *k_own;
    const uint16_t *v_own;
    int n_q, n_ctx, n_own, n_heads, q_blocks;
    int n_tiles;        // 64-key tiles per item (T)
    int split;          // 1: blocks take equal runs of the items' tiles
    int grid;           // blocks of the attention launch (G)
    int items;          // q_blocks * n_heads
    int head_tiles;     // split: tiles [0, S) of each item form the first phase
    int slots;          // split: partial slots per item
    int64_t total;      // items * n_tiles
    float c;            // softmax_scale * log2(e)
    int out_bf16;
    void *out;
    float *lse;
    float *part_o;      // [items][slots][kBM][kD] unnormalised partial outputs
    float *part_ml;     // [items][slots][kBM][2] reference max (base-2 units), row sum
    // paged context (idx != null): k_ctx / v_ctx are the pools, context key n
    // is token n % page_tokens of pool page idx[n / page_tokens]
    const int32_t *idx;
    int page_tokens;
    int max_pages;
    int tpp;            // 64-key tiles per page when page_tokens % 64 == 0, else 0
    uint64_t page_bytes;   // pool page stride in bytes
    // sparse branch (MODE 3): item i attends over the ascending 64-key tiles
    // sp_tiles[i * n_tiles + 0 .. sp_count[i]) of [ctx ++ own]; sp_plan and
    // sp_prefix are written by k_sparse_plan (see there)
    const int32_t *sp_tiles;
    const int32_t *sp_count;
    const int32_t *sp_plan;     // [split, blocks taking runs, total positions]
    const int32_t *sp_prefix;   // [items + 1] exclusive prefix of the (clamped) counts
};

// Work order of a split launch.  Position g in [0, items * T) names one 64-key
// tile of one item: first tiles [0, S) of every item, item after item (phase
// 0), then tiles [S, T) of every item (phase 1); block w takes positions
// [w total / G, (w+1) total / G).  With S = total / G, block b < items spends
// almost all its run on the first S tiles of item b, so the blocks of one head
// stream the same K/V tiles at about the same time (one L2 per XCD serves
// them), and the remaining blocks share out the tails.  Every piece of an
// item that one block computes is one partial slot of that item.
struct SplitMap {
    int64_t total;
    int grid, items, T, S;
    __device__ explicit SplitMap(const AttnArgs &a)
        : total(a.total), grid(a.grid), items(a.items), T(a.n_tiles), S(a.head_tiles) {}
    __device__ int64_t bnd(int w) const { return (int64_t)w * total / grid; }
    // the block whose run holds position x (the last one, past empty runs)
    __device__ int block_of(int64_t x) const { return (int)(((x + 1) * grid - 1) / total); }
    __device__ int64_t part_begin(int i, int p) const {
        return p == 0 ? (int64_t)i * S : (int64_t)items * S + (int64_t)i * (T - S);
    }
    __device__ int64_t part_end(int i, int p) const { return part_begin(i, p) + (p == 0 ? S : T - S); }
    // partial slot of the piece of part p of item i computed by block w
    __device__ int slot(int i, int p, int w) const {
        int base = 0;
        if (p == 1 && S > 0) base = block_of(part_end(i, 0) - 1) - block_of(part_begin(i, 0)) + 1;
        return base + (w - block_of(part_begin(i, p)));
    }
};

// One 16-byte-per-lane DMA from global memory into LDS: lane i's 16 bytes
// land at lds_base + OFF + 16 i, where lds_base is a wave-uniform SGPR and OFF
// a compile-time offset (m0 is set with one scalar add).  Issued through
// inline assembly so that the compiler does not insert its own (conservative)
// waits for the copy before unrelated LDS reads; the kernel waits for the
// copies itself (vmcnt) before the barrier that publishes a tile.  Nothing
// else in the kernel uses m0.  The scalar add writes SCC, so SCC is declared
// clobbered: the compiler must not keep a carry live across the copy.
template <unsigned OFF>
__device__ __forceinline__ void dma16(const void *gptr, unsigned lds_base) {
    asm volatile("s_add_u32 m0, %0, %2\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(gptr), "i"(OFF)
                 : "memory", "m0", "scc");
}
// The same copy with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset: the per-lane offsets of a tile never change, so issuing a tile
// costs no vector instructions beyond the copies themselves.
template <unsigned OFF>
__device__ __forceinline__ void dma16_sbase(const void *sbase, unsigned voff, unsigned lds_base) {
    asm volatile("s_add_u32 m0, %0, %3\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_base), "v"(voff), "s"(sbase), "i"(OFF)
                 : "memory", "m0", "scc");
}
// A wave-uniform pointer kept in SGPRs: the empty asm makes the value opaque,
// so the compiler cannot re-load it from the kernel arguments (with a wait on
// every outstanding LDS read) each time it is used.
template <typename T>
__device__ __forceinline__ T *sgpr_ptr(T *p) {
    uint64_t x = (uint64_t)(uintptr_t)p;
    asm volatile("" : "+s"(x));
    return (T *)(uintptr_t)x;
}
// A pointer that is the same in every lane, declared so (it derives from the
// block index only, which the compiler cannot always see through loops).
// readfirstlane returns a signed int: each half goes through unsigned before
// it is widened, or a low half with bit 31 set would fill the high half.
template <typename T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
    const uint64_t x = (uint64_t)(uintptr_t)p;
    const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)x);
    const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(x >> 32));
    return (T *)(uintptr_t)(lo | (hi << 32));
}
__device__ __forceinline__ void wait_vm4() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); }
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

// The K/V ring in one LDS array: the kStages K tiles, then the kStages V
// tiles.  Every access names its stage at compile time, so each address is a
// per-lane (or wave-uniform) base plus a constant.
static constexpr unsigned kTileBytes = kTileElems * 2;
static constexpr int kStageBytes = kTileElems * 2;   // one K or V tile
static constexpr int kSubBytes = 32 * kD * 2;        // one 32-key sub-tile
__shared__ __attribute__((aligned(1024))) uint16_t lds_ring[2 * kStages * kTileElems];
// MODE 3: this block's tile list (only that kernel references it, so only it
// allocates the 16 KB)
__shared__ int sp_list[WA_MAX_SPARSE_TILES];
static_assert(WA_HSA_Q_BLOCK == kBM, "one pooled query block per attention block");

template <int S>
struct StageTag {
    static constexpr int value = S;
};

template <int S>
__device__ __forceinline__ uint16_t *kst() {
    static_assert(S >= 0 && S < kStages, "stage");
    return lds_ring + S * kTileElems;
}
template <int S>
__device__ __forceinline__ uint16_t *vst() {
    static_assert(S >= 0 && S < kStages, "stage");
    return lds_ring + (kStages + S) * kTileElems;
}

// Where the context keys come from (see AttnArgs): MODE 0, one contiguous
// buffer; MODE 1, pool pages through a.idx, page_tokens a multiple of 64
// (whole tiles per page: the copies take the same fast path as a contiguous
// buffer); MODE 2, pool pages, other page sizes (context tiles copied row by
// row); MODE 3, contiguous buffers and a list of tiles per item (the sparse
// branch): the loop runs over list positions, and each copy looks its tile
// up in the list.
template <int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_attn_bf16(AttnArgs a) {

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, lr = lane & 31, hb = lane >> 5;
    // consecutive logical blocks run on one XCD (one L2): with the split, they
    // take consecutive runs of the same head's work
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    if constexpr (kPoison) {
        // the whole ring holds NaN before anything is copied into it
        for (int i = tid; i < 2 * kStages * kTileElems; i += kThreads) lds_ring[i] = 0x7fc0;
        __syncthreads();
    }
    const int64_t hd = (int64_t)a.n_heads * kD;
    const int n_keys = a.n_ctx + a.n_own;
    const int n_tiles = a.n_tiles;
    const bool ragged = (n_keys % kBN) != 0;
    const float c = a.c;
    constexpr int kPf = kPrefetch;

    // ---- tile loads: wavefront w copies rows 8w ... 8w+7 of the K and V
    // tiles, 4 rows (1 KB) per instruction; lane -> (row 8w+4i+lane/16, slot lane%16)
    const int ld_row0 = kRowsPerWave * wave + (lane >> 4);
    const int ld_slot = lane & 15;
    const unsigned ld_base =
        __builtin_amdgcn_readfirstlane(lds_addr(lds_ring) + kRowsPerWave * wave * kD * 2);
    const uint16_t *const k_ctx = sgpr_ptr(a.k_ctx), *const v_ctx = sgpr_ptr(a.v_ctx);
    const uint16_t *const k_own = sgpr_ptr(a.k_own), *const v_own = sgpr_ptr(a.v_own);
    // DMA sources: tile t holds keys [64t, 64t + 64).  It lies inside one
    // segment unless it straddles n_ctx (t == t_mid) or passes the end
    // (t >= t_full); inside one, its first row is base + t * tile_bytes, where
    // the own segment's base is shifted back by the n_ctx keys before it.
    const int t_ctx = a.n_ctx / kBN;
    const int t_mid = (a.n_ctx % kBN) != 0 ? t_ctx : -1;
    const int t_full = n_keys / kBN;
    const uint32_t tile_bytes = (uint32_t)(kBN * hd * 2);
    const uint64_t ctx_shift = (uint64_t)a.n_ctx * (uint64_t)hd * 2u;
    const uint64_t kb_ctx = (uint64_t)(uintptr_t)k_ctx, vb_ctx = (uint64_t)(uintptr_t)v_ctx;
    const uint64_t kb_own = (uint64_t)(uintptr_t)k_own - ctx_shift;
    const uint64_t vb_own = (uint64_t)(uintptr_t)v_own - ctx_shift;

    // ---- per-lane LDS byte addresses of the operand reads in stage 0; other
    // stages and sub-tiles add a constant that fits the 16-bit offset of the
    // read (the V stages lie above 64 KB, so their base is in the register)
    // K (A operand of S^T = K Q^T): row lr of the 32-key sub-tile, d chunk 2st+hb
    int kofs[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        kofs[st] = (int)lds_addr(kst<0>()) + 2 * (lr * kD + (((2 * st + hb) ^ (lr & 15)) << 3));
        asm volatile("" : "+v"(kofs[st]));
    }
    // V^T (A operand of O^T += V^T P^T) for dv block b: lane group g = lane/16
    // supplies keys 4hb + u/4 (+16jj, +8 for the upper half of the 16 keys) and
    // dims 32b + 16(g&1) + 4(u%4) .. +3 of the row-major tile; the transpose
    // read hands lane 16g+i dim 32b+16(g&1)+i over those keys, in the key order
    // of the S^T accumulator (keys 8(i/4) + 4hb + i%4 of each 16-key step).
    int vofs[4];
    {
        const int u = lane & 15, g = lane >> 4;
        const int r = 4 * hb + (u >> 2);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int cidx = 4 * b + 2 * (g & 1) + ((u & 3) >> 1);
            vofs[b] = (int)lds_addr(vst<0>()) + r * (kD * 2) + ((cidx ^ (4 * (r & 3))) << 4) + 8 * (u & 1);
            asm volatile("" : "+v"(vofs[b]));
        }
    }
    // `off` = ring byte offset of a (stage, sub-tile) within the K or the V
    // tiles, kStageBytes * stage + kSubBytes * sub: a compile-time constant in
    // every call, so it lands in the 16-bit offset of the read
    auto read_k = [&](int off, int st) __attribute__((always_inline)) -> bf16x8 {
        return *(const WA_LDS bf16x8 *)((const WA_LDS char *)(uintptr_t)(unsigned)kofs[st] + off);
    };
    // V^T operand `op` = 4 jj + b of the sub-tile at `off`
    auto read_v = [&](int off, int op) __attribute__((always_inline)) -> bf16x8 {
        const int jj = op >> 2, b = op & 3;
        const WA_LDS char *base =
            (const WA_LDS char *)(uintptr_t)(unsigned)vofs[b] + off + 16 * jj * kD * 2;
        i16x4 half[2];
        half[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((WA_LDS i16x4 *)base);
        half[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((WA_LDS i16x4 *)(base + 8 * kD * 2));
        bf16x8 av;
        __builtin_memcpy(&av, half, sizeof(av));
        return av;
    };

    // MODE 3: the tile at list position `pos` (the list is in LDS, the same
    // for every lane)
    auto sp_tile = [&](int pos) __attribute__((always_inline)) -> int {
        return __builtin_amdgcn_readfirstlane(sp_list[pos]);
    };

  // One segment: tiles [t_begin, t_end) of item `item` (query block
  // item % q_blocks of head item / q_blocks).  Without the split a segment is
  // a whole item, normalised and written out; with it, a piece leaves its
  // unnormalised output, reference max and row sum in partial slot `slot` of
  // the item.
  auto segment = [&](int item, int t_begin, int t_end, int slot) __attribute__((always_inline)) {
    const int h = item / a.q_blocks;
    const int q0 = (item % a.q_blocks) * kBM + wave * kWQ;
    // per-lane byte offsets of this lane's 16 bytes within a tile whose first
    // row is at a uniform base (fast path: the tile lies inside one segment)
    unsigned koff[kCopies], voff[kCopies];
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
        const int row = ld_row0 + 4 * i;
        const unsigned rowb = (unsigned)(row * hd + h * kD) * 2u;
        koff[i] = rowb + 16u * (unsigned)(ld_slot ^ (row & 15));
        voff[i] = rowb + 16u * (unsigned)(ld_slot ^ (4 * (row & 3)));
    }
    // paged context with whole tiles per page (page_tokens % 64 == 0): the
    // page of the context tile the copies reach next.  Its base is shifted
    // back by the tiles of the pages before it, so that tile t's first row
    // is at base + t * tile_bytes as in a contiguous buffer.  Tiles are
    // issued in increasing order, so the page only moves forward, one page at
    // a time, with one scalar load of its id.  An id outside the pool is
    // clamped into it (memory safety only: the caller passes valid ids).
    int pg = 0, pg_next = 0x7fffffff;   // pg_next: first tile of the next page
    uint64_t kb_pg = kb_ctx, vb_pg = vb_ctx;
    auto set_page = [&](int r) __attribute__((always_inline)) {
        asm volatile("; set page" ::: "memory");
        int id = __builtin_amdgcn_readfirstlane(a.idx[r]);
        id = id < 0 ? 0 : (id >= a.max_pages ? a.max_pages - 1 : id);
        pg = r;
        pg_next = (r + 1) * a.tpp < t_ctx ? (r + 1) * a.tpp : 0x7fffffff;
        const uint64_t back = (uint64_t)(uint32_t)(r * a.tpp) * tile_bytes;
        kb_pg = kb_ctx + (uint64_t)(uint32_t)id * a.page_bytes - back;
        vb_pg = vb_ctx + (uint64_t)(uint32_t)id * a.page_bytes - back;
    };
    if (MODE == 1 && t_begin < t_ctx) set_page(t_begin / a.tpp);

    static_assert(kCopies == 2, "issue_tile writes two 1 KB copies per tensor");
    auto issue_tile = [&](int pos, auto stage_tag) __attribute__((always_inline)) {
        constexpr unsigned S = decltype(stage_tag)::value;
        const int t = MODE == 3 ? sp_tile(pos) : pos;
        constexpr unsigned OK = S * kTileBytes, OV = (kStages + S) * kTileBytes;
        if constexpr (kPoison) {
            // NaN over this wavefront's 8 rows (2 KB) of the K and V stage,
            // written and waited for before the copies that refill them
            typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 nan4 = {0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
            WA_LDS char *kr = (WA_LDS char *)(uintptr_t)(ld_base + OK) + 32 * lane;
            WA_LDS char *vr = (WA_LDS char *)(uintptr_t)(ld_base + OV) + 32 * lane;
            *(WA_LDS u32x4 *)kr = nan4;
            *(WA_LDS u32x4 *)(kr + 16) = nan4;
            *(WA_LDS u32x4 *)vr = nan4;
            *(WA_LDS u32x4 *)(vr + 16) = nan4;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        constexpr unsigned ROWS4 = 4 * kD * 2;    // four tile rows
        const int key0 = t * kBN;
        if (t != t_mid && t < t_full && (MODE != 2 || t >= t_ctx)) {
            const uint64_t off = (uint64_t)(uint32_t)t * tile_bytes;
            const bool in_ctx = t < t_ctx;
            if (MODE == 1 && t >= pg_next) set_page(pg + 1);
            const uint16_t *kb = uniform_ptr((const uint16_t *)(uintptr_t)((in_ctx ? kb_pg : kb_own) + off));
            const uint16_t *vb = uniform_ptr((const uint16_t *)(uintptr_t)((in_ctx ? vb_pg : vb_own) + off));
            dma16_sbase<OK>(kb, koff[0], ld_base);
            dma16_sbase<OV>(vb, voff[0], ld_base);
            dma16_sbase<OK + ROWS4>(kb, koff[1], ld_base);
            dma16_sbase<OV + ROWS4>(vb, voff[1], ld_base);
            return;
        }
        // tile across the ctx/own boundary or past the end: per-lane rows
        asm volatile("; dma slow path" ::: "memory");
        const uint16_t *kr[kCopies], *vr[kCopies];
#pragma unroll
        for (int i = 0; i < kCopies; ++i) {
            const int row = ld_row0 + 4 * i;
            int n = key0 + row;
            n = n < n_keys ? n : n_keys - 1;           // rows past the end repeat the last key
            const bool in_ctx = n < a.n_ctx;
            int64_t row_at = in_ctx ? n : n - a.n_ctx;   // row in its buffer
            if (MODE == 2 && in_ctx) {
                const int r = n / a.page_tokens;
                int id = a.idx[r];
                id = id < 0 ? 0 : (id >= a.max_pages ? a.max_pages - 1 : id);
                row_at = (int64_t)id * a.page_tokens + (n - r * a.page_tokens);
            }
            const int64_t off = row_at * hd + h * kD;
            kr[i] = (in_ctx ? k_ctx : k_own) + off + 8 * (ld_slot ^ (row & 15));
            vr[i] = (in_ctx ? v_ctx : v_own) + off + 8 * (ld_slot ^ (4 * (row & 3)));
        }
        asm volatile("; dma slow path copies" ::: "memory");
        dma16<OK>(kr[0], ld_base);
        dma16<OV>(vr[0], ld_base);
        dma16<OK + ROWS4>(kr[1], ld_base);
        dma16<OV + ROWS4>(vr[1], ld_base);
    };

    // ---- this wavefront's 32 queries as B operands, as given:
    // qf[st] = Q[q0+lr][16st+8hb ..+7]
    bf16x8 qf[8];
    {
        const int row = q0 + lr;
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            if (row < a.n_q)
                qf[st] = *(const bf16x8 *)(a.q + (int64_t)row * hd + h * kD + 16 * st + 8 * hb);
            else
                qf[st] = (bf16x8)(__bf16)0.f;
        }
    }

    f32x16 o[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[b][i] = 0.f;
    float m = 0.f, l = 0.f;   // reference max (base-2 units), row sum
    const f32x16 zero16 = {};  // start of each score chain (an inline constant)

    // ---- keys past the end (last tile only) get score -inf.  Their rows were
    // loaded as copies of the last key, so maxima taken before masking are
    // still maxima over real keys; masking only has to precede the exponentials.
    auto mask_tail = [&](f32x16 &s, int key0) __attribute__((always_inline)) {
        // element i holds key key0 + 8(i/4) + 4hb + i%4; the limit is made
        // opaque so that the compares stay here instead of being hoisted out
        // of the loop into 32 live scalar registers
        int lim = n_keys - key0 - 4 * hb;
        asm volatile("; mask tail" : "+v"(lim));
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (8 * (i >> 2) + (i & 3) >= lim) s[i] = -INFINITY;
    };
    // ---- region QK+SOFTMAX: sn = K Q^T of the sub-tile at koff (8 MFMAs)
    // interleaved with the exponentials of sc (2 elements per MFMA), P packed to
    // bf16 for the P V products, l accumulated from the bf16 values; then the
    // lazy-rescale test (see kSumLimit).  Operands are read kPf products
    // ahead: ak[0 .. kPf) arrive prefetched, and the first kPf V^T
    // operands of the following P V region (at voff) are read during the last
    // products of this one.
    auto qk_softmax = [&](int koff, f32x16 &sn, const f32x16 &sc, bf16x8 (&pb)[2],
                          bf16x8 (&ak)[8], int voff, bf16x8 (&av)[8]) __attribute__((always_inline)) {
        float ls0 = 0.f, ls1 = 0.f;
        const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[st], qf[st], st == 0 ? zero16 : sn, 0, 0, 0);
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * st], c, -m));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * st + 1], c, -m));
            const bf16x2 pr = {(__bf16)p0, (__bf16)p1};
            pb[st >> 2][2 * (st & 3)] = pr[0];
            pb[st >> 2][2 * (st & 3) + 1] = pr[1];
            if (st & 1) ls1 = __builtin_amdgcn_fdot2_f32_bf16(pr, one, ls1, false);
            else ls0 = __builtin_amdgcn_fdot2_f32_bf16(pr, one, ls0, false);
            if (st + kPf < 8) ak[st + kPf] = read_k(koff, st + kPf);
            if (st >= 8 - kPf) av[st - (8 - kPf)] = read_v(voff, st - (8 - kPf));
        }
        float lsub = ls0 + ls1;
        if (__builtin_amdgcn_ballot_w64(lsub > kSumLimit) != 0) {
            asm volatile("; rescale" ::: "memory");
            float x = fmaxf(sc[0], sc[1]);
#pragma unroll
            for (int i = 1; i < 8; ++i) x = fmaxf(x, fmaxf(sc[2 * i], sc[2 * i + 1]));
            // the new reference max is m + dm (x: the sub-tile's row max, in
            // natural units)
            const float dm = fmaxf(xhalf_max(x) * c - m, 0.f);
            const float corr = __builtin_amdgcn_exp2f(-dm);
            l *= corr;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[b][i] *= corr;
            m += dm;
            lsub = 0.f;
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * st], c, -m));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * st + 1], c, -m));
                const bf16x2 pr = {(__bf16)p0, (__bf16)p1};
                pb[st >> 2][2 * (st & 3)] = pr[0];
                pb[st >> 2][2 * (st & 3) + 1] = pr[1];
                lsub = __builtin_amdgcn_fdot2_f32_bf16(pr, one, lsub, false);
            }
        }
        l += lsub;
    };

    // ---- region PV: O^T += V^T P^T (8 MFMAs); reads the V^T operands
    // kPf products ahead and, during its last products, the first
    // kPf K operands of the next QK+SOFTMAX region.
    auto pv = [&](int voff, const bf16x8 (&pb)[2], bf16x8 (&av)[8], int koff_next,
                  bf16x8 (&ak)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int op = 0; op < 8; ++op) {
            const int jj = op >> 2, b = op & 3;
            o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[op], pb[jj], o[b], 0, 0, 0);
            if (op + kPf < 8) av[op + kPf] = read_v(voff, op + kPf);
            if (op >= 8 - kPf) ak[op - (8 - kPf)] = read_k(koff_next, op - (8 - kPf));
        }
    };

    // ---- prologue: every wave is past its reads of the previous segment's
    // tiles; tiles t_begin .. t_begin+2 in flight, wait for t_begin.  Every
    // issue names a tile: near the end of the segment, the last tile again
    // (into a stage nobody reads), so that each tile issues the same number
    // of copies and one fixed vmcnt wait fits every tile.
    static_assert(2 * kCopies == 4, "the waits below count 4 copies per tile");
    __syncthreads();
    const int t_last = t_end - 1;
    // the position of the tile whose second half is masked (the last tile,
    // keys [mask_key0, n_keys)), and the one before it (whose successor's
    // first half is masked); -2 when the keys fill every tile or the list
    // leaves the last tile out
    int mask_tile = ragged ? n_tiles - 1 : -2;
    if (MODE == 3) mask_tile = ragged && sp_tile(t_last) == n_tiles - 1 ? t_last : -2;
    const int mask_tile_prev = mask_tile >= 0 ? mask_tile - 1 : -2;
    const int mask_key0 = (n_tiles - 1) * kBN;
    issue_tile(t_begin, StageTag<0>{});
    issue_tile(min(t_begin + 1, t_last), StageTag<1>{});
    issue_tile(min(t_begin + 2, t_last), StageTag<2>{});
    wait_vm8();
    __syncthreads();

    f32x16 sa, sb;
    bf16x8 pa[2], pbk[2];
    bf16x8 ak[8], av[8];
    {
        // S of the segment's first sub-tile
#pragma unroll
        for (int st = 0; st < 8; ++st) ak[st] = read_k(0, st);
        const f32x16 zero = {};
#pragma unroll
        for (int st = 0; st < 8; ++st)
            sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[st], qf[st], st == 0 ? zero : sa, 0, 0, 0);
        if (t_begin == mask_tile) mask_tail(sa, mask_key0);
        // its row max (times c) is the first reference max (a masked
        // sub-tile still holds at least one real key: the last tile's first
        // key)
        float x = fmaxf(sa[0], sa[1]);
#pragma unroll
        for (int i = 1; i < 8; ++i) x = fmaxf(x, fmaxf(sa[2 * i], sa[2 * i + 1]));
        m = xhalf_max(x) * c;
#pragma unroll
        for (int st = 0; st < kPf; ++st) ak[st] = read_k(kSubBytes, st);
    }

    // Tile t in stage S; on entry sa = S(t, 0) - m, and the first kPf K
    // operands of S(t, 1) prefetched.  Stages S+1
    // and S+2 hold (or are receiving) tiles t+1 and t+2; stage S+3 is refilled
    // with tile min(t+3, last).  On exit sa = S(t+1, 0), likewise.  The last
    // tile runs the same code: its products of the (nonexistent) next tile
    // read a stale stage and are discarded, which keeps every fused region one
    // basic block.
    auto tile = [&](int t, auto stage_tag) __attribute__((always_inline)) -> bool {
        constexpr int S = decltype(stage_tag)::value;
        constexpr int S1 = (S + 1) % kStages, S3 = (S + 3) % kStages;
        const bool last = t == t_end - 1;
        constexpr int KS = S * kStageBytes, KS1 = S1 * kStageBytes;
        qk_softmax(KS + kSubBytes, sb, sa, pa, ak, KS, av);
        // tile t+1 must be in LDS for every wave (the copies of tile t+2 may
        // still be in flight: exactly 4 of them), and every wave is past its
        // reads of tile t-1, whose stage is refilled
        wait_vm4();
        __syncthreads();
        issue_tile(min(t + 3, t_last), StageTag<S3>{});
        pv(KS, pa, av, KS1, ak);
        if (t == mask_tile) mask_tail(sb, mask_key0 + 32);
        qk_softmax(KS1, sa, sb, pbk, ak, KS + kSubBytes, av);
        pv(KS + kSubBytes, pbk, av, KS1 + kSubBytes, ak);
        if (t == mask_tile_prev && !last) mask_tail(sa, mask_key0);
        return last;
    };
    for (int t = t_begin;; t += 4) {
        if (tile(t, StageTag<0>{})) break;
        if (tile(t + 1, StageTag<1>{})) break;
        if (tile(t + 2, StageTag<2>{})) break;
        if (tile(t + 3, StageTag<3>{})) break;
    }

    // ---- epilogue: O^T[dv][q] / l; lanes l and l^32 hold halves of l
    const float lt = xhalf_sum(l);
    // MODE 3: slot < 0 marks a piece that is a whole item (written out here)
    if (MODE == 3 ? slot >= 0 : a.split != 0) {
        // piece of an item: unnormalised output, reference max, row sum
        const int64_t prow =
            (MODE == 3 ? (int64_t)slot : (int64_t)item * a.slots + slot) * kBM + wave * kWQ + lr;
        float *po = a.part_o + prow * kD;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *(float4 *)(po + 32 * b + 8 * g + 4 * hb) =
                    make_float4(o[b][4 * g], o[b][4 * g + 1], o[b][4 * g + 2], o[b][4 * g + 3]);
        if (hb == 0) *(float2 *)(a.part_ml + 2 * prow) = make_float2(m, lt);
        return;
    }
    const float inv = 1.f / lt;
    const int row = q0 + lr;
    if (row < a.n_q) {
        const int64_t base = (int64_t)row * hd + h * kD;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dv = 32 * b + 8 * g + 4 * hb;
                const float x0 = o[b][4 * g] * inv, x1 = o[b][4 * g + 1] * inv;
                const float x2 = o[b][4 * g + 2] * inv, x3 = o[b][4 * g + 3] * inv;
                if (a.out_bf16) {
                    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                    bf16x4 v = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
                    *(bf16x4 *)((uint16_t *)a.out + base + dv) = v;
                } else {
                    *(float4 *)((float *)a.out + base + dv) = make_float4(x0, x1, x2, x3);
                }
            }
        if (a.lse && hb == 0)
            a.lse[(int64_t)h * a.n_q + row] = (m + __log2f(lt)) * 0.69314718055994531f;
    }
  };

    // ---- this block's work: one whole item, or (split) its run of positions
    if (MODE == 3) {
        // Entries [b, e) of item i's tile list into LDS (published by the
        // barrier at the top of the segment); an entry out of range is
        // clamped, so that every copy stays inside the keys.
        auto load_list = [&](int i, int b, int e) __attribute__((always_inline)) {
            const int32_t *src = a.sp_tiles + (int64_t)i * n_tiles + b;
            for (int k = tid; k < e - b; k += kThreads) {
                const int v = src[k];
                sp_list[k] = v < 0 ? 0 : (v >= n_tiles ? n_tiles - 1 : v);
            }
        };
        if (__builtin_amdgcn_readfirstlane(a.sp_plan[0]) == 0) {
            // one block per item (counts clamped into [1, n_tiles] as the
            // plan does, so that the loop ends)
            if (blk >= a.items) return;
            int cnt = __builtin_amdgcn_readfirstlane(a.sp_count[blk]);
            cnt = cnt < 1 ? 1 : (cnt > n_tiles ? n_tiles : cnt);
            load_list(blk, 0, cnt);
            segment(blk, 0, cnt, -1);
            return;
        }
        // split: block blk takes list positions [blk total / G, (blk+1) total
        // / G) of the items' lists laid end to end; a piece that is not a
        // whole item leaves a partial result in slot item + blk (pieces in
        // position order raise item, block or both, so the slots differ)
        const int geff = __builtin_amdgcn_readfirstlane(a.sp_plan[1]);
        const int total = __builtin_amdgcn_readfirstlane(a.sp_plan[2]);
        if (blk >= geff) return;
        const int g0 = (int)((int64_t)blk * total / geff);
        const int g1 = (int)((int64_t)(blk + 1) * total / geff);
        auto item_of = [&](int g) -> int {   // sp_prefix[lo] <= g < sp_prefix[lo + 1]
            int lo = 0, hi = a.items;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (__builtin_amdgcn_readfirstlane(a.sp_prefix[mid]) <= g) lo = mid;
                else hi = mid;
            }
            return lo;
        };
        // Order of a run's pieces: a run that starts inside an item and
        // reaches past its end begins at that item's end and takes its
        // leading piece last (positions [start, g1), then [g0, start)).  The
        // items of one head have lists of about the same length L, so every
        // block of that head whose run holds an item boundary is then at list
        // position (t mod L) or ((t - run) mod L) after t tiles, whatever the
        // run's offset: the blocks of a head read the same tiles at about the
        // same time and share one L2.  In position order each block sat at its
        // own offset (3.5 GB fetched per Wan-shaped launch against 0.96 GB,
        // 4 % slower).  The pieces and their slots are the same either way,
        // so the results are too.
        int start = g0;
        if (g0 < g1) {
            const int i0 = item_of(g0);
            const int q0 = __builtin_amdgcn_readfirstlane(a.sp_prefix[i0]);
            const int q1 = __builtin_amdgcn_readfirstlane(a.sp_prefix[i0 + 1]);
            if (g0 > q0 && q1 < g1) start = q1;
        }
        for (int g = start, left = g1 - g0; left > 0;) {
            const int end = g >= start ? g1 : start;
            const int lo = item_of(g);
            const int p0 = __builtin_amdgcn_readfirstlane(a.sp_prefix[lo]);
            const int p1 = __builtin_amdgcn_readfirstlane(a.sp_prefix[lo + 1]);
            const int e = p1 < end ? p1 : end;
            __syncthreads();   // every wave is done with the previous piece's list
            load_list(lo, g - p0, e - p0);
            // (the arguments made uniform, as in the dense split: the compiler
            // then keeps them in scalar registers)
            segment(__builtin_amdgcn_readfirstlane(lo), 0, __builtin_amdgcn_readfirstlane(e - g),
                    __builtin_amdgcn_readfirstlane((g == p0 && e == p1) ? -1 : lo + blk));
            left -= e - g;
            g = e == g1 ? g0 : e;
        }
        return;
    }
    if (!a.split) {
        segment(blk, 0, n_tiles, 0);
        return;
    }
    const SplitMap map(a);
    const int64_t g1 = map.bnd(blk + 1), phase0 = (int64_t)a.items * map.S;
    for (int64_t g = map.bnd(blk); g < g1;) {
        int item, part, t_begin;
        if (g < phase0) {
            part = 0;
            item = (int)(g / map.S);
            t_begin = (int)(g - (int64_t)item * map.S);
        } else {
            part = 1;
            const int64_t h1 = g - phase0;
            item = (int)(h1 / (n_tiles - map.S));
            t_begin = map.S + (int)(h1 - (int64_t)item * (n_tiles - map.S));
        }
        const int64_t pend = map.part_end(item, part);
        const int64_t gend = pend < g1 ? pend : g1;
        const int t_end = t_begin + (int)(gend - g);
        segment(__builtin_amdgcn_readfirstlane(item), __builtin_amdgcn_readfirstlane(t_begin),
                __builtin_amdgcn_readfirstlane(t_end), map.slot(item, part, blk));
        g = gend;
    }
}

// Merge the pieces of every item of a split launch: for each query row,
// M = max of the reference maxima, L = sum l_j 2^{c(m_j - M)},
// O = sum O_j 2^{c(m_j - M)} / L, pieces in slot order (a running maximum
// with rescaling, so all the pieces' loads are independent).  One block of
// 256 threads per 8 query rows of an item: lane group (wave, lane / 32) owns
// a row, 32 lanes x 4 dims cover its 128 dims.
static constexpr int kMergeRows = 8;
template <bool SPARSE>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
    __shared__ int slot_list[kMaxSlots];
    __shared__ int n_pieces;
    const int item = blockIdx.x / (kBM / kMergeRows);
    const int r = (blockIdx.x % (kBM / kMergeRows)) * kMergeRows + (threadIdx.x >> 5);
    // sparse branch: the pieces of item i are the blocks w0 .. w1 whose runs
    // meet its positions [P_i, P_i+1), in slots i + w0 .. i + w1; one piece
    // was written out directly
    int first_slot = 0, np_sparse = 0;
    if (SPARSE) {
        if (a.sp_plan[0] == 0) return;
        const int64_t geff = a.sp_plan[1], total = a.sp_plan[2];
        const int64_t p0 = a.sp_prefix[item], p1 = a.sp_prefix[item + 1];
        const int w0 = (int)(((p0 + 1) * geff - 1) / total);
        const int w1 = (int)((p1 * geff - 1) / total);
        if (w0 == w1) return;
        first_slot = item + w0;
        np_sparse = w1 - w0 + 1;
    } else if (threadIdx.x == 0) {
        const SplitMap map(a);
        int n = 0;
        for (int p = 0; p < 2; ++p) {
            const int64_t b = map.part_begin(item, p), e = map.part_end(item, p);
            if (b >= e) continue;
            for (int w = map.block_of(b), wl = map.block_of(e - 1); w <= wl; ++w)
                if (map.bnd(w + 1) > map.bnd(w) && n < kMaxSlots) slot_list[n++] = map.slot(item, p, w);
        }
        n_pieces = n;
    }
    __syncthreads();
    const int np = SPARSE ? np_sparse : n_pieces;
    const int h = item / a.q_blocks, qb = item % a.q_blocks;
    const int row = qb * kBM + r;
    if (row >= a.n_q) return;
    const int64_t hd = (int64_t)a.n_heads * kD;
    const int d = 4 * (threadIdx.x & 31);
    const int64_t row0 = SPARSE ? (int64_t)first_slot * kBM + r : (int64_t)item * a.slots * kBM + r;
    float M = -INFINITY, L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < np; ++j) {
        const int64_t pr = row0 + (int64_t)(SPARSE ? j : slot_list[j]) * kBM;
        const float2 ml = *(const float2 *)(a.part_ml + 2 * pr);
        const float4 v = *(const float4 *)(a.part_o + pr * kD + d);
        const float mn = fmaxf(M, ml.x);
        const float fo = __builtin_amdgcn_exp2f(M - mn);   // 0 on the first piece
        const float f = __builtin_amdgcn_exp2f(ml.x - mn);
        L = L * fo + ml.y * f;
        acc.x = acc.x * fo + v.x * f;
        acc.y = acc.y * fo + v.y * f;
        acc.z = acc.z * fo + v.z * f;
        acc.w = acc.w * fo + v.w * f;
        M = mn;
    }
    const float inv = 1.f / L;
    const int64_t base = (int64_t)row * hd + h * kD + d;
    if (a.out_bf16) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v = {(__bf16)(acc.x * inv), (__bf16)(acc.y * inv), (__bf16)(acc.z * inv),
                    (__bf16)(acc.w * inv)};
        *(bf16x4 *)((uint16_t *)a.out + base) = v;
    } else {
        *(float4 *)((float *)a.out + base) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    if (a.lse && d == 0)
        a.lse[(int64_t)h * a.n_q + row] = (M + __log2f(L)) * 0.69314718055994531f;
}

// Plan of a sparse launch, from the item counts on the device (the host never
// sees them): the exclusive prefix P of the counts, each clamped into
// [1, n_tiles] as the attention kernel clamps them, and whether to split.
// Without the split one block runs each item, so the launch lasts about the
// longest item times the rounds of blocks (ceil(items / CUs)); with it, G =
// min(CUs, 32 items) blocks take equal runs of total / G positions.  Split
// when runs are at least kMinSplitTiles long and the unsplit launch would
// take over 1.25 times a run (the dense launch measured no faster split at
// 1.12).  One block of 1024 threads.
static constexpr int kPlanThreads = 1024;
__global__ __launch_bounds__(kPlanThreads) void k_sparse_plan(const int32_t *__restrict__ count,
                                                              int items, int n_tiles, int cu_count,
                                                              int32_t *__restrict__ plan,
                                                              int32_t *__restrict__ prefix) {
    __shared__ int sc[kPlanThreads];
    __shared__ int mx[kPlanThreads];
    const int t = threadIdx.x;
    const int per = (items + kPlanThreads - 1) / kPlanThreads;
    const int i0 = min(items, t * per), i1 = min(items, i0 + per);
    auto clamped = [&](int i) { const int c = count[i]; return c < 1 ? 1 : (c > n_tiles ? n_tiles : c); };
    int s = 0, m = 0;
    for (int i = i0; i < i1; ++i) {
        const int c = clamped(i);
        s += c;
        m = max(m, c);
    }
    sc[t] = s;
    mx[t] = m;
    __syncthreads();
    for (int d = 1; d < kPlanThreads; d <<= 1) {   // inclusive prefix sum, prefix max
        const int as = t >= d ? sc[t - d] : 0, am = t >= d ? mx[t - d] : 0;
        __syncthreads();
        sc[t] += as;
        mx[t] = max(mx[t], am);
        __syncthreads();
    }
    int run = sc[t] - s;
    for (int i = i0; i < i1; ++i) {
        prefix[i] = run;
        run += clamped(i);
    }
    if (t == kPlanThreads - 1) {
        const int total = sc[t], maxc = mx[t];
        prefix[items] = total;
        const int geff = min(cu_count, items * kMaxBlocksPerItem);
        const int64_t rounds = (items + cu_count - 1) / cu_count;
        const int64_t runlen = total / geff;
        plan[0] = runlen >= kMinSplitTiles && (int64_t)maxc * rounds * 4 > runlen * 5;
        plan[1] = geff;
        plan[2] = total;
    }
}

// Sparse workspace: plan (256 bytes), prefix [items + 1], then partial
// outputs and (max, sum) pairs for items + cu_count slots.
static size_t sparse_prefix_bytes(int items) { return align_up((size_t)(items + 1) * 4, 256); }
size_t sparse_workspace_bytes(int items, int cu_count) {
    return 256 + sparse_prefix_bytes(items) +
           (size_t)(items + cu_count) * kBM * (kD + 2) * sizeof(float);
}

AttnPlan attention_plan(int32_t n_heads, int32_t n_q, int32_t n_keys, int cu_count) {
    AttnPlan p;
    const int q_blocks = (n_q + kBM - 1) / kBM;
    const int items = q_blocks * n_heads;
    p.n_tiles = (n_keys + kBN - 1) / kBN;
    p.total = (int64_t)items * p.n_tiles;
    p.items = items;
    int g = cu_count < kMaxSplitBlocks ? cu_count : kMaxSplitBlocks;
    if ((int64_t)items * kMaxBlocksPerItem < g) g = items * kMaxBlocksPerItem;
    // split when one block per item would leave more than a quarter of the
    // CUs idle, and each block still gets a long run of tiles.  (With 89 % of
    // the CUs busy the split measured no faster: under a full matrix-core
    // load the clock falls as more CUs draw power, and the merge costs 1-2 %.)
    p.split = (int64_t)items * 4 <= (int64_t)g * 3 && p.total / g >= kMinSplitTiles;
    p.grid = p.split ? g : items;
    p.head_tiles = p.split ? (int)(p.total / g) : 0;
    p.slots = 0;
    if (p.split) {
        // pieces per item: a part of length n meets at most ceil(n / run) + 1
        // runs, runs being at least total / G = S long
        const int64_t run = p.total / g, tail = p.n_tiles - p.head_tiles;
        p.slots = (p.head_tiles > 0 ? 2 : 0) + (int)((tail + run - 1) / run) + 1;
        if (p.slots > kMaxSlots) {   // cannot happen with at most 32 blocks per item
            p.split = 0;
            p.grid = items;
            p.head_tiles = p.slots = 0;
        }
    }
    p.workspace = (size_t)items * p.slots * kBM * (kD + 2) * sizeof(float);
    return p;
}

hipError_t launch_attention_bf16(int32_t n_heads, const uint16_t *q, int32_t n_q,
                                 const uint16_t *k_ctx, const uint16_t *v_ctx, int32_t n_ctx,
                                 const uint16_t *k_own, const uint16_t *v_own, int32_t n_own,
                                 float scale, int32_t out_dtype, void *out, float *lse,
                                 const AttnPlan &plan, void *workspace, const PagedCtx &pg,
                                 hipStream_t s, const SparseCtx &sp) {
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
    a.n_tiles = plan.n_tiles;
    a.split = plan.split;
    a.grid = plan.grid;
    a.items = plan.items;
    a.head_tiles = plan.head_tiles;
    a.slots = plan.slots;
    a.total = plan.total;
    a.c = scale * 1.4426950408889634f;
    a.out_bf16 = out_dtype == WA_BF16;
    a.out = out;
    a.lse = lse;
    a.part_o = plan.split ? (float *)workspace : nullptr;
    a.part_ml = plan.split ? (float *)workspace + (size_t)plan.items * plan.slots * kBM * kD : nullptr;
    a.idx = pg.idx;
    a.page_tokens = pg.page_tokens;
    a.max_pages = pg.max_pages;
    a.tpp = pg.idx && pg.page_tokens % kBN == 0 ? pg.page_tokens / kBN : 0;
    a.page_bytes = (uint64_t)pg.page_tokens * (uint64_t)n_heads * kD * 2u;
    a.sp_tiles = sp.tiles;
    a.sp_count = sp.count;
    a.sp_plan = a.sp_prefix = nullptr;
    if (sp.tiles) {
        // plan on the device, then one block per item or per CU, then the
        // merge of split items
        char *ws = (char *)workspace;
        int32_t *plan_d = (int32_t *)ws, *prefix = (int32_t *)(ws + 256);
        a.sp_plan = plan_d;
        a.sp_prefix = prefix;
        a.split = 0;
        a.slots = 0;
        a.grid = sp.cu_count;
        a.part_o = (float *)(ws + 256 + sparse_prefix_bytes(plan.items));
        a.part_ml = a.part_o + (size_t)(plan.items + sp.cu_count) * kBM * kD;
        hipLaunchKernelGGL(k_sparse_plan, dim3(1), dim3(kPlanThreads), 0, s, sp.count, plan.items,
                           plan.n_tiles, sp.cu_count, plan_d, prefix);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int grid = plan.items > sp.cu_count ? plan.items : sp.cu_count;
        hipLaunchKernelGGL(k_attn_bf16<3>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_attn_merge<true>, dim3((unsigned)(plan.items * (kBM / kMergeRows))),
                           dim3(256), 0, s, a);
        return hipGetLastError();
    }
    if (!pg.idx)
        hipLaunchKernelGGL(k_attn_bf16<0>, dim3((unsigned)plan.grid), dim3(kThreads), 0, s, a);
    else if (a.tpp > 0)
        hipLaunchKernelGGL(k_attn_bf16<1>, dim3((unsigned)plan.grid), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(k_attn_bf16<2>, dim3((unsigned)plan.grid), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !plan.split) return e;
    hipLaunchKernelGGL(k_attn_merge<false>, dim3((unsigned)(a.q_blocks * n_heads * (kBM / kMergeRows))),
                       dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace wa
