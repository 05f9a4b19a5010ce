// Device helpers and launch declarations shared by the HIP kernels of the
// MoE expert-parallel dispatch/combine layout transform (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_ep.h"

namespace moe_ep {

// Tokens per block of the routing kernel (4 waves, one token per lane).
constexpr int kRouteTile = 256;
// Up to this many token tiles, pack_copy derives tile offsets itself.
#ifndef MOE_EP_PACK_FUSE_TILES
#define MOE_EP_PACK_FUSE_TILES 64
#endif
constexpr int kPackFuseTiles = MOE_EP_PACK_FUSE_TILES;
// Pick entries per block of the receive-scan kernel (256 lanes x 4 rounds).
constexpr int kBatchTile = 1024;
constexpr int kBatchRounds = kBatchTile / 256;
constexpr int kBatchChunks = kBatchTile / 64;   // wave-sized chunks per tile
// Up to this many pick tiles, moe_ep_expert_batch runs no column_scan: the
// copy kernel sums tile offsets itself and writes expert_num_tokens.
#ifndef MOE_EP_BATCH_FUSE_TILES
#define MOE_EP_BATCH_FUSE_TILES 64
#endif
constexpr int kBatchFuseTiles = MOE_EP_BATCH_FUSE_TILES;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Row data is touched once per call. The combine kernels and the expert
// batch copy load and store it with the nontemporal hint, which measured
// faster on gfx950; the pack (one read, several writes per token) stores
// with the hint but loads without it (nontemporal loads measured slower
// there). Knobs for tuning builds; the defaults are the product settings.
#ifndef MOE_EP_PACK_LD_NT
#define MOE_EP_PACK_LD_NT 0
#endif
#ifndef MOE_EP_PACK_ST_NT
#define MOE_EP_PACK_ST_NT 1
#endif
#ifndef MOE_EP_BATCH_LD_NT
#define MOE_EP_BATCH_LD_NT 1
#endif
#ifndef MOE_EP_BATCH_ST_NT
#define MOE_EP_BATCH_ST_NT 1
#endif
#ifndef MOE_EP_COMBINE_NT
#define MOE_EP_COMBINE_NT 1
#endif
// Grid cap of the kernels that walk received slot rows (grid-stride).
#ifndef MOE_EP_ROW_GRID
#define MOE_EP_ROW_GRID 16384
#endif

template <bool NT>
__device__ __forceinline__ u32x4 ld_row(const uint8_t* p) {
    if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return *reinterpret_cast<const u32x4*>(p);
}

template <bool NT>
__device__ __forceinline__ void st_row(uint8_t* p, const u32x4& v) {
    if (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
    else *reinterpret_cast<u32x4*>(p) = v;
}

// A row of `bytes` bytes as a buffer resource (a longer row is covered up to
// 2^31 - 1 bytes): a 16-byte load at an offset past that end returns zeros
// without touching memory (the
// buffer unit's range check), so lanes past the end need no branch and a
// lane's loads are issued back to back. (Loads under a per-lane branch
// whose registers stay live past it are each followed by a wait, for the
// copy that merges the branch.) Dword 3 selects the 32-bit data format,
// which raw buffer accesses need on gfx9.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint8_t* p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0,
                                             (int)(bytes < INT32_MAX ? bytes : INT32_MAX),
                                             0x00020000);
}

template <bool NT>
__device__ __forceinline__ u32x4 ld_row_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4,
                              __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0));
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Quantize-on-pack arguments: bf16 rows in; codes and per-group scale rows
// out, for every destination of the token. mode 1, fp8: codes [W, cap, H]
// (one byte per column), fp32 scales. mode 2, fp4: codes [W, cap, H/2]
// (two E2M1 codes per byte), E4M3 scale codes (one byte per 16 columns).
// Scale rows are padded to a multiple of 16 bytes with zero bytes (+0.0).
struct QuantArgs {
    const uint8_t* src;   // bf16 rows [T, H]
    int64_t src_stride;   // bytes between tokens
    uint8_t* q;           // codes
    int64_t q_stride;     // bytes between destination blocks
    uint8_t* s;           // scale rows [W, cap, s_pitch bytes]
    int64_t s_stride;     // bytes between destination blocks
    int64_t s_pitch;      // bytes per scale row
    int64_t n_scales;     // scales per row: H / group
    int64_t H;
    int group;            // fp8: 32, 64 or 128 columns; fp4: 16
    int mode;             // 1 fp8, 2 fp4
};

// Payload descriptors passed by value as a kernel argument.
struct PayloadSet {
    const uint8_t* src[MOE_EP_MAX_PAYLOADS];
    uint8_t* dst[MOE_EP_MAX_PAYLOADS];
    int64_t src_stride[MOE_EP_MAX_PAYLOADS];
    int64_t dst_stride[MOE_EP_MAX_PAYLOADS];
    int64_t row_bytes[MOE_EP_MAX_PAYLOADS];
    int n;
};

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ int rank_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi(
        (uint32_t)(mask >> 32),
        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ void report(uint32_t* err, uint32_t bits) {
    if (bits && err) atomicOr(err, bits);
}

// Destination mask of one token: bit d is set when some routed pick of the
// token lives on rank d = id / e_local. Negative ids are padding; ids >= E
// are dropped and flagged. The ids are read 8 at a time with all 8 loads in
// flight before the first is used (a load per pick followed by its use
// would cost one memory latency per pick).
__device__ __forceinline__ uint64_t token_dest_mask(const int32_t* __restrict__ row, int K,
                                                    int E, int e_local, uint32_t& bad) {
    uint64_t mask = 0;
    for (int k0 = 0; k0 < K; k0 += 8) {
        int32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = k0 + u < K ? row[k0 + u] : -1;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int32_t id = v[u];
            if (id >= E) bad |= MOE_EP_ERR_ID_RANGE;
            if (id >= 0 && id < E) mask |= 1ull << ((uint32_t)id / (uint32_t)e_local);
        }
    }
    return mask;
}

// ---------------------------------------------------------------------
// Send-side per-expert ranks. On the vLLM alltoall_batched page the
// receive side gives a local expert's rows to its picks in (source, slot,
// column) order; within one source that is the order it sends in (tokens
// ascending, router order), so a source can count its own share: each kept
// pick's rank among the source's kept picks of the same expert, and the
// number per expert. The receiver adds the counts of the sources before.
// Limits of this form: K <= kRankMaxK picks per token and E <= kRankMaxE.
// ---------------------------------------------------------------------
constexpr int kRankMaxK = 16;
constexpr int kRankMaxE = 4096;
// Up to this many experts the masks of the fast form fit in LDS
// (4 waves x E x 8 bytes).
constexpr int kRankMaskE = 1024;

struct RankArgs {
    int32_t* send_rank;          // like send_eloc (meta stride); nullptr: not asked for
    int32_t* send_ecnt;          // [W, e_local] dense, every entry written
    const int32_t* prank;        // in-tile ranks [T * K] (route_local), or nullptr
    const int32_t* ecnt_tile;    // [tiles][E] counts per tile (prefix summed here)
    const int32_t* eoff_tile;    // [tiles][E] tile offsets (column_scan), or nullptr
    int nbits;                   // bits of an expert id: E <= 2^nbits
};

// The K ids of one token into registers (v[k] = -1 for k >= K), all loads
// in flight together. K <= kRankMaxK.
template <int KB = kRankMaxK>
__device__ __forceinline__ void load_row_ids(const int32_t* __restrict__ row, int K,
                                             int32_t (&v)[kRankMaxK]) {
#pragma unroll
    for (int k = 0; k < KB; ++k) v[k] = k < K ? row[k] : -1;
}

// Destination mask of one token from its ids in registers (as
// token_dest_mask).
template <int KB = kRankMaxK>
__device__ __forceinline__ uint64_t dest_mask_of(const int32_t (&v)[kRankMaxK], int E,
                                                 int e_local, uint32_t& bad) {
    uint64_t mask = 0;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        if (v[k] >= E) bad |= MOE_EP_ERR_ID_RANGE;
        if (v[k] >= 0 && v[k] < E) mask |= 1ull << ((uint32_t)v[k] / (uint32_t)e_local);
    }
    return mask;
}

// Kept picks of one token in router order, in place on its ids in
// registers: a valid id (0 <= id < E) is kept while fewer than `slots`
// earlier valid picks of the token go to the same rank (the others are
// dropped, as the pack drops them). key[k] = id of a kept pick, else -1
// (also for k >= K). Loops are unrolled to kRankMaxK so that the ids stay
// in registers.
template <int KB = kRankMaxK>
__device__ __forceinline__ void keep_keys(int K, int E, int e_local, int slots,
                                          int32_t (&key)[kRankMaxK]) {
    int32_t dst[kRankMaxK];
#pragma unroll
    for (int k = 0; k < KB; ++k)
        if (key[k] >= E || key[k] < 0) key[k] = -1;
    if (slots >= K) return;   // a rank can take all K picks of a token
#pragma unroll
    for (int k = 0; k < KB; ++k)
        dst[k] = key[k] >= 0 ? (int32_t)((uint32_t)key[k] / (uint32_t)e_local) : -1;
#pragma unroll
    for (int k = KB - 1; k > 0; --k) {
        int before = 0;
#pragma unroll
        for (int k2 = 0; k2 < k; ++k2) before += (dst[k2] >= 0 && dst[k2] == dst[k]) ? 1 : 0;
        if (before >= slots) key[k] = -1;
    }
}

// Whether a token's kept ids hold an expert twice (only possible with
// duplicate ids in its routing).
template <int KB = kRankMaxK>
__device__ __forceinline__ bool has_repeated_key(const int32_t (&key)[kRankMaxK]) {
    bool rep = false;
#pragma unroll
    for (int k = 1; k < KB; ++k)
#pragma unroll
        for (int k2 = 0; k2 < k; ++k2) rep |= key[k] >= 0 && key[k] == key[k2];
    return rep;
}

// Ranks of the kept picks of one tile of tokens among the tile's kept picks
// of the same expert, in (token, router order). keys[i], i = t_local*K + k
// for the tile's n entries (LDS): expert id or -1. Wave w owns the entries
// of its 64 tokens, [64*K*w, 64*K*(w+1)), and walks them in chunks of 64:
// a multi-split over the nbits bits of the id gives each entry its rank
// among the chunk's entries of the same expert, to which the wave's running
// count of that expert (hist row w, LDS, zeroed by the caller) is added;
// the group's first lane then advances that count. The rows of hist become
// prefixes over the waves, and row `waves` the tile's count per expert.
// rank[i] (LDS): the rank within the tile, -1 for an entry that is not a
// kept pick. All threads of the block call this; it ends with a barrier.
__device__ __forceinline__ void tile_expert_ranks(const int16_t* keys, int16_t* rank,
                                                  int n, int K, int E, int nbits,
                                                  int16_t* hist, int waves) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int16_t* h = hist + wave * E;
    for (int c = 0; c < K; ++c) {
        const int i = wave * 64 * K + c * 64 + lane;
        const int32_t g = i < n ? keys[i] : -1;
        uint64_t peers = __ballot(g >= 0);
        for (int b = 0; b < nbits; ++b) {
            const uint64_t ones = __ballot(g >= 0 && ((g >> b) & 1));
            peers &= ((g >> b) & 1) ? ones : ~ones;
        }
        // every lane reads the running count before the group's first lane
        // advances it (one instruction stream: the read precedes the write)
        const int32_t before = g >= 0 ? h[g] : 0;
        const int r = rank_below(peers);
        if (g >= 0 && r == 0) h[g] = (int16_t)(before + __popcll(peers));
        if (i < n) rank[i] = (int16_t)(g >= 0 ? before + r : -1);
    }
    __syncthreads();
    for (int g = threadIdx.x; g < E; g += blockDim.x) {
        int32_t run = 0;
        for (int w = 0; w < waves; ++w) {
            const int32_t v = hist[w * E + g];
            hist[w * E + g] = (int16_t)run;
            run += v;
        }
        hist[waves * E + g] = (int16_t)run;
    }
    __syncthreads();
    for (int c = 0; c < K; ++c) {
        const int i = wave * 64 * K + c * 64 + lane;
        if (i < n && keys[i] >= 0) rank[i] = (int16_t)(rank[i] + hist[wave * E + keys[i]]);
    }
    __syncthreads();
}

// The fast form of the per-expert ranks, for tiles where no token holds an
// expert twice: then a pick's rank is the number of the tile's tokens
// before its own that hold the same expert. Each wave ORs its lanes' bits
// into masks[wave * E + g] for every kept id g of its tokens (LDS atomics:
// the result does not depend on their order); masks must be zeroed before
// and a barrier must separate this from the queries.
template <int KB = kRankMaxK>
__device__ __forceinline__ void mark_expert_masks(const int32_t (&key)[kRankMaxK],
                                                  unsigned long long* masks, int E) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < KB; ++k)
        if (key[k] >= 0) atomicOr(&masks[wave * E + key[k]], 1ull << lane);
}

// Rank of expert g at tile-local token tl (fast form): the tokens of the
// waves before tl's that hold g, plus those below tl in its own wave. All
// WAVES masks of g are read at once (their loads in flight together).
template <int WAVES>
__device__ __forceinline__ int32_t mask_rank(const unsigned long long* masks, int E, int tl,
                                             int32_t g) {
    const int w = tl >> 6;
    const unsigned long long below = (1ull << (tl & 63)) - 1ull;
    unsigned long long m[WAVES];
#pragma unroll
    for (int w2 = 0; w2 < WAVES; ++w2) m[w2] = masks[w2 * E + g];
    int32_t r = 0;
#pragma unroll
    for (int w2 = 0; w2 < WAVES; ++w2)
        r += w2 < w ? __popcll(m[w2]) : (w2 == w ? __popcll(m[w2] & below) : 0);
    return r;
}

// Largest s in [0, W) with pre[s] <= v, for an ascending prefix array
// pre[0..W] (pre[0] = 0) and v < pre[W].
__device__ __forceinline__ int find_source(const int32_t* pre, int W, int32_t v) {
    int lo = 0, hi = W - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= v) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// Counts received from each source, clamped to [0, cap], and their
// exclusive prefix pre[0..W]. Run by wave 0 of a block; W <= 64.
__device__ __forceinline__ void load_recv_prefix(const int32_t* recv_cnt,
                                                 int64_t cnt_stride, int W,
                                                 int64_t cap, int32_t* pre,
                                                 uint32_t* err, int skip = -1) {
    const int lane = threadIdx.x & 63;
    int32_t c = 0;
    uint32_t bad = 0;
    if (lane < W && lane != skip) {
        int64_t v = recv_cnt[(int64_t)lane * cnt_stride];
        if (v < 0 || v > cap) {
            bad = MOE_EP_ERR_CNT;
            v = v < 0 ? 0 : cap;
        }
        c = (int32_t)v;
    }
    report(err, bad);
    const int32_t inc = wave_inclusive_scan(c);
    if (lane == 0) pre[0] = 0;
    if (lane < W) pre[lane + 1] = inc;
}

// bf16 <-> fp32. bf16 is the upper half of a binary32; rounding to bf16 is
// to nearest, ties to even, NaNs stay quiet NaNs.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------
// Launchers (defined next to their kernels). All return hipError_t of the
// launch; grids are computed from host-known sizes only.
// ---------------------------------------------------------------------
// Column parts a row is cut into so that `rows` rows still give enough
// blocks to fill the chip; no part is narrower than one pass of 256 lanes.
#ifndef MOE_EP_SPLIT_BLOCKS
#define MOE_EP_SPLIT_BLOCKS 2048
#endif
inline int row_split(int64_t rows, int64_t max_vecs) {
    int64_t s = rows > 0 ? (MOE_EP_SPLIT_BLOCKS + rows - 1) / rows : 1;
    const int64_t by_width = max_vecs / 256 > 0 ? max_vecs / 256 : 1;
    if (s > by_width) s = by_width;
    if (s < 1) s = 1;
    return (int)s;
}

// prank != nullptr: also the per-expert in-tile ranks of the kept picks
// (prank [T * K]) and the tiles' counts per expert (ecnt_tile [tiles][E]).
hipError_t launch_route_local(const int32_t* ids, int64_t T, int K, int E,
                              int e_local, int W, int slots, int32_t* rank,
                              int32_t* tile_cnt, int32_t* prank, int32_t* ecnt_tile,
                              int nbits, uint32_t* err, hipStream_t stream);

hipError_t launch_column_scan(const int32_t* cnt, int ntiles, int nkeys,
                              int32_t* off, int32_t* total, int32_t clamp_max,
                              hipStream_t stream);

// rank: the in-tile ranks of route_local ([W, T], -1 = no pair).
// tile_cnt != nullptr selects the fused tile offsets (ntiles <=
// kPackFuseTiles): offsets are summed from tile_cnt and block 0 writes
// send_cnt; otherwise tile_off holds the offsets from column_scan.
// quant != nullptr adds quantize-on-pack of a bf16 row (QuantArgs).
hipError_t launch_pack_copy(const int32_t* ids, const float* wts, int64_t T,
                            int K, int E, int e_local, int W, int slots,
                            int64_t cap, const int32_t* rank,
                            int32_t* token_slot, const int32_t* tile_cnt,
                            const int32_t* tile_off, int32_t* send_cnt,
                            const PayloadSet& P, const QuantArgs* quant,
                            int32_t* send_eloc, float* send_w, int64_t meta_stride,
                            const RankArgs* ranks, uint32_t* err, hipStream_t stream);

hipError_t launch_batch_local(const int32_t* recv_cnt, int64_t cnt_stride,
                              const int32_t* recv_eloc, int64_t eloc_stride,
                              int W, int e_local, int slots, int64_t cap,
                              int ntiles, int32_t* recv_row, int32_t* tile_cnt,
                              uint32_t* err, hipStream_t stream);

// tile_cnt != nullptr selects the fused tile offsets (fused_tiles <=
// kBatchFuseTiles): offsets are summed from tile_cnt and block 0 writes
// expert_num_tokens (clamped to clamp_max); otherwise tile_off holds the
// offsets from column_scan.
// recv_rank != nullptr: rows from the sources' per-expert ranks (same
// layout and stride as recv_eloc) and counts (recv_ecnt, source s's
// [e_local] at recv_ecnt + s * ecnt_stride); no receive scan.
hipError_t launch_batch_copy(const int32_t* recv_cnt, int64_t cnt_stride,
                             const int32_t* recv_eloc, int64_t eloc_stride,
                             int W, int e_local, int slots, int64_t cap,
                             const int32_t* tile_off, const int32_t* tile_cnt,
                             int fused_tiles, const int32_t* recv_rank,
                             const int32_t* recv_ecnt, int64_t ecnt_stride,
                             int32_t* expert_num_tokens, int32_t clamp_max,
                             int32_t* recv_row, const PayloadSet& P, uint32_t* err,
                             hipStream_t stream);

hipError_t launch_sanitize_ids(const int32_t* recv_cnt, int64_t cnt_stride,
                               const int32_t* recv_eloc, int64_t eloc_stride,
                               int W, int e_local, int slots, int64_t cap,
                               int32_t invalid_id, int32_t* out,
                               int64_t out_stride, uint32_t* err,
                               hipStream_t stream);

hipError_t launch_combine_reduce(const void* Y, int64_t y_expert_stride,
                                 int dtype, int64_t H, const int32_t* recv_cnt,
                                 int64_t cnt_stride, const int32_t* recv_eloc,
                                 const float* recv_w, int64_t meta_stride,
                                 const int32_t* recv_row, int W, int e_local,
                                 int slots, int64_t cap, void* ret,
                                 int64_t ret_stride, int skip_src,
                                 hipStream_t stream);

hipError_t launch_combine_unpack(const void* back, int64_t back_stride,
                                 int dtype, int64_t H,
                                 const int32_t* token_slot, int64_t T, int W,
                                 int64_t cap, void* out, hipStream_t stream);

hipError_t launch_combine_unpack_fused(
    const void* back, int64_t back_stride, int dtype, int64_t H,
    const int32_t* token_slot, int64_t T, int W, int64_t cap, int self_rank,
    const void* Y, int64_t y_expert_stride, const int32_t* self_eloc,
    const float* self_w, const int32_t* self_row, int e_local, int slots,
    void* out, hipStream_t stream);

}  // namespace moe_ep
