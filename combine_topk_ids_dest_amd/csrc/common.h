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
// faster on gfx950; the pack (one read, several writes per token) uses plain
// loads and stores, which measured faster for it. Knobs for tuning builds;
// the defaults are the product settings.
#ifndef MOE_EP_PACK_NT
#define MOE_EP_PACK_NT 0
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

hipError_t launch_route_local(const int32_t* ids, int64_t T, int K, int E,
                              int e_local, int W, int32_t* rank,
                              int32_t* tile_cnt, uint32_t* err,
                              hipStream_t stream);

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
                            uint32_t* err, hipStream_t stream);

hipError_t launch_batch_local(const int32_t* recv_cnt, int64_t cnt_stride,
                              const int32_t* recv_eloc, int64_t eloc_stride,
                              int W, int e_local, int slots, int64_t cap,
                              int ntiles, int32_t* recv_row, int32_t* tile_cnt,
                              uint32_t* err, hipStream_t stream);

// tile_cnt != nullptr selects the fused tile offsets (fused_tiles <=
// kBatchFuseTiles): offsets are summed from tile_cnt and block 0 writes
// expert_num_tokens (clamped to clamp_max); otherwise tile_off holds the
// offsets from column_scan.
hipError_t launch_batch_copy(const int32_t* recv_cnt, int64_t cnt_stride,
                             const int32_t* recv_eloc, int64_t eloc_stride,
                             int W, int e_local, int slots, int64_t cap,
                             const int32_t* tile_off, const int32_t* tile_cnt,
                             int fused_tiles, int32_t* expert_num_tokens,
                             int32_t clamp_max, int32_t* recv_row,
                             const PayloadSet& P, uint32_t* err,
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
