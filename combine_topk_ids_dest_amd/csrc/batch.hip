// Receive-side expert batching of one destination rank (prepare() on the
// vLLM "alltoall_batched" documentation page after the exchange: a pick
// (s, slot, j) is valid when slot < recv_cnt[s] and its local id is >= 0;
// valid picks, taken in (s, slot, j) order, take the next row of their local
// expert; rows are copied into [e_local, W*cap, row]; expert_num_tokens
// counts them).
//
// The valid slots of all sources are numbered densely, v = pre[s] + slot
// (pre = prefix of the received counts), and the picks q = v*slots + j are
// cut into tiles of 1024. Rows come from a two-level scan with no atomics:
//   batch_local: in each wave, a multi-split over the bits of the local id
//     (log2(e_local) ballots) gives every pick its rank among the wave's
//     picks of the same expert; a per-tile scan over the 16 wave chunks
//     gives the in-tile rank, stored provisionally in recv_row, and the
//     tile's count per expert goes to the workspace.
//   column_scan: tile offsets per expert and expert_num_tokens.
//   batch_copy: one slot row per block; final row = provisional + tile
//     offset; the row is read once and stored to each of its experts' rows.
// With few tiles (moe_ep_expert_batch, at most kBatchFuseTiles) there is no
// column_scan: batch_copy sums the tile offset of each pick from the tile
// counts itself and its block 0 writes expert_num_tokens. With the sources'
// per-expert ranks (moe_ep_expert_batch_ranked) neither scan runs: a row is
// the counts of the sources before plus the rank, so batch_copy is the
// whole receive side.
#include "common.h"

namespace moe_ep {

__global__ __launch_bounds__(256) void batch_local_kernel(
    const int32_t* __restrict__ recv_cnt, int64_t cnt_stride,
    const int32_t* __restrict__ recv_eloc, int64_t eloc_stride, int W,
    int e_local, int slots, int64_t cap, int nbits,
    int32_t* __restrict__ recv_row, int32_t* __restrict__ tile_cnt,
    uint32_t* __restrict__ err) {
    // [kBatchChunks][e_local]; per-chunk counts and in-tile prefixes are
    // at most kBatchTile, so 16 bits hold them.
    extern __shared__ int16_t chunk_cnt[];
    __shared__ int32_t pre[MOE_EP_MAX_WORLD + 1];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;

    if (tid < 64) load_recv_prefix(recv_cnt, cnt_stride, W, cap, pre, err);
    for (int i = tid; i < kBatchChunks * e_local; i += 256) chunk_cnt[i] = 0;
    __syncthreads();

    // Pick indices fit in 32 bits (W * cap * slots < 2^31 is checked on the
    // host), which keeps the divisions below 32-bit.
    const int32_t nq = pre[W] * slots;
    const int32_t q0 = (int32_t)blockIdx.x * kBatchTile;
    if (q0 >= nq) {
        for (int e = tid; e < e_local; e += 256)
            tile_cnt[(int64_t)blockIdx.x * e_local + e] = 0;
        return;
    }

    int64_t at[kBatchRounds];    // recv_row index of this lane's pick
    int32_t key[kBatchRounds];   // local expert, -1 if none
    int32_t rnk[kBatchRounds];   // rank among the wave's picks of that key
    uint32_t bad = 0;
    // All rounds' loads first, so their latencies overlap.
#pragma unroll
    for (int c = 0; c < kBatchRounds; ++c) {
        const int32_t q = q0 + c * 256 + tid;
        key[c] = -1;
        at[c] = -1;
        if (q < nq) {
            const int32_t v = q / slots;
            const int j = q - v * slots;
            const int s = find_source(pre, W, v);
            const int32_t slot = v - pre[s];
            key[c] = recv_eloc[s * eloc_stride + (int64_t)slot * slots + j];
            at[c] = ((int64_t)s * cap + slot) * slots + j;
        }
    }
#pragma unroll
    for (int c = 0; c < kBatchRounds; ++c) {
        int32_t e = key[c];
        if (e >= e_local) { bad |= MOE_EP_ERR_ELOC; e = -1; }
        // Multi-split: lanes whose keys agree on every bit are peers.
        uint64_t peers = __ballot(e >= 0);
        for (int b = 0; b < nbits; ++b) {
            const uint64_t ones = __ballot(e >= 0 && ((e >> b) & 1));
            peers &= ((e >> b) & 1) ? ones : ~ones;
        }
        key[c] = e;
        rnk[c] = rank_below(peers);
        if (e >= 0 && rnk[c] == 0)
            chunk_cnt[(c * 4 + wave) * e_local + e] = (int16_t)__popcll(peers);
    }
    report(err, bad);
    __syncthreads();

    for (int e = tid; e < e_local; e += 256) {
        int32_t run = 0;
        for (int ch = 0; ch < kBatchChunks; ++ch) {
            const int32_t v = chunk_cnt[ch * e_local + e];
            chunk_cnt[ch * e_local + e] = (int16_t)run;
            run += v;
        }
        tile_cnt[(int64_t)blockIdx.x * e_local + e] = run;
    }
    __syncthreads();

#pragma unroll
    for (int c = 0; c < kBatchRounds; ++c) {
        if (at[c] >= 0)
            recv_row[at[c]] = key[c] >= 0
                ? chunk_cnt[(c * 4 + wave) * e_local + key[c]] + rnk[c] : -1;
    }
}

constexpr int kBatchThreads = 256;

// Sum of tile_cnt[j][key] over tiles j < tiles of a [tiles][nkeys] table
// (loads issued 8 at a time).
__device__ __forceinline__ int32_t sum_tile_column(const int32_t* __restrict__ tile_cnt,
                                                   int32_t tiles, int nkeys, int key) {
    int32_t s = 0;
    for (int32_t j0 = 0; j0 < tiles; j0 += 8) {
        int32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = j0 + u < tiles ? tile_cnt[(int64_t)(j0 + u) * nkeys + key] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    return s;
}
constexpr int kBatchUnroll = 4;
// A row of one payload above this many 16-byte vectors has its first pass
// loaded before the slot's expert rows are known (the loads overlap wave 0's
// planning). It costs registers (6 waves per SIMD instead of 8), which
// narrower rows, with less to overlap, and rows of several payloads, whose
// later payloads are not prefetched, need more: at the DS-V3 shape (one
// 14 KiB payload) the early pass took the copy from 152-155 to 148 us, at
// the multi-payload shape (14 KiB + four more payloads) it made it slower,
// 365 against 345 us.
#ifndef MOE_EP_BATCH_PREFETCH_VECS
#define MOE_EP_BATCH_PREFETCH_VECS 512
#endif

// Where a pick's expert row comes from:
//   kRowsScanned: the receive scan (batch_local's in-tile rank in recv_row
//     plus the tile offset from column_scan, tile_off);
//   kRowsFused: the same, with the tile offset summed here from tile_cnt
//     (fused_tiles tiles) and expert_num_tokens written by block 0;
//   kRowsRanked: the sources' per-expert ranks (recv_rank, beside the local
//     ids) plus the counts of the sources before. Each block first copies
//     all W x e_local counts (recv_ecnt) into LDS, so a pick's sum is a few
//     LDS reads instead of a second round of global loads after its id
//     (and the planning needs fewer registers: 7 waves per SIMD instead of
//     5 with the early pass); block 0 writes expert_num_tokens. No receive
//     scan and no workspace.
constexpr int kRowsScanned = 0;
constexpr int kRowsFused = 1;
constexpr int kRowsRanked = 2;

// Sum of v[0..n) saturated at cap, for 0 <= v[i] <= cap < 2^31 (the sum
// stays below 2^32 before each saturation, so 32 unsigned bits hold it).
__device__ __forceinline__ int32_t saturating_sum(const int32_t* v, int n, int32_t cap) {
    uint32_t sum = 0;
#pragma unroll 8
    for (int i = 0; i < n; ++i) {
        sum += (uint32_t)v[i];
        sum = sum < (uint32_t)cap ? sum : (uint32_t)cap;
    }
    return (int32_t)sum;
}

template <bool PREFETCH, int ROWS>
__global__ __launch_bounds__(kBatchThreads) void batch_copy_kernel(
    const int32_t* __restrict__ recv_cnt, int64_t cnt_stride,
    const int32_t* __restrict__ recv_eloc, int64_t eloc_stride, int W,
    int e_local, int slots, int64_t cap, const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ tile_cnt, int32_t fused_tiles,
    const int32_t* __restrict__ recv_rank, const int32_t* __restrict__ recv_ecnt,
    int64_t ecnt_stride, int32_t* __restrict__ expert_num_tokens, int32_t clamp_max,
    int32_t* __restrict__ recv_row, const PayloadSet P,
    uint32_t* __restrict__ err) {
    __shared__ int32_t pre[MOE_EP_MAX_WORLD + 1];
    __shared__ int32_t s_exp[MOE_EP_MAX_SLOTS];
    __shared__ int32_t s_row[MOE_EP_MAX_SLOTS];
    __shared__ int s_n;
    // ranked: every source's count of each local expert, clamped to
    // [0, expert_cap], as [e_local][W] (dynamic LDS, W * e_local <= kRankMaxE)
    extern __shared__ int32_t s_ecnt[];
    const int tid = threadIdx.x;
    const int64_t expert_cap = (int64_t)W * cap;
    const int32_t ecap = (int32_t)expert_cap;   // < 2^31, checked on the host

    if (ROWS == kRowsRanked) {
        const int n = W * e_local;
#pragma unroll 4
        for (int i = tid; i < n; i += kBatchThreads) {
            const int s = i / e_local;
            const int e = i - s * e_local;
            const int32_t c = recv_ecnt[(int64_t)s * ecnt_stride + e];
            s_ecnt[e * W + s] = c < 0 ? 0 : (c > ecap ? ecap : c);
        }
    }

    // (a count outside [0, cap] is reported by the receive scan, or here
    // by block 0 when no scan runs)
    if (tid < 64)
        load_recv_prefix(recv_cnt, cnt_stride, W, cap, pre,
                         ROWS == kRowsRanked && blockIdx.x == 0 ? err : nullptr);
    if (ROWS == kRowsFused && blockIdx.x == 0) {
        for (int e = tid; e < e_local; e += kBatchThreads) {
            const int32_t tot = sum_tile_column(tile_cnt, fused_tiles, e_local, e);
            expert_num_tokens[e] = tot < clamp_max ? tot : clamp_max;
        }
    }
    __syncthreads();
    if (ROWS == kRowsRanked && blockIdx.x == 0) {
        for (int e = tid; e < e_local; e += kBatchThreads) {
            const int32_t tot = saturating_sum(s_ecnt + e * W, W, ecap);
            expert_num_tokens[e] = tot < clamp_max ? tot : clamp_max;
        }
    }
    const int32_t S = pre[W];

    for (int32_t v = blockIdx.x; v < S; v += gridDim.x) {
        const int s = find_source(pre, W, v);
        const int32_t slot = v - pre[s];
        // The source row does not depend on the expert rows: with the
        // prefetch its first pass is in flight while wave 0 plans the rows.
        u32x4 x0[kBatchUnroll];
        int64_t first = 0;
        if (PREFETCH && P.n > 0) {
            const int64_t rb = P.row_bytes[0];
            const int64_t nvec = rb >> 4;
            const uint8_t* src = P.src[0] + s * P.src_stride[0] + (int64_t)slot * rb;
            if (ROWS == kRowsRanked) {
                // all of the lane's loads in flight at once (buffer loads:
                // no branch per load); the planning's only global loads
                // follow them
                const __amdgpu_buffer_rsrc_t rs = row_rsrc(src, rb);
#pragma unroll
                for (int u = 0; u < kBatchUnroll; ++u)
                    x0[u] = ld_row_buf<MOE_EP_BATCH_LD_NT>(
                        rs, (uint32_t)(tid + u * kBatchThreads) * 16u);
            } else {
                // guarded loads: the compiler waits for each before the
                // next, which measured faster for the scanned rows than
                // all four in flight (buffer loads: DS-V3 148.9-149.5
                // against 145.5 us), while the ranked rows gain from it
                // (decode 10.6 against 11.2 us)
#pragma unroll
                for (int u = 0; u < kBatchUnroll; ++u) {
                    const int64_t i = tid + u * kBatchThreads;
                    if (i < nvec) x0[u] = ld_row<MOE_EP_BATCH_LD_NT>(src + i * 16);
                }
            }
            first = kBatchThreads * kBatchUnroll;
        }
        if (tid < 64) {
            const int j = tid;
            int32_t row = -1;
            int32_t e = -1;
            uint32_t bad = 0;
            if (j < slots) {
                const int64_t at = ((int64_t)s * cap + slot) * slots + j;
                const int64_t meta = s * eloc_stride + (int64_t)slot * slots + j;
                if (ROWS == kRowsRanked) {
                    // the rank is loaded with the id, not after it
                    e = recv_eloc[meta];
                    const int32_t rk = recv_rank[meta];
                    if (e >= e_local) bad |= MOE_EP_ERR_ELOC;
                    if (e >= 0 && e < e_local) {
                        const int64_t r =
                            (int64_t)saturating_sum(s_ecnt + e * W, s, ecap) + rk;
                        if (rk >= 0 && r < expert_cap) row = (int32_t)r;
                        else bad |= MOE_EP_ERR_ROWCAP;
                    }
                } else {
                    // the provisional row is loaded with the id, not after it
                    e = recv_eloc[meta];
                    const int32_t prov = recv_row[at];
                    const bool ok = e >= 0 && e < e_local;
                    const int32_t q = v * slots + j;
                    const int32_t off =
                        ROWS == kRowsFused
                            ? sum_tile_column(tile_cnt, q / kBatchTile, e_local, ok ? e : 0)
                            : tile_off[(int64_t)(q / kBatchTile) * e_local + (ok ? e : 0)];
                    if (ok) {
                        const int64_t r = (int64_t)prov + off;
                        if (r < expert_cap) row = (int32_t)r;
                        else bad |= MOE_EP_ERR_ROWCAP;
                    }
                }
                recv_row[at] = row;
            }
            const uint64_t act = __ballot(row >= 0);
            if (row >= 0) {
                const int pos = rank_below(act);
                s_exp[pos] = e;
                s_row[pos] = row;
            }
            report(err, bad);
            if (tid == 0) s_n = __popcll(act);
        }
        __syncthreads();
        const int n = s_n;

        if (PREFETCH && P.n > 0) {
            const int64_t rb = P.row_bytes[0];
            const int64_t nvec = rb >> 4;
            for (int a = 0; a < n; ++a) {
                uint8_t* dst = P.dst[0] + s_exp[a] * P.dst_stride[0] + (int64_t)s_row[a] * rb;
#pragma unroll
                for (int u = 0; u < kBatchUnroll; ++u) {
                    const int64_t i = tid + u * kBatchThreads;
                    if (i < nvec) st_row<MOE_EP_BATCH_ST_NT>(dst + i * 16, x0[u]);
                }
            }
        }
        for (int p = 0; p < P.n; ++p) {
            const int64_t rb = P.row_bytes[p];
            const uint8_t* src = P.src[p] + s * P.src_stride[p] + (int64_t)slot * rb;
            const int64_t nvec = rb >> 4;
            for (int64_t i0 = tid + (p == 0 ? first : 0); i0 < nvec;
                 i0 += kBatchThreads * kBatchUnroll) {
                u32x4 x[kBatchUnroll];
#pragma unroll
                for (int u = 0; u < kBatchUnroll; ++u) {
                    const int64_t i = i0 + u * kBatchThreads;
                    if (i < nvec) x[u] = ld_row<MOE_EP_BATCH_LD_NT>(src + i * 16);
                }
                for (int a = 0; a < n; ++a) {
                    uint8_t* dst = P.dst[p] + s_exp[a] * P.dst_stride[p] +
                                   (int64_t)s_row[a] * rb;
#pragma unroll
                    for (int u = 0; u < kBatchUnroll; ++u) {
                        const int64_t i = i0 + u * kBatchThreads;
                        if (i < nvec) st_row<MOE_EP_BATCH_ST_NT>(dst + i * 16, x[u]);
                    }
                }
            }
        }
        __syncthreads();
    }
}

// Received expert ids for consumers that read the received slots in place:
// every entry of the [W, cap, slots] layout is written, with the local id of
// a valid pick (slot < count, id in [0, e_local)) or invalid_id. May run in
// place (out == recv_eloc with the same stride): each entry is read and
// written by one lane.
__global__ __launch_bounds__(256) void sanitize_ids_kernel(
    const int32_t* recv_cnt, int64_t cnt_stride, const int32_t* recv_eloc,
    int64_t eloc_stride, int W, int e_local, int slots, int64_t cap,
    int32_t invalid_id, int32_t* out, int64_t out_stride,
    uint32_t* __restrict__ err) {
    __shared__ int32_t pre[MOE_EP_MAX_WORLD + 1];
    if (threadIdx.x < 64) load_recv_prefix(recv_cnt, cnt_stride, W, cap, pre, err);
    __syncthreads();
    const int32_t per_rank = (int32_t)cap * slots;
    const int32_t total = W * per_rank;
    uint32_t bad = 0;
    for (int32_t idx = blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += gridDim.x * 256) {
        const int32_t s = idx / per_rank;
        const int32_t rem = idx - s * per_rank;
        const int32_t slot = rem / slots;
        int32_t v = invalid_id;
        if (slot < pre[s + 1] - pre[s]) {
            const int32_t e = recv_eloc[s * eloc_stride + rem];
            if (e >= e_local) bad |= MOE_EP_ERR_ELOC;
            if (e >= 0 && e < e_local) v = e;
        }
        out[s * out_stride + rem] = v;
    }
    report(err, bad);
}

hipError_t launch_sanitize_ids(const int32_t* recv_cnt, int64_t cnt_stride,
                               const int32_t* recv_eloc, int64_t eloc_stride,
                               int W, int e_local, int slots, int64_t cap,
                               int32_t invalid_id, int32_t* out,
                               int64_t out_stride, uint32_t* err,
                               hipStream_t stream) {
    const int64_t total = (int64_t)W * cap * slots;
    if (total == 0) return hipSuccess;
    int64_t grid = (total + 255) / 256;
    if (grid > 4096) grid = 4096;
    sanitize_ids_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(
        recv_cnt, cnt_stride, recv_eloc, eloc_stride, W, e_local, slots, cap,
        invalid_id, out, out_stride, err);
    return hipGetLastError();
}

hipError_t launch_batch_local(const int32_t* recv_cnt, int64_t cnt_stride,
                              const int32_t* recv_eloc, int64_t eloc_stride,
                              int W, int e_local, int slots, int64_t cap,
                              int ntiles, int32_t* recv_row, int32_t* tile_cnt,
                              uint32_t* err, hipStream_t stream) {
    if (ntiles == 0) return hipSuccess;
    int nbits = 0;
    while ((1 << nbits) < e_local) ++nbits;
    const size_t lds = sizeof(int16_t) * kBatchChunks * (size_t)e_local;
    batch_local_kernel<<<dim3(ntiles), dim3(256), lds, stream>>>(
        recv_cnt, cnt_stride, recv_eloc, eloc_stride, W, e_local, slots, cap,
        nbits, recv_row, tile_cnt, err);
    return hipGetLastError();
}

hipError_t launch_batch_copy(const int32_t* recv_cnt, int64_t cnt_stride,
                             const int32_t* recv_eloc, int64_t eloc_stride,
                             int W, int e_local, int slots, int64_t cap,
                             const int32_t* tile_off, const int32_t* tile_cnt,
                             int fused_tiles, const int32_t* recv_rank,
                             const int32_t* recv_ecnt, int64_t ecnt_stride,
                             int32_t* expert_num_tokens, int32_t clamp_max,
                             int32_t* recv_row, const PayloadSet& P, uint32_t* err,
                             hipStream_t stream) {
    const int64_t max_rows = (int64_t)W * cap;
    // (the ranked form also writes expert_num_tokens when nothing arrives)
    if (max_rows == 0 && recv_rank == nullptr) return hipSuccess;
    int64_t grid = max_rows < MOE_EP_ROW_GRID ? max_rows : MOE_EP_ROW_GRID;
    if (grid < 1) grid = 1;
    const bool pf = P.n == 1 && P.row_bytes[0] / 16 > MOE_EP_BATCH_PREFETCH_VECS;
    const size_t lds = recv_rank ? sizeof(int32_t) * (size_t)W * e_local : 0;
#define MOE_EP_BATCH_COPY_LAUNCH(PFV, ROWSV)                                                \
    batch_copy_kernel<PFV, ROWSV><<<dim3((unsigned)grid), dim3(kBatchThreads), lds, stream>>>( \
        recv_cnt, cnt_stride, recv_eloc, eloc_stride, W, e_local, slots, cap, tile_off,      \
        tile_cnt, fused_tiles, recv_rank, recv_ecnt, ecnt_stride, expert_num_tokens,          \
        clamp_max, recv_row, P, err)
    if (recv_rank) {
        if (pf) MOE_EP_BATCH_COPY_LAUNCH(true, kRowsRanked);
        else MOE_EP_BATCH_COPY_LAUNCH(false, kRowsRanked);
    } else if (tile_cnt) {
        if (pf) MOE_EP_BATCH_COPY_LAUNCH(true, kRowsFused);
        else MOE_EP_BATCH_COPY_LAUNCH(false, kRowsFused);
    } else {
        if (pf) MOE_EP_BATCH_COPY_LAUNCH(true, kRowsScanned);
        else MOE_EP_BATCH_COPY_LAUNCH(false, kRowsScanned);
    }
#undef MOE_EP_BATCH_COPY_LAUNCH
    return hipGetLastError();
}

}  // namespace moe_ep
