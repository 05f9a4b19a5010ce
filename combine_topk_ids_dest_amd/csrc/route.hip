// Routing and slot assignment of the send side (prepare() on the vLLM
// "alltoall_batched" documentation page: padding filter, destination =
// floor(id / e_local), one slot per (destination, token) pair, slots in
// ascending token order), plus the column scan shared by the send and
// receive sides.
//
// Slot of (d, t) = number of tokens t' < t that also go to d. It is built in
// two levels without atomics, so the result does not depend on scheduling:
//   route_local: per tile of 256 tokens, a wave64 ballot per destination
//     gives each token its rank among the tile's tokens for d (kept in the
//     workspace, destination-major [W][T] so that every store of a wave is
//     contiguous); the tile's count per destination goes to the workspace.
//   tile offsets: the exclusive prefix of the tile counts per destination.
//     With at most kPackFuseTiles tiles, pack_copy sums the counts of the
//     earlier tiles itself (and block 0 writes send_cnt); otherwise
//     column_scan computes them and send_cnt.
// pack_copy adds the tile offset to the in-tile rank. With a single tile
// (T <= 256, decode-sized batches) neither kernel runs: every pack_copy
// block derives the ranks of its token from the masks of all T tokens.
//
// With the send-side per-expert ranks (RankArgs; KB > 0, the number of
// picks per token the ranking code is unrolled for): route_local also ranks
// each kept pick of the tile among the tile's kept picks of the same expert
// into prank [T * K], and writes the tile's count per expert to ecnt_tile
// [tiles][E]; the tile offsets per expert are summed by pack_copy or come
// from column_scan, like the destination ones. When no token of the tile
// holds an expert twice (distinct ids) and E <= kRankMaskE, a rank is a
// count of earlier tokens, read off per-wave token masks (mark_expert_masks);
// otherwise the general multi-split (tile_expert_ranks) runs.
#include "common.h"

namespace moe_ep {

// KB: 0 without the per-expert ranks, else the unrolled bound on K (8 or
// kRankMaxK) of the ranking code.
template <int KB>
__global__ __launch_bounds__(kRouteTile) void route_local_kernel(
    const int32_t* __restrict__ ids, int64_t T, int K, int E, int e_local,
    int W, int slots, int nbits, int32_t* __restrict__ rank,
    int32_t* __restrict__ tile_cnt, int32_t* __restrict__ prank,
    int32_t* __restrict__ ecnt_tile, uint32_t* __restrict__ err) {
    // RANKED: keys [kRouteTile * K], ranks [kRouteTile * K] and the wave
    // counts [(waves + 1) * E], all int16
    extern __shared__ int16_t rank_lds[];
    __shared__ int32_t wave_cnt[kRouteTile / 64][MOE_EP_MAX_WORLD];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t t = (int64_t)blockIdx.x * kRouteTile + tid;

    // Destination mask of the token: bit d set when some routed pick of the
    // token lives on rank d. Negative ids are padding; ids >= E are dropped.
    // With the ranks the ids stay in registers for the kept ids below (one
    // load of them instead of two).
    uint64_t mask = 0;
    uint32_t bad = 0;
    int32_t key[kRankMaxK];
    constexpr int KL = KB > 0 ? KB : 1;
    if (KB > 0) {
#pragma unroll
        for (int k = 0; k < kRankMaxK; ++k) key[k] = -1;
        if (t < T) load_row_ids<KL>(ids + t * K, K, key);
        mask = dest_mask_of<KL>(key, E, e_local, bad);
    } else if (t < T) {
        mask = token_dest_mask(ids + t * K, K, E, e_local, bad);
    }
    report(err, bad);

    for (int d = 0; d < W; ++d) {
        const uint64_t b = __ballot((mask >> d) & 1ull);
        if (lane == 0) wave_cnt[wave][d] = __popcll(b);
    }
    __syncthreads();
    // Per destination: the tile's count, and wave_cnt[w][d] becomes the
    // number of the tile's tokens for d in waves before w.
    if (tid < W) {
        int32_t run = 0;
#pragma unroll
        for (int w = 0; w < kRouteTile / 64; ++w) {
            const int32_t v = wave_cnt[w][tid];
            wave_cnt[w][tid] = run;
            run += v;
        }
        tile_cnt[(int64_t)blockIdx.x * W + tid] = run;
    }
    __syncthreads();

    for (int d = 0; d < W; ++d) {
        const uint64_t b = __ballot((mask >> d) & 1ull);
        const int32_t before = wave_cnt[wave][d];
        if (t < T)
            rank[d * T + t] = ((mask >> d) & 1ull) ? before + rank_below(b) : -1;
    }

    if (KB > 0) {
        constexpr int waves = kRouteTile / 64;
        int16_t* keys = rank_lds;
        int16_t* rnk = keys + kRouteTile * K;
        // wave counts [(waves + 1) * E] int16, or the masks [waves * E] u64
        int16_t* hist = rnk + kRouteTile * K;
        unsigned long long* masks = reinterpret_cast<unsigned long long*>(hist);
        const int64_t t0 = (int64_t)blockIdx.x * kRouteTile;
        const int ntok = T - t0 < kRouteTile ? (int)(T - t0) : kRouteTile;
        const int n = ntok * K;
        keep_keys<KB>(K, E, e_local, slots, key);
        const bool fast = E <= kRankMaskE && !__syncthreads_or(has_repeated_key<KB>(key));
        if (fast) {
            for (int i = tid; i < waves * E; i += kRouteTile) masks[i] = 0;
            __syncthreads();
            mark_expert_masks<KB>(key, masks, E);
            __syncthreads();
            // this thread's token's picks (queries unrolled, all in flight)
#pragma unroll
            for (int k = 0; k < KB; ++k)
                if (k < K && t < T)
                    prank[t * K + k] = key[k] >= 0 ? mask_rank<waves>(masks, E, tid, key[k]) : -1;
            for (int g = tid; g < E; g += kRouteTile) {
                int32_t c = 0;
                for (int w = 0; w < waves; ++w) c += __popcll(masks[w * E + g]);
                ecnt_tile[(int64_t)blockIdx.x * E + g] = c;
            }
        } else {
#pragma unroll
            for (int k = 0; k < KB; ++k)
                if (k < K && t < T) keys[tid * K + k] = (int16_t)key[k];
            for (int i = tid; i < (waves + 1) * E; i += kRouteTile) hist[i] = 0;
            __syncthreads();
            tile_expert_ranks(keys, rnk, n, K, E, nbits, hist, waves);
            for (int i = tid; i < n; i += kRouteTile) prank[t0 * K + i] = rnk[i];
            for (int g = tid; g < E; g += kRouteTile)
                ecnt_tile[(int64_t)blockIdx.x * E + g] = hist[waves * E + g];
        }
    }
}

// Exclusive prefix down the columns of cnt [ntiles][nkeys] into off, and the
// column totals (clamped to clamp_max) into total. A block of 1024 lanes per
// 1024 keys: lane (g, key) sums a contiguous run of tiles (loads issued
// kScanBatch at a time so their latencies overlap), each lane then adds the
// runs of the groups before it from LDS, and finally writes its run's
// prefixes.
constexpr int kScanBatch = 16;
constexpr int kScanKeys = 1024;

__host__ __device__ inline int scan_groups(int ntiles, int nkeys) {
    int groups = 1024 / nkeys;
    if (groups > 64) groups = 64;
    if (groups > ntiles) groups = ntiles > 0 ? ntiles : 1;
    return groups;
}

__global__ __launch_bounds__(1024) void column_scan_kernel(
    const int32_t* __restrict__ cnt, int ntiles, int nkeys_all,
    int32_t* __restrict__ off, int32_t* __restrict__ total, int32_t clamp_max) {
    extern __shared__ int32_t part[];   // [groups][nkeys]
    // this block's keys: [key0, key0 + nkeys)
    const int key0 = blockIdx.x * kScanKeys;
    const int nkeys = nkeys_all - key0 < kScanKeys ? nkeys_all - key0 : kScanKeys;
    cnt += key0;
    off += key0;
    total += key0;
    const int groups = scan_groups(ntiles, nkeys);
    const int chunk = (ntiles + groups - 1) / groups;
    const int i = threadIdx.x;
    const bool active = i < groups * nkeys;
    const int g = active ? i / nkeys : 0;
    const int key = active ? i - g * nkeys : 0;
    const int lo = g * chunk;
    const int hi = active ? min(ntiles, lo + chunk) : lo;

    int32_t run = 0;
    for (int r0 = lo; r0 < hi; r0 += kScanBatch) {
        int32_t v[kScanBatch];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u)
            v[u] = r0 + u < hi ? cnt[(int64_t)(r0 + u) * nkeys_all + key] : 0;
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) run += v[u];
    }
    if (active) part[i] = run;
    __syncthreads();
    if (!active) return;
    int32_t before = 0;
    for (int g2 = 0; g2 < g; ++g2) before += part[g2 * nkeys + key];
    if (g == groups - 1) {
        const int32_t tot = before + run;
        total[key] = tot < clamp_max ? tot : clamp_max;
    }
    for (int r0 = lo; r0 < hi; r0 += kScanBatch) {
        int32_t v[kScanBatch];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u)
            v[u] = r0 + u < hi ? cnt[(int64_t)(r0 + u) * nkeys_all + key] : 0;
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) {
            if (r0 + u < hi) off[(int64_t)(r0 + u) * nkeys_all + key] = before;
            before += v[u];
        }
    }
}

hipError_t launch_route_local(const int32_t* ids, int64_t T, int K, int E,
                              int e_local, int W, int slots, int32_t* rank,
                              int32_t* tile_cnt, int32_t* prank, int32_t* ecnt_tile,
                              int nbits, uint32_t* err, hipStream_t stream) {
    const int64_t ntiles = (T + kRouteTile - 1) / kRouteTile;
    if (ntiles == 0) return hipSuccess;
    if (prank) {
        // keys and ranks, then the wave counts or (E <= kRankMaskE) the masks
        const size_t counts = sizeof(int16_t) * (size_t)(kRouteTile / 64 + 1) * E;
        const size_t masks = E <= kRankMaskE ? sizeof(uint64_t) * (size_t)(kRouteTile / 64) * E
                                             : 0;
        const size_t lds = sizeof(int16_t) * (size_t)2 * kRouteTile * K +
                           (counts > masks ? counts : masks);
        if (K <= 8)
            route_local_kernel<8><<<dim3((unsigned)ntiles), dim3(kRouteTile), lds, stream>>>(
                ids, T, K, E, e_local, W, slots, nbits, rank, tile_cnt, prank, ecnt_tile, err);
        else
            route_local_kernel<kRankMaxK><<<dim3((unsigned)ntiles), dim3(kRouteTile), lds,
                                            stream>>>(ids, T, K, E, e_local, W, slots, nbits,
                                                      rank, tile_cnt, prank, ecnt_tile, err);
    } else {
        route_local_kernel<0><<<dim3((unsigned)ntiles), dim3(kRouteTile), 0, stream>>>(
            ids, T, K, E, e_local, W, slots, nbits, rank, tile_cnt, nullptr, nullptr, err);
    }
    return hipGetLastError();
}

hipError_t launch_column_scan(const int32_t* cnt, int ntiles, int nkeys,
                              int32_t* off, int32_t* total, int32_t clamp_max,
                              hipStream_t stream) {
    const int per = nkeys < kScanKeys ? nkeys : kScanKeys;
    const size_t lds = sizeof(int32_t) * (size_t)scan_groups(ntiles, per) * per + 16;
    const int blocks = (nkeys + kScanKeys - 1) / kScanKeys;
    column_scan_kernel<<<dim3(blocks > 0 ? blocks : 1), dim3(1024), lds, stream>>>(
        cnt, ntiles, nkeys, off, total, clamp_max);
    return hipGetLastError();
}

}  // namespace moe_ep
