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
#include "common.h"

namespace moe_ep {

__global__ __launch_bounds__(kRouteTile) void route_local_kernel(
    const int32_t* __restrict__ ids, int64_t T, int K, int E, int e_local,
    int W, int32_t* __restrict__ rank, int32_t* __restrict__ tile_cnt,
    uint32_t* __restrict__ err) {
    __shared__ int32_t wave_cnt[kRouteTile / 64][MOE_EP_MAX_WORLD];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t t = (int64_t)blockIdx.x * kRouteTile + tid;

    // Destination mask of the token: bit d set when some routed pick of the
    // token lives on rank d. Negative ids are padding; ids >= E are dropped.
    uint64_t mask = 0;
    uint32_t bad = 0;
    if (t < T) mask = token_dest_mask(ids + t * K, K, E, e_local, bad);
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
}

// Exclusive prefix down the columns of cnt [ntiles][nkeys] into off, and the
// column totals (clamped to clamp_max) into total. One block of 1024 lanes:
// lane (g, key) sums a contiguous run of tiles (loads issued kScanBatch at a
// time so their latencies overlap), each lane then adds the runs of the
// groups before it from LDS, and finally writes its run's prefixes.
constexpr int kScanBatch = 16;

__host__ __device__ inline int scan_groups(int ntiles, int nkeys) {
    int groups = 1024 / nkeys;
    if (groups > 64) groups = 64;
    if (groups > ntiles) groups = ntiles > 0 ? ntiles : 1;
    return groups;
}

__global__ __launch_bounds__(1024) void column_scan_kernel(
    const int32_t* __restrict__ cnt, int ntiles, int nkeys,
    int32_t* __restrict__ off, int32_t* __restrict__ total, int32_t clamp_max) {
    extern __shared__ int32_t part[];   // [groups][nkeys]
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
            v[u] = r0 + u < hi ? cnt[(int64_t)(r0 + u) * nkeys + key] : 0;
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
            v[u] = r0 + u < hi ? cnt[(int64_t)(r0 + u) * nkeys + key] : 0;
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) {
            if (r0 + u < hi) off[(int64_t)(r0 + u) * nkeys + key] = before;
            before += v[u];
        }
    }
}

hipError_t launch_route_local(const int32_t* ids, int64_t T, int K, int E,
                              int e_local, int W, int32_t* rank,
                              int32_t* tile_cnt, uint32_t* err,
                              hipStream_t stream) {
    const int64_t ntiles = (T + kRouteTile - 1) / kRouteTile;
    if (ntiles == 0) return hipSuccess;
    route_local_kernel<<<dim3((unsigned)ntiles), dim3(kRouteTile), 0, stream>>>(
        ids, T, K, E, e_local, W, rank, tile_cnt, err);
    return hipGetLastError();
}

hipError_t launch_column_scan(const int32_t* cnt, int ntiles, int nkeys,
                              int32_t* off, int32_t* total, int32_t clamp_max,
                              hipStream_t stream) {
    const size_t lds = sizeof(int32_t) * (size_t)scan_groups(ntiles, nkeys) * nkeys + 16;
    column_scan_kernel<<<dim3(1), dim3(1024), lds, stream>>>(
        cnt, ntiles, nkeys, off, total, clamp_max);
    return hipGetLastError();
}

}  // namespace moe_ep
