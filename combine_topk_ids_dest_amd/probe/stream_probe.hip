// HBM stream probes: plain grid-stride streams of 16-byte vector accesses
// in the read/write proportions of the path's copy kernels, without their
// index work, to measure what such streams reach on this GPU (the
// practical ceilings the copy kernels are compared with). Measurement
// tooling for `bench.py --probe stream`, built into its own library
// (libmoe_ep_probe.so); not part of the path or of its C ABI.
//
// For every vector i of [0, n): v = src[i] (^ src2[i] for i below the extra
// read), dst[i] = v (when dst is given), dst2[i] = v (for i below the extra
// write), so reads and writes come in any proportion: read-only (no dst;
// the XOR of the values goes to one word per block), write-only (no src: a
// pattern), a 1 : 1 copy, the 1 : 1.5 of the expert batch copy, the 5 : 3
// of the combine reduce. Every count is a whole number of chunks (one
// block pass: 256 lanes x 4 vectors) and each launch covers a range with
// the same parts, so no lane needs a guard and a lane's loads are all in
// flight together. Up to three launches (ranges with both extras, with
// one, with none) make one stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define PROBE_API extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kU = 4;
constexpr int64_t kChunk = (int64_t)kThreads * kU;   // vectors per block pass

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <bool NT>
__device__ __forceinline__ void st(u32x4* p, const u32x4& v) {
    if (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Vectors [lo, hi) of the stream (whole chunks). READ: v = src[i], else a
// pattern; READ2: v ^= src2[i]; WRITE: dst[i] = v, else v goes into the
// block's XOR; WRITE2: dst2[i] = v. Straight-line code: every load of a
// lane is issued before the first is used.
template <bool NT_LD, bool NT_ST, bool READ, bool READ2, bool WRITE, bool WRITE2>
__global__ __launch_bounds__(kThreads) void stream_kernel(
    const u32x4* __restrict__ src, const u32x4* __restrict__ src2, u32x4* __restrict__ dst,
    u32x4* __restrict__ dst2, int64_t lo, int64_t hi, uint32_t* __restrict__ sink) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t c = lo + (int64_t)blockIdx.x * kChunk; c < hi; c += (int64_t)gridDim.x * kChunk) {
        u32x4 v[kU], w[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = c + u * kThreads + threadIdx.x;
            v[u] = READ ? ld<NT_LD>(src + i) : u32x4{(uint32_t)i, 1u, 2u, 3u};
            if (READ2) w[u] = ld<NT_LD>(src2 + i);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = c + u * kThreads + threadIdx.x;
            if (READ2) v[u] ^= w[u];
            if (WRITE) st<NT_ST>(dst + i, v[u]);
            else acc ^= v[u];
            if (WRITE2) st<NT_ST>(dst2 + i, v[u]);
        }
    }
    if (!WRITE && threadIdx.x == 0) sink[blockIdx.x] ^= acc.x ^ acc.y ^ acc.z ^ acc.w;
}

template <bool NT_LD, bool NT_ST, bool READ, bool WRITE>
void launch_segments(const u32x4* a, const u32x4* a2, u32x4* d, u32x4* d2, int64_t n,
                     int64_t n_r2, int64_t n_w2, uint32_t* sink, int grid, hipStream_t s) {
    // [0, both extras), then [min extra, max extra) with one of them, then
    // the rest with neither
    const int64_t both = n_r2 < n_w2 ? n_r2 : n_w2;
    const int64_t more = n_r2 > n_w2 ? n_r2 : n_w2;
    if (both > 0)
        stream_kernel<NT_LD, NT_ST, READ, true, WRITE, true>
            <<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(a, a2, d, d2, 0, both, sink);
    if (more > both) {
        if (n_r2 > n_w2)
            stream_kernel<NT_LD, NT_ST, READ, true, WRITE, false>
                <<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(a, a2, d, d2, both, more, sink);
        else
            stream_kernel<NT_LD, NT_ST, READ, false, WRITE, true>
                <<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(a, a2, d, d2, both, more, sink);
    }
    if (n > more)
        stream_kernel<NT_LD, NT_ST, READ, false, WRITE, false>
            <<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(a, a2, d, d2, more, n, sink);
}

}  // namespace

// Status: 0 on success, -1 for arguments that break the rules below, -6 for
// a launch error. bytes, extra_read_bytes and extra_write_bytes are whole
// numbers of 16 KiB chunks with extra_* <= bytes; every pointer is 16-byte
// aligned; src may be null (a pattern is written), dst may be null (then
// sink [grid] is XORed with one word per block); src2 / dst2 are read /
// written over their first extra_* bytes. grid: blocks of 256 lanes
// (grid-stride).
PROBE_API int moe_ep_probe_stream(const void* src, const void* src2, int64_t bytes,
                                  int64_t extra_read_bytes, void* dst, void* dst2,
                                  int64_t extra_write_bytes, uint32_t* sink, int32_t grid,
                                  int32_t nt_load, int32_t nt_store, void* stream) {
    const int64_t chunk_bytes = kChunk * 16;
    if (bytes <= 0 || bytes % chunk_bytes || extra_read_bytes < 0 ||
        extra_read_bytes % chunk_bytes || extra_read_bytes > bytes || extra_write_bytes < 0 ||
        extra_write_bytes % chunk_bytes || extra_write_bytes > bytes || grid <= 0)
        return -1;
    if ((extra_read_bytes && (!src2 || !src)) || (extra_write_bytes && !dst2) ||
        (!dst && !sink) || (!src && !dst))
        return -1;
    const void* ptrs[] = {src, src2, dst, dst2};
    for (const void* p : ptrs)
        if (reinterpret_cast<uintptr_t>(p) % 16) return -1;
    const int64_t n = bytes / 16;
    auto s = static_cast<hipStream_t>(stream);
    const u32x4* a = static_cast<const u32x4*>(src);
    const u32x4* a2 = static_cast<const u32x4*>(src2);
    u32x4* d = static_cast<u32x4*>(dst);
    u32x4* d2 = static_cast<u32x4*>(dst2);
#define PROBE_SEGMENTS(L, S)                                                            \
    do {                                                                                \
        if (a && d) launch_segments<L, S, true, true>(a, a2, d, d2, n, n_r2, n_w2, sink, grid, s); \
        else if (a) launch_segments<L, S, true, false>(a, a2, d, d2, n, n_r2, n_w2, sink, grid, s); \
        else launch_segments<L, S, false, true>(a, a2, d, d2, n, n_r2, n_w2, sink, grid, s); \
    } while (0)
    const int64_t n_r2 = extra_read_bytes / 16, n_w2 = extra_write_bytes / 16;
    if (nt_load && nt_store) PROBE_SEGMENTS(true, true);
    else if (nt_load) PROBE_SEGMENTS(true, false);
    else if (nt_store) PROBE_SEGMENTS(false, true);
    else PROBE_SEGMENTS(false, false);
#undef PROBE_SEGMENTS
    return hipGetLastError() == hipSuccess ? 0 : -6;
}
