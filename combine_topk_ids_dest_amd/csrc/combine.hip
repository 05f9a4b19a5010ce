// Combine (finalize() on the vLLM "alltoall_batched" documentation page).
//
// combine_reduce, on the destination rank: for every valid received slot,
// the fp32 sum over its picks, in ascending pick order, of
// fp32(expert output row) * router weight, each product rounded to fp32
// before the add (__fmul_rn / __fadd_rn: no contraction into an FMA); the
// slot's sum is stored in the data type (bf16: round to nearest even): one
// row per (source, token) pair goes back, not one per expert.
//
// combine_unpack, on the source rank: each token's partials from the ranks
// it went to, summed in fp32 in ascending rank order from +0.0f and rounded
// once; a token that went nowhere (padding) gets +0.0.
//
// combine_unpack_fused, on a rank that is both a token's source and one of
// its destinations: the destination's reduce skips the rank's own source
// (skip_src), and the unpack computes that term from the rank's own expert
// output instead of reading it back, rounded to the data type exactly as
// the reduce would store it, in its place in the ascending rank order. The
// result is bit-identical to reduce + unpack; the local slice's partial is
// neither written nor read.
//
// All are one row (the unpack: one column part of a row when there are few
// tokens) per block with 16-byte vector lanes. Wave 0 gathers the row's
// sources (expert rows with weights, or returned partial slots) into LDS in
// summation order; every lane then streams its columns.
#include "common.h"

namespace moe_ep {

constexpr int kCombineThreads = 256;
// Vectors each lane keeps in flight per pick (VU), and picks loaded per
// group: a received slot averages 1.5 picks at 256 experts, top-8, 8 ranks,
// so the loads of several vectors are issued before any is summed. A block
// covering at most kNarrowVecs vectors of a row (8 KiB of bf16) uses VU = 2,
// which fits its part of the row in one pass with fewer registers (more
// waves per SIMD; measured 11 % faster at 8 KiB rows); wider rows use VU = 4.
constexpr int kNarrowVecs = 2 * kCombineThreads;
#ifndef MOE_EP_REDUCE_PG
#define MOE_EP_REDUCE_PG 2
#endif
#ifndef MOE_EP_UNPACK_PG
#define MOE_EP_UNPACK_PG 4
#endif

// fp32 -> bf16 by gfx950's conversion instruction (v_cvt_pk_bf16_f32, two
// values per instruction: round to nearest even, NaN kept quiet with its
// upper payload bits, the same bits as to_bf16_rne on every input), or by
// to_bf16_rne (0).
#ifndef MOE_EP_HW_BF16
#define MOE_EP_HW_BF16 1
#endif
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to bf16 (nearest even), packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    if (MOE_EP_HW_BF16) {
        const f32x2 f = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
    }
    return to_bf16_rne(lo) | (to_bf16_rne(hi) << 16);
}

struct Bf16Elems {
    static constexpr int kPerVec = 8;
    __device__ static void to_f32(const u32x4& v, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16_lo(v[i]);
            f[2 * i + 1] = bf16_hi(v[i]);
        }
    }
    __device__ static u32x4 from_f32(const float* f) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
        return v;
    }
    // the value the data type stores for x
    __device__ static float round(float x) {
        return __uint_as_float(pack_bf16x2(x, 0.0f) << 16);
    }
};

struct F32Elems {
    static constexpr int kPerVec = 4;
    __device__ static void to_f32(const u32x4& v, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
    }
    __device__ static u32x4 from_f32(const float* f) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
        return v;
    }
    __device__ static float round(float x) { return x; }
};

// out[i] = sum over a < n, in order, of (w_a *) fp32(row_a[i]) for the
// 16-byte vectors v_lo <= i < nvec of a row, accumulated from +0.0f with
// each product rounded to fp32 before the add. Row a starts at
// base + off[a] (bytes).
template <class Elems, bool WEIGHTED, int PG, int VU>
__device__ __forceinline__ void sum_rows(const uint8_t* __restrict__ base,
                                         const int64_t* off, const float* w,
                                         int n, int64_t v_lo, int64_t nvec,
                                         uint8_t* __restrict__ out) {
    constexpr int V = Elems::kPerVec;
    for (int64_t i0 = v_lo + threadIdx.x; i0 < nvec; i0 += kCombineThreads * VU) {
        float acc[VU][V];
#pragma unroll
        for (int v = 0; v < VU; ++v)
#pragma unroll
            for (int c = 0; c < V; ++c) acc[v][c] = 0.0f;
        for (int a0 = 0; a0 < n; a0 += PG) {
            u32x4 y[PG][VU];
#pragma unroll
            for (int u = 0; u < PG; ++u) {
                if (a0 + u < n) {
                    const uint8_t* row = base + off[a0 + u];
#pragma unroll
                    for (int v = 0; v < VU; ++v) {
                        const int64_t i = i0 + v * kCombineThreads;
                        if (i < nvec) y[u][v] = ld_row<MOE_EP_COMBINE_NT>(row + i * 16);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < PG; ++u) {
                if (a0 + u < n) {
                    const float wa = WEIGHTED ? w[a0 + u] : 1.0f;
#pragma unroll
                    for (int v = 0; v < VU; ++v) {
                        if (i0 + v * kCombineThreads < nvec) {
                            float f[V];
                            Elems::to_f32(y[u][v], f);
#pragma unroll
                            for (int c = 0; c < V; ++c)
                                acc[v][c] = WEIGHTED ? __fadd_rn(acc[v][c], __fmul_rn(f[c], wa))
                                                     : __fadd_rn(acc[v][c], f[c]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int v = 0; v < VU; ++v) {
            const int64_t i = i0 + v * kCombineThreads;
            if (i < nvec) st_row<MOE_EP_COMBINE_NT>(out + i * 16, Elems::from_f32(acc[v]));
        }
    }
}

template <class Elems, int ELEM_BYTES, int VU>
__global__ __launch_bounds__(kCombineThreads) void combine_reduce_kernel(
    const uint8_t* __restrict__ Y, int64_t y_expert_stride, int64_t H,
    const int32_t* __restrict__ recv_cnt, int64_t cnt_stride,
    const int32_t* __restrict__ recv_eloc, const float* __restrict__ recv_w,
    int64_t meta_stride, const int32_t* __restrict__ recv_row, int W,
    int e_local, int slots, int64_t cap, uint8_t* __restrict__ ret,
    int64_t ret_stride, int skip_src) {
    __shared__ int32_t pre[MOE_EP_MAX_WORLD + 1];
    __shared__ int64_t s_base[MOE_EP_MAX_SLOTS];   // byte offset of the row
    __shared__ float s_w[MOE_EP_MAX_SLOTS];
    __shared__ int s_n;
    const int tid = threadIdx.x;
    const int64_t nvec = (H * ELEM_BYTES) >> 4;
    const int64_t expert_cap = (int64_t)W * cap;

    // Valid slots of all sources, numbered densely through the prefix of the
    // (clamped) counts; the skipped source counts as empty.
    if (tid < 64) load_recv_prefix(recv_cnt, cnt_stride, W, cap, pre, nullptr, skip_src);
    __syncthreads();
    const int32_t S = pre[W];

    for (int32_t v = blockIdx.x; v < S; v += gridDim.x) {
        const int s = find_source(pre, W, v);
        const int32_t slot = v - pre[s];
        if (tid < 64) {
            const int j = tid;
            bool ok = false;
            int64_t base = 0;
            float w = 0.0f;
            // the slot's metadata loads are issued together
            if (j < slots) {
                const int64_t m = s * meta_stride + (int64_t)slot * slots + j;
                const int32_t row = recv_row[((int64_t)s * cap + slot) * slots + j];
                const int32_t e = recv_eloc[m];
                w = recv_w[m];
                if (row >= 0 && row < expert_cap && e >= 0 && e < e_local) {
                    ok = true;
                    base = (e * y_expert_stride + (int64_t)row * H) * ELEM_BYTES;
                }
            }
            const uint64_t act = __ballot(ok);
            if (ok) {
                const int pos = rank_below(act);
                s_base[pos] = base;
                s_w[pos] = w;
            }
            if (tid == 0) s_n = __popcll(act);
        }
        __syncthreads();
        sum_rows<Elems, true, MOE_EP_REDUCE_PG, VU>(
            Y, s_base, s_w, s_n, 0, nvec,
            ret + (s * ret_stride + (int64_t)slot * H) * ELEM_BYTES);
        __syncthreads();
    }
}

template <class Elems, int ELEM_BYTES, int VU>
__global__ __launch_bounds__(kCombineThreads) void combine_unpack_kernel(
    const uint8_t* __restrict__ back, int64_t back_stride, int64_t H,
    const int32_t* __restrict__ token_slot, int64_t T, int W, int64_t cap,
    int nsplit, uint8_t* __restrict__ out) {
    __shared__ int64_t s_base[MOE_EP_MAX_WORLD];
    __shared__ int s_n;
    const int tid = threadIdx.x;
    const int64_t row_bytes = H * ELEM_BYTES;
    const int64_t nvec = row_bytes >> 4;
    const int64_t per = (nvec + nsplit - 1) / nsplit;

    for (int64_t b = blockIdx.x; b < T * nsplit; b += gridDim.x) {
        const int64_t t = b / nsplit;
        const int64_t v_lo = (b - t * nsplit) * per;
        const int64_t v_hi = v_lo + per < nvec ? v_lo + per : nvec;
        if (tid < 64) {
            const int d = tid;
            int32_t slot = -1;
            if (d < W) slot = token_slot[t * W + d];
            if (slot >= cap) slot = -1;          // not a slot of this layout
            const uint64_t act = __ballot(slot >= 0);
            if (slot >= 0)
                s_base[rank_below(act)] = (d * back_stride + (int64_t)slot * H) * ELEM_BYTES;
            if (tid == 0) s_n = __popcll(act);
        }
        __syncthreads();
        sum_rows<Elems, false, MOE_EP_UNPACK_PG, VU>(back, s_base, nullptr, s_n, v_lo,
                                                     v_hi, out + t * row_bytes);
        __syncthreads();
    }
}

// acc[v] += (w[a] *) fp32(ptr[a][i]) for a in [0, n) in order, for the
// vectors i = i0 + v * kCombineThreads below nvec; products rounded to fp32
// before the add.
template <class Elems, bool WEIGHTED, int PG, int VU>
__device__ __forceinline__ void accumulate(float (&acc)[VU][Elems::kPerVec],
                                           const uint8_t* const* ptr,
                                           const float* w, int n, int64_t i0,
                                           int64_t nvec) {
    constexpr int V = Elems::kPerVec;
    for (int a0 = 0; a0 < n; a0 += PG) {
        u32x4 y[PG][VU];
#pragma unroll
        for (int u = 0; u < PG; ++u) {
            if (a0 + u < n) {
                const uint8_t* row = ptr[a0 + u];
#pragma unroll
                for (int v = 0; v < VU; ++v) {
                    const int64_t i = i0 + v * kCombineThreads;
                    if (i < nvec) y[u][v] = ld_row<MOE_EP_COMBINE_NT>(row + i * 16);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < PG; ++u) {
            if (a0 + u < n) {
                const float wa = WEIGHTED ? w[a0 + u] : 1.0f;
#pragma unroll
                for (int v = 0; v < VU; ++v) {
                    if (i0 + v * kCombineThreads < nvec) {
                        float f[V];
                        Elems::to_f32(y[u][v], f);
#pragma unroll
                        for (int c = 0; c < V; ++c)
                            acc[v][c] = WEIGHTED ? __fadd_rn(acc[v][c], __fmul_rn(f[c], wa))
                                                 : __fadd_rn(acc[v][c], f[c]);
                    }
                }
            }
        }
    }
}

// Entries in LDS, in summation order: the returned partials of ranks below
// self_rank, then the own expert rows of the local slot (weighted), then the
// returned partials of ranks above self_rank.
template <class Elems, int ELEM_BYTES, int VU>
__global__ __launch_bounds__(kCombineThreads) void combine_unpack_fused_kernel(
    const uint8_t* __restrict__ back, int64_t back_stride, int64_t H,
    const int32_t* __restrict__ token_slot, int64_t T, int W, int64_t cap,
    int self_rank, const uint8_t* __restrict__ Y, int64_t y_expert_stride,
    const int32_t* __restrict__ self_eloc, const float* __restrict__ self_w,
    const int32_t* __restrict__ self_row, int e_local, int slots, int nsplit,
    uint8_t* __restrict__ out) {
    constexpr int V = Elems::kPerVec;
    __shared__ const uint8_t* s_ptr[MOE_EP_MAX_WORLD + MOE_EP_MAX_SLOTS];
    __shared__ float s_w[MOE_EP_MAX_SLOTS];
    __shared__ int s_lo, s_nloc, s_n, s_local;
    const int tid = threadIdx.x;
    const int64_t row_bytes = H * ELEM_BYTES;
    const int64_t nvec = row_bytes >> 4;
    const int64_t per = (nvec + nsplit - 1) / nsplit;
    const int64_t expert_cap = (int64_t)W * cap;

    for (int64_t b = blockIdx.x; b < T * nsplit; b += gridDim.x) {
        const int64_t t = b / nsplit;
        const int64_t v_lo = (b - t * nsplit) * per;
        const int64_t v_hi = v_lo + per < nvec ? v_lo + per : nvec;
        if (tid < 64) {
            const int lane = tid;
            int32_t slot = -1;
            if (lane < W) slot = token_slot[t * W + lane];
            if (slot >= cap) slot = -1;          // not a slot of this layout
            int32_t lslot = token_slot[t * W + self_rank];
            if (lslot >= cap) lslot = -1;
            const bool remote = slot >= 0 && lane != self_rank;
            const uint64_t act = __ballot(remote);
            const int lo = __popcll(act & ((1ull << self_rank) - 1));
            // the local slot's picks, as the reduce takes them
            bool ok = false;
            const uint8_t* yrow = nullptr;
            float w = 0.0f;
            if (lslot >= 0 && lane < slots) {
                const int64_t m = (int64_t)lslot * slots + lane;
                const int32_t row = self_row[m];
                const int32_t e = self_eloc[m];
                w = self_w[m];
                if (row >= 0 && row < expert_cap && e >= 0 && e < e_local) {
                    ok = true;
                    yrow = Y + (e * y_expert_stride + (int64_t)row * H) * ELEM_BYTES;
                }
            }
            const uint64_t pk = __ballot(ok);
            const int nloc = __popcll(pk);
            if (remote)
                s_ptr[rank_below(act) + (lane > self_rank ? nloc : 0)] =
                    back + (lane * back_stride + (int64_t)slot * H) * ELEM_BYTES;
            if (ok) {
                const int pos = rank_below(pk);
                s_ptr[lo + pos] = yrow;
                s_w[pos] = w;
            }
            if (tid == 0) {
                s_lo = lo;
                s_nloc = nloc;
                s_n = __popcll(act) + nloc;
                s_local = lslot >= 0;
            }
        }
        __syncthreads();
        const int lo = s_lo, nloc = s_nloc, n = s_n;
        const bool local = s_local;
        uint8_t* dst = out + t * row_bytes;
        for (int64_t i0 = v_lo + tid; i0 < v_hi; i0 += kCombineThreads * VU) {
            float acc[VU][V];
#pragma unroll
            for (int v = 0; v < VU; ++v)
#pragma unroll
                for (int c = 0; c < V; ++c) acc[v][c] = 0.0f;
            accumulate<Elems, false, MOE_EP_UNPACK_PG, VU>(acc, s_ptr, nullptr, lo, i0, v_hi);
            if (local) {
                float loc[VU][V];
#pragma unroll
                for (int v = 0; v < VU; ++v)
#pragma unroll
                    for (int c = 0; c < V; ++c) loc[v][c] = 0.0f;
                accumulate<Elems, true, MOE_EP_REDUCE_PG, VU>(loc, s_ptr + lo, s_w, nloc, i0, v_hi);
#pragma unroll
                for (int v = 0; v < VU; ++v)
#pragma unroll
                    for (int c = 0; c < V; ++c)
                        acc[v][c] = __fadd_rn(acc[v][c], Elems::round(loc[v][c]));
            }
            accumulate<Elems, false, MOE_EP_UNPACK_PG, VU>(acc, s_ptr + lo + nloc, nullptr,
                                                        n - lo - nloc, i0, v_hi);
#pragma unroll
            for (int v = 0; v < VU; ++v) {
                const int64_t i = i0 + v * kCombineThreads;
                if (i < v_hi) st_row<MOE_EP_COMBINE_NT>(dst + i * 16, Elems::from_f32(acc[v]));
            }
        }
        __syncthreads();
    }
}

hipError_t launch_combine_reduce(const void* Y, int64_t y_expert_stride,
                                 int dtype, int64_t H, const int32_t* recv_cnt,
                                 int64_t cnt_stride, const int32_t* recv_eloc,
                                 const float* recv_w, int64_t meta_stride,
                                 const int32_t* recv_row, int W, int e_local,
                                 int slots, int64_t cap, void* ret,
                                 int64_t ret_stride, int skip_src,
                                 hipStream_t stream) {
    const int64_t max_rows = (int64_t)W * cap;
    if (max_rows == 0) return hipSuccess;
    const int64_t grid = max_rows < MOE_EP_ROW_GRID ? max_rows : MOE_EP_ROW_GRID;
    const uint8_t* y = static_cast<const uint8_t*>(Y);
    uint8_t* r = static_cast<uint8_t*>(ret);
    const bool narrow = H * (dtype == MOE_EP_BF16 ? 2 : 4) / 16 <= kNarrowVecs;
#define MOE_EP_REDUCE(E, EB, VU)                                                             \
    combine_reduce_kernel<E, EB, VU><<<dim3((unsigned)grid), dim3(kCombineThreads), 0, stream>>>( \
        y, y_expert_stride, H, recv_cnt, cnt_stride, recv_eloc, recv_w, meta_stride,         \
        recv_row, W, e_local, slots, cap, r, ret_stride, skip_src)
    if (dtype == MOE_EP_BF16) {
        if (narrow) MOE_EP_REDUCE(Bf16Elems, 2, 2); else MOE_EP_REDUCE(Bf16Elems, 2, 4);
    } else {
        if (narrow) MOE_EP_REDUCE(F32Elems, 4, 2); else MOE_EP_REDUCE(F32Elems, 4, 4);
    }
#undef MOE_EP_REDUCE
    return hipGetLastError();
}

hipError_t launch_combine_unpack(const void* back, int64_t back_stride,
                                 int dtype, int64_t H,
                                 const int32_t* token_slot, int64_t T, int W,
                                 int64_t cap, void* out, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int eb = dtype == MOE_EP_BF16 ? 2 : 4;
    const int nsplit = row_split(T, H * eb / 16);
    const int64_t blocks = T * nsplit;
    const int64_t grid = blocks < 65536 ? blocks : 65536;
    const uint8_t* b = static_cast<const uint8_t*>(back);
    uint8_t* o = static_cast<uint8_t*>(out);
    const int64_t nvec = H * eb / 16;
    const bool narrow = (nvec + nsplit - 1) / nsplit <= kNarrowVecs;
#define MOE_EP_UNPACK(E, EB, VU)                                                             \
    combine_unpack_kernel<E, EB, VU><<<dim3((unsigned)grid), dim3(kCombineThreads), 0, stream>>>( \
        b, back_stride, H, token_slot, T, W, cap, nsplit, o)
    if (dtype == MOE_EP_BF16) {
        if (narrow) MOE_EP_UNPACK(Bf16Elems, 2, 2); else MOE_EP_UNPACK(Bf16Elems, 2, 4);
    } else {
        if (narrow) MOE_EP_UNPACK(F32Elems, 4, 2); else MOE_EP_UNPACK(F32Elems, 4, 4);
    }
#undef MOE_EP_UNPACK
    return hipGetLastError();
}

hipError_t launch_combine_unpack_fused(
    const void* back, int64_t back_stride, int dtype, int64_t H,
    const int32_t* token_slot, int64_t T, int W, int64_t cap, int self_rank,
    const void* Y, int64_t y_expert_stride, const int32_t* self_eloc,
    const float* self_w, const int32_t* self_row, int e_local, int slots,
    void* out, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int eb = dtype == MOE_EP_BF16 ? 2 : 4;
    const int nsplit = row_split(T, H * eb / 16);
    const int64_t blocks = T * nsplit;
    const int64_t grid = blocks < 65536 ? blocks : 65536;
    const uint8_t* b = static_cast<const uint8_t*>(back);
    const uint8_t* y = static_cast<const uint8_t*>(Y);
    uint8_t* o = static_cast<uint8_t*>(out);
    const int64_t nvec = H * eb / 16;
    const bool narrow = (nvec + nsplit - 1) / nsplit <= kNarrowVecs;
#define MOE_EP_FUSED(E, EB, VU)                                                              \
    combine_unpack_fused_kernel<E, EB, VU><<<dim3((unsigned)grid), dim3(kCombineThreads), 0,  \
                                             stream>>>(                                      \
        b, back_stride, H, token_slot, T, W, cap, self_rank, y, y_expert_stride, self_eloc,  \
        self_w, self_row, e_local, slots, nsplit, o)
    if (dtype == MOE_EP_BF16) {
        if (narrow) MOE_EP_FUSED(Bf16Elems, 2, 2); else MOE_EP_FUSED(Bf16Elems, 2, 4);
    } else {
        if (narrow) MOE_EP_FUSED(F32Elems, 4, 2); else MOE_EP_FUSED(F32Elems, 4, 4);
    }
#undef MOE_EP_FUSED
    return hipGetLastError();
}

}  // namespace moe_ep
