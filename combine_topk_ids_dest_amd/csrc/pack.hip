// Payload and metadata pack of the send side (prepare() on the vLLM
// "alltoall_batched" documentation page: send_x[dest, slot] = row of the
// token; pick column j of the slot holds the j-th routed expert the token
// wants on that rank, in router order, as a local id with its fp32 weight;
// unused columns hold -1 and +0.0).
//
// Token-major: a token's row is read from HBM once into registers (16-byte
// vectors) and stored to every destination the token goes to (5.3 on average
// for 256 experts, top-8, 8 ranks). When there are few tokens (decode), each
// row is cut into `nsplit` column parts handled by different blocks, so the
// grid still fills the chip. In every block wave 0 turns the token's in-tile
// ranks into final slots (adding the offset of its tile, summed here from
// the tile counts when there are few tiles) and leaves the destination list
// in LDS; the block of part 0 also writes the final token_slot context and
// the pick metadata.
#include "common.h"

namespace moe_ep {

constexpr int kPackThreads = 256;
constexpr int kPackUnroll = 4;

// Sum of tile_cnt[j][d] over tiles j < tiles (loads issued 8 at a time).
__device__ __forceinline__ int32_t sum_tiles(const int32_t* __restrict__ tile_cnt,
                                             int64_t tiles, int W, int d) {
    int32_t s = 0;
    for (int64_t j0 = 0; j0 < tiles; j0 += 8) {
        int32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = j0 + u < tiles ? tile_cnt[(j0 + u) * W + d] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    return s;
}

// Quantises the vectors [lo, hi) of one bf16 row (8 columns per 16-byte
// vector) and stores codes and scales to the n destinations in LDS. Scale of
// a group = its amax / 448 (1 if amax = 0), each code = e4m3(x / scale), the
// quotient correctly rounded (__fdiv_rn), the conversion the hardware one
// (round to nearest even). lo and hi are multiples of the group's vectors,
// so the 16-byte vectors of a group sit in consecutive, aligned lanes and
// its amax is a butterfly over those lanes.
__device__ __forceinline__ void quantize_row(const QuantArgs& Q, int64_t t,
                                             int64_t lo, int64_t hi, int n,
                                             const int32_t* s_dest,
                                             const int32_t* s_slot) {
    const int gv = Q.group >> 3;                 // vectors per group
    const uint8_t* src = Q.src + t * Q.src_stride;
    for (int64_t base = lo; base < hi; base += kPackThreads * kPackUnroll) {
#pragma unroll
        for (int u = 0; u < kPackUnroll; ++u) {
            const int64_t i = base + u * kPackThreads + threadIdx.x;
            const bool valid = i < hi;
            float f[8];
            float m = 0.0f;
            if (valid) {
                const u32x4 v = ld_row<MOE_EP_COPY_NT>(src + i * 16);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    f[2 * c] = bf16_lo(v[c]);
                    f[2 * c + 1] = bf16_hi(v[c]);
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) m = fmaxf(m, fabsf(f[c]));
            }
            for (int x = 1; x < gv; x <<= 1) m = fmaxf(m, __shfl_xor(m, x, 64));
            if (!valid) continue;
            const float scale = m > 0.0f ? __fdiv_rn(m, 448.0f) : 1.0f;
            u32x2 codes;
            int lo16 = __builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(f[0], scale),
                                                       __fdiv_rn(f[1], scale), 0, false);
            codes[0] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                __fdiv_rn(f[2], scale), __fdiv_rn(f[3], scale), lo16, true);
            int hi16 = __builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(f[4], scale),
                                                       __fdiv_rn(f[5], scale), 0, false);
            codes[1] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                __fdiv_rn(f[6], scale), __fdiv_rn(f[7], scale), hi16, true);
            const bool first = (i % gv) == 0;
            for (int a = 0; a < n; ++a) {
                uint8_t* qrow = Q.q + s_dest[a] * Q.q_stride + (int64_t)s_slot[a] * Q.H;
                *reinterpret_cast<u32x2*>(qrow + i * 8) = codes;
                if (first)
                    Q.s[s_dest[a] * Q.s_stride + (int64_t)s_slot[a] * Q.s_pitch + i / gv] = scale;
            }
        }
    }
}

template <bool QUANT>
__global__ __launch_bounds__(kPackThreads) void pack_copy_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int64_t T,
    int K, int E, int e_local, int W, int slots, int64_t cap, int nsplit,
    const int32_t* __restrict__ rank, int32_t* __restrict__ token_slot,
    const int32_t* __restrict__ tile_cnt, const int32_t* __restrict__ tile_off,
    int32_t* __restrict__ send_cnt, const PayloadSet P, const QuantArgs Q,
    int32_t* __restrict__ send_eloc, float* __restrict__ send_w,
    uint32_t* __restrict__ err) {
    __shared__ int32_t s_dest[MOE_EP_MAX_WORLD];
    __shared__ int32_t s_slot[MOE_EP_MAX_WORLD];
    __shared__ int s_n;
    const int tid = threadIdx.x;

    if (tile_cnt && blockIdx.x == 0 && tid < W)
        send_cnt[tid] = sum_tiles(tile_cnt, (T + kRouteTile - 1) / kRouteTile, W, tid);

    for (int64_t b = blockIdx.x; b < T * nsplit; b += gridDim.x) {
        const int64_t t = b / nsplit;
        const int part = (int)(b - t * nsplit);
        if (tid < 64) {
            const int d = tid;
            int32_t slot = -1;
            if (d < W) {
                slot = rank[t * W + d];
                if (slot >= 0)
                    slot += tile_cnt ? sum_tiles(tile_cnt, t / kRouteTile, W, d)
                                     : tile_off[(t / kRouteTile) * W + d];
            }
            const uint64_t act = __ballot(slot >= 0);
            if (slot >= 0) {
                const int pos = rank_below(act);
                s_dest[pos] = d;
                s_slot[pos] = slot;
            }
            if (part == 0 && d < W) {
                token_slot[t * W + d] = slot;
                uint32_t bad = 0;
                if (slot >= 0) {
                    const int64_t meta = ((int64_t)d * cap + slot) * slots;
                    int j = 0;
#pragma unroll 8
                    for (int k = 0; k < K; ++k) {
                        const int32_t id = ids[t * K + k];
                        if (id < 0 || id >= E || id / e_local != d) continue;
                        if (j >= slots) { bad |= MOE_EP_ERR_PICKS; continue; }
                        send_eloc[meta + j] = id - d * e_local;
                        send_w[meta + j] = wts[t * K + k];
                        ++j;
                    }
                    for (; j < slots; ++j) {
                        send_eloc[meta + j] = -1;
                        send_w[meta + j] = 0.0f;
                    }
                }
                report(err, bad);
            }
            if (tid == 0) s_n = __popcll(act);
        }
        __syncthreads();
        const int n = s_n;

        if (QUANT) {
            const int gv = Q.group >> 3;
            const int64_t nvq = Q.H >> 3;
            int64_t per = (nvq + nsplit - 1) / nsplit;
            per = (per + gv - 1) / gv * gv;
            const int64_t lo = part * per;
            const int64_t hi = lo + per < nvq ? lo + per : nvq;
            quantize_row(Q, t, lo, hi, n, s_dest, s_slot);
            // the padding of each scale row is +0.0
            const int64_t G = Q.H / Q.group;
            if (part == 0 && tid < n)
                for (int64_t g = G; g < Q.s_pitch; ++g)
                    Q.s[s_dest[tid] * Q.s_stride + (int64_t)s_slot[tid] * Q.s_pitch + g] = 0.0f;
        }

        for (int p = 0; p < P.n; ++p) {
            const int64_t rb = P.row_bytes[p];
            const int64_t nvec = rb >> 4;
            const int64_t per = (nvec + nsplit - 1) / nsplit;
            const int64_t v_lo = part * per;
            const int64_t v_hi = v_lo + per < nvec ? v_lo + per : nvec;
            const uint8_t* src = P.src[p] + t * P.src_stride[p];
            for (int64_t i0 = v_lo + tid; i0 < v_hi; i0 += kPackThreads * kPackUnroll) {
                u32x4 v[kPackUnroll];
#pragma unroll
                for (int u = 0; u < kPackUnroll; ++u) {
                    const int64_t i = i0 + u * kPackThreads;
                    if (i < v_hi) v[u] = ld_row<MOE_EP_COPY_NT>(src + i * 16);
                }
                for (int a = 0; a < n; ++a) {
                    uint8_t* dst = P.dst[p] + s_dest[a] * P.dst_stride[p] +
                                   (int64_t)s_slot[a] * rb;
#pragma unroll
                    for (int u = 0; u < kPackUnroll; ++u) {
                        const int64_t i = i0 + u * kPackThreads;
                        if (i < v_hi) st_row<MOE_EP_COPY_NT>(dst + i * 16, v[u]);
                    }
                }
            }
        }
        __syncthreads();   // s_dest / s_slot are rewritten for the next token
    }
}

hipError_t launch_pack_copy(const int32_t* ids, const float* wts, int64_t T,
                            int K, int E, int e_local, int W, int slots,
                            int64_t cap, const int32_t* rank,
                            int32_t* token_slot, const int32_t* tile_cnt,
                            const int32_t* tile_off, int32_t* send_cnt,
                            const PayloadSet& P, const QuantArgs* quant,
                            int32_t* send_eloc, float* send_w, uint32_t* err,
                            hipStream_t stream) {
    if (T == 0) return hipSuccess;
    int64_t max_vecs = quant ? quant->H / 8 : 0;
    for (int p = 0; p < P.n; ++p)
        if (P.row_bytes[p] / 16 > max_vecs) max_vecs = P.row_bytes[p] / 16;
    const int nsplit = row_split(T, max_vecs);
    const int64_t blocks = T * nsplit;
    const int64_t grid = blocks < 65536 ? blocks : 65536;
    if (quant)
        pack_copy_kernel<true><<<dim3((unsigned)grid), dim3(kPackThreads), 0, stream>>>(
            ids, wts, T, K, E, e_local, W, slots, cap, nsplit, rank, token_slot,
            tile_cnt, tile_off, send_cnt, P, *quant, send_eloc, send_w, err);
    else
        pack_copy_kernel<false><<<dim3((unsigned)grid), dim3(kPackThreads), 0, stream>>>(
            ids, wts, T, K, E, e_local, W, slots, cap, nsplit, rank, token_slot,
            tile_cnt, tile_off, send_cnt, P, QuantArgs{}, send_eloc, send_w, err);
    return hipGetLastError();
}

}  // namespace moe_ep
