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
// in LDS; the block of part 0 also writes the final token_slot context and,
// after its share of the copy, the pick metadata. With at most one tile of
// tokens (T <= 256) no routing kernel runs: every block derives the in-tile
// ranks of its token from the destination masks of all T tokens.
#include "common.h"

namespace moe_ep {

#ifndef MOE_EP_PACK_THREADS
#define MOE_EP_PACK_THREADS 256
#endif
#ifndef MOE_EP_PACK_UNROLL
#define MOE_EP_PACK_UNROLL 4
#endif
constexpr int kPackThreads = MOE_EP_PACK_THREADS;
constexpr int kPackUnroll = MOE_EP_PACK_UNROLL;
// Leading rows above this many 16-byte vectors load their first pass early.
constexpr int64_t kPackPrefetchVecs = 512;
static_assert(kPackThreads >= kRouteTile, "own routing holds one tile of masks");

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

// Maximum over aligned groups of `lanes` lanes (2, 4, 8 or 16 lanes of a
// DPP row), by lane swaps within the row.
__device__ __forceinline__ float group_max(float m, int lanes) {
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(
                     0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));   // quad [1,0,3,2]
    if (lanes >= 4)
        m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(
                         0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));   // quad [2,3,0,1]
    if (lanes >= 8)
        m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(
                         0, __float_as_int(m), 0x141, 0xF, 0xF, false)));  // half mirror
    if (lanes >= 16)
        m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(
                         0, __float_as_int(m), 0x140, 0xF, 0xF, false)));  // row mirror
    return m;
}

#ifndef MOE_EP_QUANT_UNROLL
#define MOE_EP_QUANT_UNROLL 1
#endif
constexpr int kQU = MOE_EP_QUANT_UNROLL;

// fp32(x / s) for the reciprocal rd = 1 / s rounded to fp64. x * rd in
// fp64 is within 2^-52 (relative) of x / s, while the quotient of two
// binary32 numbers is never a binary32 midpoint and lies at least 2^-49
// (relative) away from every midpoint; so rounding the fp64 product to
// binary32 gives the correctly rounded quotient, for one fp64 multiply per
// element instead of a division.
__device__ __forceinline__ float div_by(float x, double rd) {
    return (float)((double)x * rd);
}

// One pass of the quantiser over a bf16 row. A lane unit i covers the 16
// columns 16i .. 16i+15 (two 16-byte loads of bf16, one 16-byte store of
// codes); the lane's units are i = base + u*kPackThreads + tid, u < kQU,
// below hi. For a group with amax > 0 the scale is s = amax / 448 and each
// code is e4m3(x / s) (the division correctly rounded to fp32, div_by,
// then the hardware conversion to nearest even); s = 1 when amax = 0.
// base and hi are multiples of the group's
// units, so a group's units sit in consecutive, aligned lanes and its amax
// is a reduction within a DPP row. The row's loads are all issued first.
// NaN entries never become the amax (a compare-and-select, not fmaxf,
// whose result for a signaling NaN is NaN), and each code carries the sign
// bit of its input: the sign of a NaN product is left open by IEEE 754.
struct QuantPass {
    u32x4 codes[kQU];
    float scale[kQU];
};

// max(m, |x|) where a NaN x leaves m as it is
__device__ __forceinline__ float abs_max(float m, float x) {
    const float a = fabsf(x);
    return a > m ? a : m;
}

__device__ __forceinline__ void quantize_pass(const uint8_t* __restrict__ src,
                                              int64_t base, int64_t hi, int gu,
                                              QuantPass& out) {
    u32x4 v[kQU][2];
#pragma unroll
    for (int u = 0; u < kQU; ++u) {
        const int64_t i = base + u * kPackThreads + threadIdx.x;
        if (i < hi) {
            v[u][0] = ld_row<MOE_EP_PACK_LD_NT>(src + i * 32);
            v[u][1] = ld_row<MOE_EP_PACK_LD_NT>(src + i * 32 + 16);
        }
    }
#pragma unroll
    for (int u = 0; u < kQU; ++u) {
        const int64_t i = base + u * kPackThreads + threadIdx.x;
        float f[16];
        float m = 0.0f;
        if (i < hi) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    f[8 * h + 2 * c] = bf16_lo(v[u][h][c]);
                    f[8 * h + 2 * c + 1] = bf16_hi(v[u][h][c]);
                }
#pragma unroll
            for (int c = 0; c < 16; ++c) m = abs_max(m, f[c]);
        }
        m = group_max(m, gu);
        const float s = m > 0.0f ? __fdiv_rn(m, 448.0f) : 1.0f;
        out.scale[u] = s;
        // an infinite amax gives rd = 0: finite x -> 0, infinite x -> NaN,
        // as x / s would
        const double rd = 1.0 / (double)s;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int lo16 = __builtin_amdgcn_cvt_pk_fp8_f32(
                div_by(f[4 * w], rd), div_by(f[4 * w + 1], rd), 0, false);
            const uint32_t codes = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                div_by(f[4 * w + 2], rd), div_by(f[4 * w + 3], rd), lo16, true);
            const uint32_t signs = ((__float_as_uint(f[4 * w]) >> 24) & 0x80u) |
                                   ((__float_as_uint(f[4 * w + 1]) >> 16) & 0x8000u) |
                                   ((__float_as_uint(f[4 * w + 2]) >> 8) & 0x800000u) |
                                   (__float_as_uint(f[4 * w + 3]) & 0x80000000u);
            out.codes[u][w] = (codes & 0x7F7F7F7Fu) | signs;
        }
    }
}

// 4-bit pass: a lane unit i covers columns 16i .. 16i+15, which are one
// scale block. amax is lane-local (NaN entries skipped, as above); the
// scale code is the hardware OCP e4m3 conversion of amax / 6 (correctly
// rounded division, then nearest even, saturating at 448); with s its
// value each code is the E2M1 code of fp32(x / s) (div_by with
// rd = 1 / s), or a zero of x's sign when s = 0 (rd = 0).
struct Fp4Pass {
    u32x2 codes[kQU];
    uint32_t scale[kQU];
};

// Value of a non-negative OCP e4m3 code below 0x7F (exact).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    const uint32_t e = c >> 3, f = c & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (f << 20)) : (float)f * 0x1p-9f;
}

// OCP E2M1 code of y: the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 by
// counting the midpoints below |y| (a midpoint counts when |y| passes it,
// or reaches it where the upper neighbour's code is even: ties to even),
// saturating at 6 (a NaN counts none); the sign bit is x's, the input that
// y was scaled from.
__device__ __forceinline__ uint32_t e2m1_code(float y, float x) {
    const float a = fabsf(y);
    const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) +
                       (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
                       (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
    return c | ((__float_as_uint(x) >> 28) & 8u);
}

// The E2M1 codes of fp32(x[c] / s) for 8 values, two per byte (x[0] in the
// low nibble of byte 0). gfx950's pair conversion (v_cvt_scalef32_pk_fp4_f32,
// scale 1) rounds to nearest even and saturates at 6 like e2m1_code, but
// turns a NaN into the largest code; a NaN quotient is therefore replaced
// by a zero with x's sign first, which gives e2m1_code's result on every
// input. (0: e2m1_code for each value.)
#ifndef MOE_EP_HW_FP4
#define MOE_EP_HW_FP4 1
#endif
// fp32(x / s) (x * 0 when s = 0), or a zero with x's sign when that is NaN
__device__ __forceinline__ float scaled_or_zero(float x, double rd) {
    const float y = div_by(x, rd);
    return y == y ? y : __uint_as_float(__float_as_uint(x) & 0x80000000u);
}

// byte SEL of word <- the codes of the pair (x[2*SEL], x[2*SEL+1])
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t word, const float* x, double rd) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
        word, scaled_or_zero(x[2 * SEL], rd), scaled_or_zero(x[2 * SEL + 1], rd), 1.0f, SEL);
}

__device__ __forceinline__ uint32_t e2m1_word(const float* x, double rd) {
    uint32_t word = 0;
    if (MOE_EP_HW_FP4) {
        word = e2m1_pair<0>(word, x, rd);
        word = e2m1_pair<1>(word, x, rd);
        word = e2m1_pair<2>(word, x, rd);
        word = e2m1_pair<3>(word, x, rd);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) word |= e2m1_code(div_by(x[c], rd), x[c]) << (4 * c);
    }
    return word;
}

__device__ __forceinline__ void quantize_pass_fp4(const uint8_t* __restrict__ src,
                                                  int64_t base, int64_t hi,
                                                  Fp4Pass& out) {
    u32x4 v[kQU][2];
#pragma unroll
    for (int u = 0; u < kQU; ++u) {
        const int64_t i = base + u * kPackThreads + threadIdx.x;
        if (i < hi) {
            v[u][0] = ld_row<MOE_EP_PACK_LD_NT>(src + i * 32);
            v[u][1] = ld_row<MOE_EP_PACK_LD_NT>(src + i * 32 + 16);
        }
    }
#pragma unroll
    for (int u = 0; u < kQU; ++u) {
        const int64_t i = base + u * kPackThreads + threadIdx.x;
        if (i >= hi) continue;
        float f[16];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                f[8 * h + 2 * c] = bf16_lo(v[u][h][c]);
                f[8 * h + 2 * c + 1] = bf16_hi(v[u][h][c]);
            }
        float m = 0.0f;
#pragma unroll
        for (int c = 0; c < 16; ++c) m = abs_max(m, f[c]);
        // amax / 6 at or above 448 saturates to 448 (also for an infinite
        // amax): the conversion sees at most 448
        const uint32_t s8 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                                fminf(__fdiv_rn(m, 6.0f), 448.0f), 0.0f, 0, false) & 0xFFu;
        const float sv = e4m3_value(s8);
        const double rd = sv > 0.0f ? 1.0 / (double)sv : 0.0;
        out.scale[u] = s8;
        out.codes[u][0] = e2m1_word(f, rd);
        out.codes[u][1] = e2m1_word(f + 8, rd);
    }
}

__device__ __forceinline__ void store_quant_pass_fp4(const QuantArgs& Q, int64_t base,
                                                     int64_t hi, const Fp4Pass& qp,
                                                     int n, const int32_t* s_dest,
                                                     const int32_t* s_slot) {
    for (int a = 0; a < n; ++a) {
        uint8_t* qrow = Q.q + s_dest[a] * Q.q_stride + (int64_t)s_slot[a] * (Q.H >> 1);
        uint8_t* srow = Q.s + s_dest[a] * Q.s_stride + (int64_t)s_slot[a] * Q.s_pitch;
#pragma unroll
        for (int u = 0; u < kQU; ++u) {
            const int64_t i = base + u * kPackThreads + threadIdx.x;
            if (i < hi) {
                *reinterpret_cast<u32x2*>(qrow + i * 8) = qp.codes[u];
                srow[i] = (uint8_t)qp.scale[u];
            }
        }
    }
}

__device__ __forceinline__ void store_quant_pass(const QuantArgs& Q, int64_t base,
                                                 int64_t hi, int gu,
                                                 const QuantPass& qp, int n,
                                                 const int32_t* s_dest,
                                                 const int32_t* s_slot) {
    for (int a = 0; a < n; ++a) {
        uint8_t* qrow = Q.q + s_dest[a] * Q.q_stride + (int64_t)s_slot[a] * Q.H;
        float* srow = reinterpret_cast<float*>(Q.s + s_dest[a] * Q.s_stride +
                                               (int64_t)s_slot[a] * Q.s_pitch);
#pragma unroll
        for (int u = 0; u < kQU; ++u) {
            const int64_t i = base + u * kPackThreads + threadIdx.x;
            if (i < hi) {
                st_row<MOE_EP_PACK_ST_NT>(qrow + i * 16, qp.codes[u]);
                if ((i % gu) == 0) srow[i / gu] = qp.scale[u];
            }
        }
    }
}

// The first pass (kPackThreads * kPackUnroll vectors) of block item b's
// column part of the leading payload row, into registers.
__device__ __forceinline__ void load_first_pass(const PayloadSet& P, int64_t b, int nsplit,
                                                u32x4 (&pre)[kPackUnroll], int64_t& p_mid) {
    const int64_t t = b / nsplit;
    const int part = (int)(b - t * nsplit);
    const int64_t nvec = P.row_bytes[0] >> 4;
    const int64_t per = (nvec + nsplit - 1) / nsplit;
    const int64_t p_lo = part * per;
    const int64_t p_hi = p_lo + per < nvec ? p_lo + per : nvec;
    p_mid = p_lo + kPackThreads * kPackUnroll < p_hi ? p_lo + kPackThreads * kPackUnroll : p_hi;
    const uint8_t* src = P.src[0] + t * P.src_stride[0];
#pragma unroll
    for (int u = 0; u < kPackUnroll; ++u) {
        const int64_t i = p_lo + u * kPackThreads + (int64_t)threadIdx.x;
        if (i < p_mid) pre[u] = ld_row<MOE_EP_PACK_LD_NT>(src + i * 16);
    }
}

// The rank of kept pick k (router order) of token t among the source's kept
// picks of its expert g, from the routing kernel: its rank within its tile
// plus the tile's offset for g (from column_scan, or the sum of the earlier
// tiles' counts, loads issued 8 at a time); -1 for a pick that is not kept.
__device__ __forceinline__ int32_t source_rank(const int32_t* __restrict__ ids, int64_t t,
                                               int K, int k, int E, const RankArgs& R) {
    // the id and the in-tile rank are loaded together
    const int32_t g = ids[t * K + k];
    const int32_t in_tile = R.prank[t * K + k];
    if (in_tile < 0) return -1;
    const int64_t tile = t / kRouteTile;
    if (R.eoff_tile) return in_tile + R.eoff_tile[tile * E + g];
    int32_t off = 0;
    for (int64_t j0 = 0; j0 < tile; j0 += 8) {
        int32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = j0 + u < tile ? R.ecnt_tile[(j0 + u) * E + g] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) off += v[u];
    }
    return in_tile + off;
}

// Pick metadata of token t for destination d: the local id and weight of
// each of its picks on d in router order, then -1 / +0.0 up to `slots`.
// Ids and weights are read 8 picks at a time, all 16 loads in flight before
// the first is used. RANKED: also each kept pick's rank among the source's
// kept picks of its expert (-1 for unused columns), which the block put in
// s_prank[k] (router order) while it planned the slots.
template <bool RANKED>
__device__ __forceinline__ uint32_t write_pick_meta(const int32_t* __restrict__ ids,
                                                    const float* __restrict__ wts, int64_t t,
                                                    int K, int E, int e_local, int d, int slots,
                                                    int32_t* eloc, float* w, int32_t* rk,
                                                    const int32_t* s_prank) {
    uint32_t bad = 0;
    int j = 0;
    for (int k0 = 0; k0 < K; k0 += 8) {
        int32_t id8[8];
        float w8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            id8[u] = k0 + u < K ? ids[t * K + k0 + u] : -1;
            w8[u] = k0 + u < K ? wts[t * K + k0 + u] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int32_t id = id8[u];
            if (id < 0 || id >= E || (uint32_t)id / (uint32_t)e_local != (uint32_t)d) continue;
            if (j >= slots) { bad |= MOE_EP_ERR_PICKS; continue; }
            eloc[j] = id - d * e_local;
            w[j] = w8[u];
            if (RANKED) rk[j] = s_prank[k0 + u];
            ++j;
        }
    }
    for (; j < slots; ++j) {
        eloc[j] = -1;
        w[j] = 0.0f;
        if (RANKED) rk[j] = -1;
    }
    return bad;
}

// Per-expert counts per block with the kernel's own routing: block b
// counts experts [b * r, b * r + r) when r = ceil(E / blocks) is at most
// this; otherwise block 0 counts them all with LDS atomics.
constexpr int kEcntPerBlock = 4;

// With the kernel's own routing (T at most one tile; thread i < T holds
// token i, whose kept ids are key; lanes past T hold none): the partial
// ranks of token t's kept picks among the source's kept picks of the same
// expert, in (token, router order). For kept pick k of t (kept id q[k]),
// the wave counts the kept picks of its tokens with that expert: all of a
// token's picks when the token is before t, those in columns before k for
// t itself. One ballot per pair (k, k2) of t's pick and a token's column,
// masked to the lanes whose tokens count, gives the wave's share; lane 0
// writes it to s_part[wave][k]. Also the wave's kept picks of experts
// ge .. ge + ne - 1 (none when ne = 0) into s_epart[wave][j]. KB: the
// unrolled bound on K (8 or kRankMaxK). Every lane of the block takes part
// (the ballots).
template <int KB>
__device__ __forceinline__ void own_route_counts(const int32_t (&key)[kRankMaxK],
                                                 const int32_t* q, int K, int64_t t,
                                                 int32_t (*s_part)[kRankMaxK], int ge,
                                                 int ne,
                                                 int32_t (*s_epart)[kEcntPerBlock]) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint64_t upto = __ballot(tid <= t);   // tokens up to t
    const uint64_t before = __ballot(tid < t);  // tokens before t
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        if (k < K) {   // K is the same in every lane
            const int32_t g = q[k];
            int32_t sum = 0;
            if (g >= 0) {
#pragma unroll
                for (int k2 = 0; k2 < KB; ++k2)
                    if (k2 < K)
                        sum += __popcll(__ballot(key[k2] == g) & (k2 < k ? upto : before));
            }
            if (lane == 0) s_part[wave][k] = sum;
        }
    }
    for (int j = 0; j < ne; ++j) {
        const int32_t g = ge + j;
        int32_t sum = 0;
#pragma unroll
        for (int k2 = 0; k2 < KB; ++k2)
            if (k2 < K) sum += __popcll(__ballot(key[k2] == g));
        if (lane == 0) s_epart[wave][j] = sum;
    }
}

// QMODE 0: plain rows; 1: payload 0 quantised to fp8; 2: to fp4.
// PF (plain rows): the first pass of the leading row of the block's first
// item is loaded before the routing and the slot planning, so its latency
// overlaps them. RANKED: the send-side per-expert ranks (RankArgs) as well,
// 1 with the routing kernel's in-tile ranks, 2 with the kernel's own routing
// (its own instantiation, so that the counting code does not raise the
// register count of the other forms).
// The token's kept picks get their ranks among the source's kept picks of
// the same expert, into s_prank: with the routing kernel, wave 1 adds the
// tile offsets to its in-tile ranks while wave 0 plans the slots; with the
// kernel's own routing the block counts them with its routing
// (own_route_counts), and the blocks write the per-expert counts.
template <int QMODE, bool PF, int RANKED>
__global__ __launch_bounds__(kPackThreads) void pack_copy_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int64_t T,
    int K, int E, int e_local, int W, int slots, int64_t cap, int nsplit,
    const int32_t* __restrict__ rank, int32_t* __restrict__ token_slot,
    const int32_t* __restrict__ tile_cnt, const int32_t* __restrict__ tile_off,
    int32_t* __restrict__ send_cnt, const PayloadSet P, const QuantArgs Q,
    int32_t* __restrict__ send_eloc, float* __restrict__ send_w, int64_t meta_stride,
    const RankArgs R, uint32_t* __restrict__ err) {
    // RANKED with own routing: block 0's per-expert counts [E]
    extern __shared__ int32_t rank_lds[];
    __shared__ int32_t s_prank[kRankMaxK];
    __shared__ int32_t s_part[RANKED == 2 ? kPackThreads / 64 : 1][kRankMaxK];
    __shared__ int32_t s_epart[RANKED == 2 ? kPackThreads / 64 : 1][kEcntPerBlock];
    __shared__ __align__(16) int32_t s_q[kRankMaxK];
    __shared__ int32_t s_dest[MOE_EP_MAX_WORLD];
    __shared__ int32_t s_slot[MOE_EP_MAX_WORLD];
    __shared__ int s_n;
    // Own routing (rank == nullptr, at most one tile of tokens): every
    // block derives the destination masks of all T tokens; wave w keeps, per
    // destination d, the ballot of its 64 tokens that go to d.
    __shared__ uint64_t s_bits[kPackThreads / 64][MOE_EP_MAX_WORLD];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bool own_route = rank == nullptr;

    u32x4 pre[kPackUnroll];
    int64_t p_mid = 0;
    if (PF && blockIdx.x < T * nsplit) load_first_pass(P, blockIdx.x, nsplit, pre, p_mid);

    if (tile_cnt && blockIdx.x == 0 && tid < W)
        send_cnt[tid] = sum_tiles(tile_cnt, (T + kRouteTile - 1) / kRouteTile, W, tid);

    if (own_route) {
        uint64_t mask = 0;
        uint32_t bad = 0;
        // RANKED: the token's ids, loaded once for its routing and its kept
        // ids; the thread of the block's token (one item per block) shares
        // them through s_q
        int32_t key[kRankMaxK];
        if (RANKED == 2) {
#pragma unroll
            for (int k = 0; k < kRankMaxK; ++k) key[k] = -1;
            if (K <= 8) {
                if (tid < T) load_row_ids<8>(ids + (int64_t)tid * K, K, key);
                mask = dest_mask_of<8>(key, E, e_local, bad);
                keep_keys<8>(K, E, e_local, slots, key);
            } else {
                if (tid < T) load_row_ids(ids + (int64_t)tid * K, K, key);
                mask = dest_mask_of(key, E, e_local, bad);
                keep_keys(K, E, e_local, slots, key);
            }
            if (tid == (int64_t)blockIdx.x / nsplit) {
#pragma unroll
                for (int k = 0; k < kRankMaxK; ++k) s_q[k] = key[k];
            }
            if (blockIdx.x == 0 && (E + gridDim.x - 1) / gridDim.x > kEcntPerBlock)
                for (int g = tid; g < E; g += kPackThreads) rank_lds[g] = 0;
        } else if (tid < T) {
            mask = token_dest_mask(ids + (int64_t)tid * K, K, E, e_local, bad);
        }
        if (blockIdx.x == 0) report(err, bad);
        if (wave * 64 < T) {   // the waves that hold tokens
            uint64_t mine = 0;
            for (int d = 0; d < W; ++d) {
                const uint64_t bl = __ballot((mask >> d) & 1ull);
                if (lane == d) mine = bl;
            }
            if (lane < W) s_bits[wave][lane] = mine;
        }
        __syncthreads();
        if (blockIdx.x == 0 && tid < W) {
            int32_t c = 0;
            for (int w = 0; w * 64 < T; ++w) c += __popcll(s_bits[w][tid]);
            send_cnt[tid] = c;
        }
        // RANKED: the partial ranks of the block's picks (summed over the
        // waves by wave 1 in the slot phase) and the per-expert counts
        const int ecnt_r = RANKED == 2 ? (E + (int)gridDim.x - 1) / (int)gridDim.x : 0;
        const int ecnt_g = (int)blockIdx.x * ecnt_r;
        if (RANKED == 2) {
            const int64_t t0 = (int64_t)blockIdx.x / nsplit;
            int32_t q[kRankMaxK];
#pragma unroll
            for (int k = 0; k < kRankMaxK; k += 4) {
                const int4 v = *reinterpret_cast<const int4*>(s_q + k);
                q[k] = v.x; q[k + 1] = v.y; q[k + 2] = v.z; q[k + 3] = v.w;
            }
            const bool spread = ecnt_r <= kEcntPerBlock;
            const int ne = !spread ? 0 : ecnt_g + ecnt_r <= E ? ecnt_r
                         : ecnt_g < E ? E - ecnt_g : 0;
            if (K <= 8) own_route_counts<8>(key, q, K, t0, s_part, ecnt_g, ne, s_epart);
            else own_route_counts<kRankMaxK>(key, q, K, t0, s_part, ecnt_g, ne, s_epart);
            if (!spread && blockIdx.x == 0) {
#pragma unroll
                for (int k = 0; k < kRankMaxK; ++k)
                    if (key[k] >= 0) atomicAdd(&rank_lds[key[k]], 1);
            }
        }
        // (a barrier here also keeps the compiler from carrying prologue
        // values into the token loop, which costs registers)
        __syncthreads();
        if (RANKED == 2) {
            if (ecnt_r <= kEcntPerBlock) {
                if (tid < ecnt_r && ecnt_g + tid < E) {
                    int32_t c = 0;
#pragma unroll
                    for (int w = 0; w < kPackThreads / 64; ++w) c += s_epart[w][tid];
                    R.send_ecnt[ecnt_g + tid] = c;
                }
            } else if (blockIdx.x == 0) {
                for (int g = tid; g < E; g += kPackThreads) R.send_ecnt[g] = rank_lds[g];
            }
        }
    } else if (RANKED == 1 && blockIdx.x == 0 && R.eoff_tile == nullptr) {
        // per-expert totals from the tile counts (column_scan writes them
        // when it computes the tile offsets)
        const int64_t tiles = (T + kRouteTile - 1) / kRouteTile;
        for (int g = tid; g < E; g += kPackThreads) {
            int32_t c = 0;
            for (int64_t j = 0; j < tiles; ++j) c += R.ecnt_tile[j * E + g];
            R.send_ecnt[g] = c;
        }
    }

    for (int64_t b = blockIdx.x; b < T * nsplit; b += gridDim.x) {
        const int64_t t = b / nsplit;
        const int part = (int)(b - t * nsplit);

        // The first pass over the leading row does not depend on where the
        // token goes: its loads (and, for the quantised row, its codes) are
        // issued before the destinations are known, so their latency
        // overlaps wave 0's slot work. (PF: the first item's loads were
        // issued before the routing.)
        int64_t q_lo = 0, q_hi = 0, q_mid = 0;
        int gv = 0;
        QuantPass qp;
        Fp4Pass qp4;
        if (QMODE != 0) {
            gv = QMODE == 2 ? 1 : Q.group >> 4;   // 16-column units per group
            const int64_t nvq = Q.H >> 4;
            int64_t per = (nvq + nsplit - 1) / nsplit;
            per = (per + gv - 1) / gv * gv;
            q_lo = part * per;
            q_hi = q_lo + per < nvq ? q_lo + per : nvq;
            q_mid = q_lo + kPackThreads * kQU < q_hi ? q_lo + kPackThreads * kQU : q_hi;
            if (q_lo < q_hi) {
                if (QMODE == 2) quantize_pass_fp4(Q.src + t * Q.src_stride, q_lo, q_mid, qp4);
                else quantize_pass(Q.src + t * Q.src_stride, q_lo, q_mid, gv, qp);
            }
        }
        // PF: the block's first item has its first pass in registers (with
        // own routing every block has a single item)
        const bool pf_item = PF && b == blockIdx.x;

        // Wave 0: the token's final slot per destination (lane d), and the
        // list of its destinations in LDS for the copy.
        int32_t slot = -1;
        if (tid < 64) {
            const int d = tid;
            if (d < W) {
                if (own_route) {
                    // tokens before t that go to d: whole waves, then the
                    // lanes below t's in its own wave
                    const int tw = (int)(t >> 6);
                    const int tb = (int)(t & 63);
                    const uint64_t bits = s_bits[tw][d];
                    if ((bits >> tb) & 1ull) {
                        slot = __popcll(bits & ((1ull << tb) - 1ull));
                        for (int w = 0; w < tw; ++w) slot += __popcll(s_bits[w][d]);
                    }
                } else {
                    // the tile offset does not depend on the rank: both
                    // loads are in flight together
                    const int32_t r = rank[d * T + t];
                    const int32_t off = tile_cnt ? sum_tiles(tile_cnt, t / kRouteTile, W, d)
                                                 : tile_off[(t / kRouteTile) * W + d];
                    slot = r >= 0 ? r + off : -1;
                }
                if (part == 0) token_slot[t * W + d] = slot;
            }
            const uint64_t act = __ballot(slot >= 0);
            if (slot >= 0) {
                const int pos = rank_below(act);
                s_dest[pos] = d;
                s_slot[pos] = slot;
            }
            if (tid == 0) s_n = __popcll(act);
        } else if (RANKED == 1 && !own_route && part == 0 && tid - 64 < K) {
            // wave 1, lane k: pick k's rank, in parallel with wave 0's slots
            s_prank[tid - 64] = source_rank(ids, t, K, tid - 64, E, R);
        } else if (RANKED == 2 && part == 0 && tid - 64 < K) {
            int32_t r = 0;
#pragma unroll
            for (int w = 0; w < kPackThreads / 64; ++w) r += s_part[w][tid - 64];
            s_prank[tid - 64] = r;   // read only for kept picks
        }
        __syncthreads();
        const int n = s_n;


        if (QMODE == 1) {
            if (q_lo < q_hi) store_quant_pass(Q, q_lo, q_mid, gv, qp, n, s_dest, s_slot);
            const uint8_t* src = Q.src + t * Q.src_stride;
            for (int64_t base = q_mid; base < q_hi; base += kPackThreads * kQU) {
                const int64_t top = base + kPackThreads * kQU < q_hi ? base + kPackThreads * kQU
                                                                     : q_hi;
                QuantPass more;
                quantize_pass(src, base, top, gv, more);
                store_quant_pass(Q, base, top, gv, more, n, s_dest, s_slot);
            }
            // the padding of each scale row is +0.0
            if (part == 0 && tid < n) {
                float* srow = reinterpret_cast<float*>(Q.s + s_dest[tid] * Q.s_stride +
                                                       (int64_t)s_slot[tid] * Q.s_pitch);
                for (int64_t g = Q.n_scales; g < Q.s_pitch / 4; ++g) srow[g] = 0.0f;
            }
        } else if (QMODE == 2) {
            if (q_lo < q_hi) store_quant_pass_fp4(Q, q_lo, q_mid, qp4, n, s_dest, s_slot);
            const uint8_t* src = Q.src + t * Q.src_stride;
            for (int64_t base = q_mid; base < q_hi; base += kPackThreads * kQU) {
                const int64_t top = base + kPackThreads * kQU < q_hi ? base + kPackThreads * kQU
                                                                     : q_hi;
                Fp4Pass more;
                quantize_pass_fp4(src, base, top, more);
                store_quant_pass_fp4(Q, base, top, more, n, s_dest, s_slot);
            }
            // the padding of each scale row is 0x00 (e4m3 +0.0)
            if (part == 0 && tid < n) {
                uint8_t* srow = Q.s + s_dest[tid] * Q.s_stride + (int64_t)s_slot[tid] * Q.s_pitch;
                for (int64_t g = Q.n_scales; g < Q.s_pitch; ++g) srow[g] = 0;
            }
        } else if (pf_item) {
            const int64_t rb = P.row_bytes[0];
            const int64_t nvec = rb >> 4;
            const int64_t p_lo = part * ((nvec + nsplit - 1) / nsplit);
            for (int a = 0; a < n; ++a) {
                uint8_t* dst = P.dst[0] + s_dest[a] * P.dst_stride[0] + (int64_t)s_slot[a] * rb;
#pragma unroll
                for (int u = 0; u < kPackUnroll; ++u) {
                    const int64_t i = p_lo + u * kPackThreads + tid;
                    if (i < p_mid) st_row<MOE_EP_PACK_ST_NT>(dst + i * 16, pre[u]);
                }
            }
        }

        // The rest: further passes of payload 0 and every other payload.
        for (int p = 0; p < P.n; ++p) {
            const int64_t rb = P.row_bytes[p];
            const int64_t nvec = rb >> 4;
            const int64_t per = (nvec + nsplit - 1) / nsplit;
            int64_t v_lo = part * per;
            const int64_t v_hi = v_lo + per < nvec ? v_lo + per : nvec;
            if (pf_item && p == 0) v_lo = p_mid;   // first pass done
            const uint8_t* src = P.src[p] + t * P.src_stride[p];
            for (int64_t i0 = v_lo + tid; i0 < v_hi; i0 += kPackThreads * kPackUnroll) {
                u32x4 v[kPackUnroll];
#pragma unroll
                for (int u = 0; u < kPackUnroll; ++u) {
                    const int64_t i = i0 + u * kPackThreads;
                    if (i < v_hi) v[u] = ld_row<MOE_EP_PACK_LD_NT>(src + i * 16);
                }
                for (int a = 0; a < n; ++a) {
                    uint8_t* dst = P.dst[p] + s_dest[a] * P.dst_stride[p] +
                                   (int64_t)s_slot[a] * rb;
#pragma unroll
                    for (int u = 0; u < kPackUnroll; ++u) {
                        const int64_t i = i0 + u * kPackThreads;
                        if (i < v_hi) st_row<MOE_EP_PACK_ST_NT>(dst + i * 16, v[u]);
                    }
                }
            }
        }
        // Wave 0, after its share of the copy: the pick metadata of each
        // destination slot (block of part 0 only).
        if (tid < W && part == 0) {
            uint32_t bad = 0;
            if (slot >= 0) {
                const int64_t meta = (int64_t)tid * meta_stride + (int64_t)slot * slots;
                bad = write_pick_meta<RANKED != 0>(
                    ids, wts, t, K, E, e_local, tid, slots, send_eloc + meta, send_w + meta,
                    RANKED ? R.send_rank + meta : nullptr, s_prank);
            }
            report(err, bad);
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
                            int32_t* send_eloc, float* send_w, int64_t meta_stride,
                            const RankArgs* ranks, uint32_t* err, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    int64_t max_vecs = quant ? quant->H / 8 : 0;
    for (int p = 0; p < P.n; ++p)
        if (P.row_bytes[p] / 16 > max_vecs) max_vecs = P.row_bytes[p] / 16;
    const int nsplit = row_split(T, max_vecs);
    const int64_t blocks = T * nsplit;
    const int64_t grid = blocks < 65536 ? blocks : 65536;
    // the early first pass pays with its own routing (short kernels) and
    // for leading rows wider than 8 KiB; 8 KiB rows measured slower with it
    const bool pf = P.n > 0 && (rank == nullptr || P.row_bytes[0] / 16 > kPackPrefetchVecs);
    const bool ranked = ranks != nullptr && ranks->send_rank != nullptr;
    const RankArgs R = ranked ? *ranks : RankArgs{};
    // own routing with ranks: block 0's per-expert counts, unless the
    // blocks share them out
    const size_t lds = ranked && rank == nullptr && (E + grid - 1) / grid > kEcntPerBlock
                           ? sizeof(int32_t) * (size_t)E : 0;
    const QuantArgs Q = quant ? *quant : QuantArgs{};
#define MOE_EP_PACK_LAUNCH(QM, PFV, RK)                                                   \
    pack_copy_kernel<QM, PFV, RK><<<dim3((unsigned)grid), dim3(kPackThreads), lds, stream>>>( \
        ids, wts, T, K, E, e_local, W, slots, cap, nsplit, rank, token_slot, tile_cnt,   \
        tile_off, send_cnt, P, Q, send_eloc, send_w, meta_stride, R, err)
    // ranks from the routing kernel (1) or counted by the pack itself (2)
    const int rk = !ranked ? 0 : rank != nullptr ? 1 : 2;
#define MOE_EP_PACK_RANKED(QM, PFV)                                                       \
    if (rk == 2) MOE_EP_PACK_LAUNCH(QM, PFV, 2);                                          \
    else if (rk == 1) MOE_EP_PACK_LAUNCH(QM, PFV, 1);                                     \
    else MOE_EP_PACK_LAUNCH(QM, PFV, 0);
    if (quant && quant->mode == 2) {
        MOE_EP_PACK_RANKED(2, false)
    } else if (quant) {
        MOE_EP_PACK_RANKED(1, false)
    } else if (pf) {
        MOE_EP_PACK_RANKED(0, true)
    } else {
        MOE_EP_PACK_RANKED(0, false)
    }
#undef MOE_EP_PACK_RANKED
#undef MOE_EP_PACK_LAUNCH
    return hipGetLastError();
}

}  // namespace moe_ep
