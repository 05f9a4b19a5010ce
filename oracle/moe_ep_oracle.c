/*
 * moe_ep_oracle.c -- plain, slow, single-threaded CPU oracle for the MoE
 * expert-parallel dispatch/combine layout transform.
 *
 * TEST INFRASTRUCTURE. Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load or call this library. It shares no
 * code, header, table or helper with the HIP library; neither includes or
 * links the other.
 *
 * What it computes is restated from the vLLM API documentation page
 * "vllm.model_executor.layers.fused_moe.prepare_finalize.alltoall_batched",
 * class AllToAllBatchedPrepareAndFinalize, methods capacities(), prepare()
 * and finalize(). The steps below follow the order in which that page takes
 * them. Where the page leaves a choice open, the reading taken is one of
 * these, named where it applies:
 *
 *   A1  picks of one (destination, token) pair fill columns in router
 *       order (ascending k).
 *   A2  slots within a destination follow ascending token index.
 *   A3  any negative expert id is "not routed".
 *   A4  an id >= E is dropped (error bit 0).
 *   A5  more picks for one (destination, token) than the expert slots per
 *       token: the extra picks are dropped (error bit 1).
 *   A7  rows within an expert follow (source, slot, pick) order.
 *   A8  a row index >= rows per expert is dropped (error bit 3).
 *   A10 only valid prefixes are written; tails are left as they are.
 *   A11 the weighted reduce starts at +0.0f, adds in ascending pick order,
 *       rounds each product to fp32 before adding (no fused multiply-add).
 *   A12 the fp32 partial is rounded to bf16 to nearest, ties to even.
 *   A13 the unpack sums partials in fp32 from +0.0f in ascending
 *       destination order and rounds once.
 *   A14 a token with no (destination, token) pair gets +0.0.
 *   A15 a received count outside [0, cap] is clamped (error bit 4); a
 *       received local expert id >= e_local is dropped (error bit 2).
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fPIC -shared. Floating point
 * is IEEE binary32 on SSE; no contraction, no excess precision.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_ERR_ID_RANGE 1u     /* topk id >= E                         */
#define ORACLE_ERR_PICKS    2u     /* more picks per (dest, token) than slots */
#define ORACLE_ERR_ELOC     4u     /* received local expert id out of range  */
#define ORACLE_ERR_ROWCAP   8u     /* expert row >= rows per expert          */
#define ORACLE_ERR_CNT      16u    /* received count outside [0, cap]        */

#define ORACLE_BF16 0
#define ORACLE_F32  1

/* ------------------------------------------------------------------ */
/* Number formats, written from their definitions.                     */
/* ------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32 word. */
static float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bf16, round to nearest, ties to even. The 16 discarded bits
 * are compared with the halfway point 0x8000: above it rounds up, below it
 * truncates, and exactly at it rounds to the neighbour whose last kept bit
 * is zero. A NaN is not rounded: it keeps its sign and the upper 7 bits
 * of its fraction, with the quiet bit (the leading fraction bit) set, since
 * IEEE 754 asks that a NaN result carry what of an input NaN's payload the
 * format can hold and that a signaling NaN come out quiet. */
static uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)(kept | 0x0040u);
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;                /* may carry into the exponent: correct */
    return (uint16_t)kept;
}

static float load_elem(const void* base, int32_t dtype, int64_t idx)
{
    if (dtype == ORACLE_BF16)
        return oracle_bf16_to_f32(((const uint16_t*)base)[idx]);
    return ((const float*)base)[idx];
}

static void store_elem(void* base, int32_t dtype, int64_t idx, float v)
{
    if (dtype == ORACLE_BF16)
        ((uint16_t*)base)[idx] = oracle_f32_to_bf16(v);
    else
        ((float*)base)[idx] = v;
}

/* ------------------------------------------------------------------ */
/* capacities(): token slots per rank = max_num_tokens; expert slots    */
/* per token = min(topk, local experts); rows per expert =              */
/* max_num_tokens * number of dispatchers.                              */
/* ------------------------------------------------------------------ */
int oracle_capacities(int32_t K, int32_t E, int32_t W, int64_t max_num_tokens,
                      int64_t* cap, int32_t* slots, int64_t* expert_cap)
{
    if (K <= 0 || E <= 0 || W <= 0 || E % W != 0 || max_num_tokens < 0)
        return -1;
    int32_t e_local = E / W;
    *cap = max_num_tokens;
    *slots = K < e_local ? K : e_local;
    *expert_cap = max_num_tokens * (int64_t)W;
    return 0;
}

/* ------------------------------------------------------------------ */
/* prepare(), send side of one source rank.                             */
/*                                                                      */
/* 1. Padding filter: entries with a negative id take no part (A3).     */
/* 2. Destination of an entry: floor(id / e_local) (contiguous blocks   */
/*    of local experts per rank).                                       */
/* 3. Deduplicate (destination, token) pairs, ordered by destination    */
/*    then token (A2).                                                  */
/* 4. Per-destination histogram of the unique pairs; a pair's slot is   */
/*    its position within its destination's group.                      */
/* 5. Payload scatter: send[d, slot] = row of the token, every payload. */
/* 6. Picks: within one pair, the routed entries in router order take   */
/*    columns 0, 1, ... (A1); local expert id = id - d*e_local, weight  */
/*    as given in fp32; unused columns hold -1 and +0.0f.               */
/*                                                                      */
/* send_cnt [W]; send_eloc, send_w [W, cap, slots]; token_slot [T, W]   */
/* (-1 where the token has no pair). Payload p: row t at                */
/* src[p] + t*src_row_stride[p]; slot (d, s) at                         */
/* dst[p] + d*dst_rank_stride[p] + s*dst_row_stride[p]; row_bytes[p]    */
/* bytes are copied. Returns the OR of the error bits.                  */
/* ------------------------------------------------------------------ */
uint32_t oracle_dispatch_pack(
    const int32_t* topk_ids, const float* topk_weights,
    int64_t T, int32_t K, int32_t E, int32_t W, int64_t max_num_tokens,
    int32_t n_payloads,
    const uint8_t* const* src, const int64_t* src_row_stride,
    const int64_t* row_bytes,
    uint8_t* const* dst, const int64_t* dst_rank_stride,
    const int64_t* dst_row_stride,
    int32_t* send_cnt, int32_t* send_eloc, float* send_w,
    int32_t* token_slot)
{
    int64_t cap, expert_cap;
    int32_t slots;
    uint32_t err = 0;
    if (oracle_capacities(K, E, W, max_num_tokens, &cap, &slots, &expert_cap))
        return 0xFFFFFFFFu;
    if (T > cap)
        return 0xFFFFFFFFu;
    const int32_t e_local = E / W;

    /* Steps 1-2 also record range errors once per entry. */
    for (int64_t t = 0; t < T; ++t)
        for (int32_t k = 0; k < K; ++k)
            if (topk_ids[t * K + k] >= E)
                err |= ORACLE_ERR_ID_RANGE;

    for (int32_t d = 0; d < W; ++d) {
        int32_t count = 0;                      /* histogram of pairs to d */
        for (int64_t t = 0; t < T; ++t) {
            /* entries of token t routed to d, in router order */
            int32_t npicks = 0;
            for (int32_t k = 0; k < K; ++k) {
                int32_t id = topk_ids[t * K + k];
                if (id < 0 || id >= E)
                    continue;
                if (id / e_local == d)
                    ++npicks;
            }
            if (npicks == 0) {
                token_slot[t * W + d] = -1;
                continue;
            }
            int32_t slot = count;               /* position in d's group */
            count += 1;
            token_slot[t * W + d] = slot;

            for (int32_t p = 0; p < n_payloads; ++p)
                memcpy(dst[p] + d * dst_rank_stride[p] + slot * dst_row_stride[p],
                       src[p] + t * src_row_stride[p], (size_t)row_bytes[p]);

            int64_t meta = ((int64_t)d * cap + slot) * slots;
            int32_t j = 0;
            for (int32_t k = 0; k < K; ++k) {
                int32_t id = topk_ids[t * K + k];
                if (id < 0 || id >= E || id / e_local != d)
                    continue;
                if (j >= slots) {
                    err |= ORACLE_ERR_PICKS;
                    continue;
                }
                send_eloc[meta + j] = id - d * e_local;
                send_w[meta + j] = topk_weights[t * K + k];
                j += 1;
            }
            for (; j < slots; ++j) {
                send_eloc[meta + j] = -1;
                send_w[meta + j] = 0.0f;
            }
        }
        send_cnt[d] = count;
    }
    return err;
}

/* ------------------------------------------------------------------ */
/* prepare(), receive side of one destination rank.                     */
/*                                                                      */
/* recv_cnt[s] (stride cnt_rank_stride) slots arrived from source s;    */
/* recv_eloc of source s starts at s*eloc_rank_stride and is            */
/* [cap, slots]. An entry (s, slot, j) is valid when slot < recv_cnt[s] */
/* and its local expert id is >= 0. Valid entries are taken in          */
/* (s, slot, j) order (A7); each takes the next free row of its expert  */
/* (a running count per expert). Rows at or past rows-per-expert are    */
/* dropped (A8). expert_num_tokens[e] = rows taken, clamped to          */
/* rows-per-expert. recv_row [W, cap, slots] gets the row of each valid */
/* entry and -1 for an unused pick column of a valid slot.              */
/*                                                                      */
/* Payload p: slot (s, slot) at src[p] + s*src_rank_stride[p] +         */
/* slot*src_row_stride[p]; row (e, r) at dst[p] + e*dst_expert_stride[p]*/
/* + r*dst_row_stride[p].                                               */
/* ------------------------------------------------------------------ */
uint32_t oracle_expert_batch(
    const int32_t* recv_cnt, int64_t cnt_rank_stride,
    const int32_t* recv_eloc, int64_t eloc_rank_stride,
    int32_t W, int32_t e_local, int32_t K, int64_t max_num_tokens,
    int32_t n_payloads,
    const uint8_t* const* src, const int64_t* src_rank_stride,
    const int64_t* src_row_stride, const int64_t* row_bytes,
    uint8_t* const* dst, const int64_t* dst_expert_stride,
    const int64_t* dst_row_stride,
    int32_t* expert_num_tokens, int32_t* recv_row)
{
    int64_t cap, expert_cap;
    int32_t slots;
    uint32_t err = 0;
    if (oracle_capacities(K, e_local * W, W, max_num_tokens, &cap, &slots,
                          &expert_cap))
        return 0xFFFFFFFFu;

    int64_t n[1024];                  /* running row count per expert */
    if (e_local > 1024)
        return 0xFFFFFFFFu;
    for (int32_t e = 0; e < e_local; ++e)
        n[e] = 0;

    for (int32_t s = 0; s < W; ++s) {
        int64_t cnt = recv_cnt[s * cnt_rank_stride];
        if (cnt < 0 || cnt > cap) {
            err |= ORACLE_ERR_CNT;
            cnt = cnt < 0 ? 0 : cap;
        }
        for (int64_t slot = 0; slot < cnt; ++slot) {
            for (int32_t j = 0; j < slots; ++j) {
                int32_t e = recv_eloc[s * eloc_rank_stride + slot * slots + j];
                int64_t at = ((int64_t)s * cap + slot) * slots + j;
                if (e < 0) {
                    recv_row[at] = -1;
                    continue;
                }
                if (e >= e_local) {
                    err |= ORACLE_ERR_ELOC;
                    recv_row[at] = -1;
                    continue;
                }
                int64_t row = n[e];
                n[e] += 1;
                if (row >= expert_cap) {
                    err |= ORACLE_ERR_ROWCAP;
                    recv_row[at] = -1;
                    continue;
                }
                recv_row[at] = (int32_t)row;
                for (int32_t p = 0; p < n_payloads; ++p)
                    memcpy(dst[p] + e * dst_expert_stride[p] + row * dst_row_stride[p],
                           src[p] + s * src_rank_stride[p] + slot * src_row_stride[p],
                           (size_t)row_bytes[p]);
            }
        }
    }
    for (int32_t e = 0; e < e_local; ++e)
        expert_num_tokens[e] = (int32_t)(n[e] < expert_cap ? n[e] : expert_cap);
    return err;
}

/* ------------------------------------------------------------------ */
/* Send-side form of the receive rows. The page numbers a destination's */
/* rows per local expert in (source, slot, column) order. Within one    */
/* source that is the order the source sends in (slots by token, columns */
/* by router order), so a source can count its own part: the rank of    */
/* each used pick column among its earlier columns with the same local  */
/* id, and the number of columns per local id. A destination's row for  */
/* (s, slot, j) is then the counts of sources before s plus the rank.   */
/*                                                                      */
/* For every destination d of one source, over slots [0, send_cnt[d])  */
/* ascending and columns ascending: a column with local id e >= 0 gets */
/* send_rank = (columns of d with id e seen so far); a column with a    */
/* negative id gets -1. send_ecnt[d, e] = columns of d with id e. Only  */
/* the send_cnt[d] valid slots of send_rank are written; every entry of */
/* send_ecnt is. Layouts as oracle_dispatch_pack's [W, cap, slots]     */
/* metadata; send_ecnt is [W, e_local].                                 */
/* ------------------------------------------------------------------ */
int oracle_pick_ranks(const int32_t* send_cnt, const int32_t* send_eloc,
                      int32_t W, int32_t e_local, int32_t slots, int64_t cap,
                      int32_t* send_rank, int32_t* send_ecnt)
{
    if (W <= 0 || e_local <= 0 || slots <= 0 || cap < 0)
        return -1;
    for (int32_t d = 0; d < W; ++d) {
        for (int32_t e = 0; e < e_local; ++e)
            send_ecnt[(int64_t)d * e_local + e] = 0;
        for (int64_t slot = 0; slot < send_cnt[d]; ++slot) {
            for (int32_t j = 0; j < slots; ++j) {
                int64_t at = ((int64_t)d * cap + slot) * slots + j;
                int32_t e = send_eloc[at];
                if (e < 0 || e >= e_local) {
                    send_rank[at] = -1;
                    continue;
                }
                send_rank[at] = send_ecnt[(int64_t)d * e_local + e];
                send_ecnt[(int64_t)d * e_local + e] += 1;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* vLLM alltoall_batched page, finalize(), destination side: one row    */
/* per received slot, the weighted sum of that slot's expert rows.      */
/*                                                                      */
/* For every valid received slot (s, slot): acc = +0.0f; for pick j     */
/* ascending with recv_row >= 0: acc = acc + (fp32(Y[e_j, row_j, h]) *  */
/* w_j), each product rounded to fp32 before the add (A11). The result  */
/* is stored in the data type: bf16 by round-to-nearest-even (A12), or  */
/* fp32 as is.                                                          */
/*                                                                      */
/* Y element (e, r, h) at Y + e*y_expert_stride + r*y_row_stride + h;   */
/* ret element (s, slot, h) at ret + s*ret_rank_stride +                */
/* slot*ret_row_stride + h (element strides). Only H columns are done,  */
/* so a caller can work on a column window of wider rows.               */
/* ------------------------------------------------------------------ */
uint32_t oracle_combine_reduce(
    const void* Y, int64_t y_expert_stride, int64_t y_row_stride,
    int32_t dtype, int64_t H,
    const int32_t* recv_cnt, int64_t cnt_rank_stride,
    const int32_t* recv_eloc, const float* recv_w, int64_t meta_rank_stride,
    const int32_t* recv_row,
    int32_t W, int32_t e_local, int32_t K, int64_t max_num_tokens,
    void* ret, int64_t ret_rank_stride, int64_t ret_row_stride)
{
    int64_t cap, expert_cap;
    int32_t slots;
    uint32_t err = 0;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F32)
        return 0xFFFFFFFFu;
    if (oracle_capacities(K, e_local * W, W, max_num_tokens, &cap, &slots,
                          &expert_cap))
        return 0xFFFFFFFFu;

    for (int32_t s = 0; s < W; ++s) {
        int64_t cnt = recv_cnt[s * cnt_rank_stride];
        if (cnt < 0 || cnt > cap) {
            err |= ORACLE_ERR_CNT;
            cnt = cnt < 0 ? 0 : cap;
        }
        for (int64_t slot = 0; slot < cnt; ++slot) {
            for (int64_t h = 0; h < H; ++h) {
                float acc = 0.0f;
                for (int32_t j = 0; j < slots; ++j) {
                    int64_t at = ((int64_t)s * cap + slot) * slots + j;
                    int32_t row = recv_row[at];
                    if (row < 0)
                        continue;
                    int32_t e = recv_eloc[s * meta_rank_stride + slot * slots + j];
                    float wgt = recv_w[s * meta_rank_stride + slot * slots + j];
                    float y = load_elem(Y, dtype,
                                        e * y_expert_stride + row * y_row_stride + h);
                    float prod = y * wgt;
                    acc = acc + prod;
                }
                store_elem(ret, dtype, s * ret_rank_stride + slot * ret_row_stride + h,
                           acc);
            }
        }
    }
    return err;
}

/* ------------------------------------------------------------------ */
/* vLLM alltoall_batched page, finalize(), source side: a token's row is */
/* the sum of what each of its destination ranks returned for it.       */
/*                                                                      */
/* out[t, h] = round(sum over d ascending with token_slot[t,d] >= 0 of  */
/* fp32(back[d, token_slot[t,d], h])), accumulated in fp32 from +0.0f   */
/* (A13); a token with no pair gets +0.0 (A14). Every row of out is     */
/* written.                                                             */
/*                                                                      */
/* back element (d, slot, h) at back + d*back_rank_stride +             */
/* slot*back_row_stride + h; out element (t, h) at out +                */
/* t*out_row_stride + h (element strides).                              */
/* ------------------------------------------------------------------ */
void oracle_combine_unpack(
    const void* back, int64_t back_rank_stride, int64_t back_row_stride,
    int32_t dtype, int64_t H,
    const int32_t* token_slot, int64_t T, int32_t W,
    void* out, int64_t out_row_stride)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int32_t d = 0; d < W; ++d) {
                int32_t slot = token_slot[t * W + d];
                if (slot < 0)
                    continue;
                acc = acc + load_elem(back, dtype,
                                      d * back_rank_stride + slot * back_row_stride + h);
            }
            store_elem(out, dtype, t * out_row_stride + h, acc);
        }
    }
}

/* Exposed for the pins on the number format. The _bits form takes the
 * binary32 word as an integer, so that a signaling NaN reaches the rounding
 * unchanged (a float argument may be quieted on the way in). */
uint16_t oracle_round_bf16(float f) { return oracle_f32_to_bf16(f); }

uint16_t oracle_round_bf16_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return oracle_f32_to_bf16(f);
}

/* ------------------------------------------------------------------ */
/* Quantize-on-pack (the fp8 dispatch that the FlashInfer one-sided    */
/* manager on the vLLM all2all page sizes its workspace for).           */
/* ------------------------------------------------------------------ */

/* OCP 8-bit floating point E4M3 ("FN": finite, no infinities): sign bit,
 * 4 exponent bits with bias 7, 3 fraction bits. Exponent field 0 holds the
 * subnormals f/8 * 2^-6; S.1111.111 is NaN; the largest finite magnitude is
 * S.1111.110 = 448. Encoding rounds to nearest, ties to even; a magnitude
 * that rounds past 448 saturates to 448; NaN stays NaN. */
uint8_t oracle_f32_to_e4m3(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
    if (f != f)
        return (uint8_t)(sign | 0x7Fu);
    const double a = fabs((double)f);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7Eu);
    if (a < 0x1p-6) {
        /* subnormal steps of 2^-9; 8 steps is the smallest normal, 0x08 */
        const double m = rint(a * 512.0);
        return (uint8_t)(sign | (uint8_t)m);
    }
    int e = ilogb(a);                         /* floor(log2 a): -6 .. 8 */
    double m = rint(ldexp(a, 3 - e));         /* 8 .. 16 */
    if (m == 16.0) {
        m = 8.0;
        e += 1;
    }
    if (e > 8 || (e == 8 && m > 14.0))
        return (uint8_t)(sign | 0x7Eu);
    return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | ((int)m - 8)));
}

/* Per-row, per-group fp8 quantisation of bf16 rows. For every group of
 * `group` consecutive columns: amax = max |x| over the non-NaN entries;
 * the scale is s = amax / 448 and each code is q = e4m3(x / s), both fp32
 * divisions rounded to nearest and the quotient then encoded to nearest
 * even (the plain scaled cast: divide by the scale in fp32, then convert);
 * s = 1 when amax = 0. Each code carries the sign bit of its input x
 * (IEEE 754 leaves the sign of a NaN quotient open: a NaN input, or an
 * infinite one divided by an infinite scale, gives the NaN code with x's
 * sign). Dequantisation is q * s. Row t of x at x + t*x_row_stride
 * (elements); codes of row t at q + t*q_row_stride (bytes); scales of row t
 * at scale + t*scale_row_stride (elements). */
void oracle_quantize_fp8(const uint16_t* x, int64_t T, int64_t H,
                         int64_t x_row_stride, int32_t group, uint8_t* q,
                         int64_t q_row_stride, float* scale,
                         int64_t scale_row_stride)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t g = 0; g * group < H; ++g) {
            float amax = 0.0f;
            for (int64_t h = g * group; h < (g + 1) * group && h < H; ++h) {
                float v = fabsf(oracle_bf16_to_f32(x[t * x_row_stride + h]));
                if (v > amax)
                    amax = v;
            }
            const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
            scale[t * scale_row_stride + g] = s;
            for (int64_t h = g * group; h < (g + 1) * group && h < H; ++h) {
                const float v = oracle_bf16_to_f32(x[t * x_row_stride + h]);
                const float y = v / s;
                const uint8_t c = oracle_f32_to_e4m3(y);
                q[t * q_row_stride + h] = (uint8_t)((c & 0x7Fu) | (signbit(v) ? 0x80u : 0u));
            }
        }
    }
}

/* OCP E4M3 code -> value (exact in binary32): exponent field 0 holds the
 * subnormals f/8 * 2^-6, otherwise (1 + f/8) * 2^(e-7); S.1111.111 is NaN. */
float oracle_e4m3_to_f32(uint8_t c)
{
    const int e = (c >> 3) & 0xF;
    const int f = c & 0x7;
    double v;
    if (e == 0xF && f == 0x7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)f, -9);
    else
        v = ldexp(8.0 + f, e - 10);
    return (float)((c & 0x80) ? -v : v);
}

/* OCP 4-bit floating point E2M1: sign bit, 2 exponent bits with bias 1,
 * 1 fraction bit; the eight magnitudes of codes 0..7 are 0, 0.5, 1, 1.5,
 * 2, 3, 4, 6 (no infinities, no NaN). Encoding takes the nearest
 * magnitude; a tie goes to the code whose last bit is 0 (ties to even);
 * magnitudes above 6 saturate to 6. A NaN (not produced from finite bf16
 * rows) encodes as a zero of its sign. Returns the 4-bit code. */
uint8_t oracle_f32_to_e2m1(float f)
{
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint8_t sign = (uint8_t)((u >> 28) & 0x8u);
    if (f != f)
        return sign;
    const double a = fabs((double)f);
    if (a >= 6.0)                  /* saturation (distances to 4 and 6 */
        return (uint8_t)(sign | 7);  /* would tie in double for huge a) */
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        const double dc = fabs(a - mag[c]);
        const double db = fabs(a - mag[best]);
        if (dc < db || (dc == db && (c & 1) == 0))
            best = c;
    }
    return (uint8_t)(sign | best);
}

/* 4-bit quantisation of bf16 rows with 8-bit scales, in blocks of 16
 * columns (the dispatch that FlashInferNVLinkOneSidedManager on the vLLM
 * "device_communicators.all2all" documentation page sizes as H/2 code
 * bytes plus H/16 scale bytes per token). For every block: amax = max |x|;
 * the stored scale is the E4M3 code of amax / 6 (fp32 division, then
 * rounded to nearest even, saturating at 448); with s its value, the codes
 * are q = e2m1(x / s) (fp32 division rounded to nearest, then the E2M1
 * encoding), or zeros when s = 0.
 * NaN entries do not take part in amax, and each code carries the sign
 * bit of its input x (a NaN input gives a zero of its sign).
 * Dequantisation is value(q) * s. Two codes per byte: the even column in
 * the low nibble. Row t of x at x + t*x_row_stride (elements); codes of
 * row t at q + t*q_row_stride (bytes, H/2 of them); scales of row t at
 * scale + t*scale_row_stride (bytes, H/16 of them). H is a multiple of 16. */
void oracle_quantize_fp4(const uint16_t* x, int64_t T, int64_t H,
                         int64_t x_row_stride, uint8_t* q, int64_t q_row_stride,
                         uint8_t* scale, int64_t scale_row_stride)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t b = 0; b * 16 < H; ++b) {
            float amax = 0.0f;
            for (int64_t h = b * 16; h < b * 16 + 16; ++h) {
                float v = fabsf(oracle_bf16_to_f32(x[t * x_row_stride + h]));
                if (v > amax)
                    amax = v;
            }
            const uint8_t s8 = oracle_f32_to_e4m3(amax / 6.0f);
            const float s = oracle_e4m3_to_f32(s8);
            scale[t * scale_row_stride + b] = s8;
            for (int64_t h = b * 16; h < b * 16 + 16; h += 2) {
                const float v0 = oracle_bf16_to_f32(x[t * x_row_stride + h]);
                const float v1 = oracle_bf16_to_f32(x[t * x_row_stride + h + 1]);
                const float y0 = s > 0.0f ? v0 / s : 0.0f;
                const float y1 = s > 0.0f ? v1 / s : 0.0f;
                const uint8_t c0 = (uint8_t)((oracle_f32_to_e2m1(y0) & 7u) |
                                             (signbit(v0) ? 8u : 0u));
                const uint8_t c1 = (uint8_t)((oracle_f32_to_e2m1(y1) & 7u) |
                                             (signbit(v1) ? 8u : 0u));
                q[t * q_row_stride + h / 2] = (uint8_t)(c0 | (c1 << 4));
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* Received expert ids for consumers that read the received slots in   */
/* place (FlashInfer module, moe_a2a_sanitize_expert_ids: the ids of   */
/* received entries that are not valid tokens are set to a sentinel).  */
/*                                                                      */
/* out[s, slot, j] = recv_eloc[s, slot, j] when slot < recv_cnt[s]      */
/* (clamped to [0, cap]) and the id is in [0, e_local); invalid_id      */
/* otherwise. Every entry of the [W, cap, slots] layout is written.     */
/* ------------------------------------------------------------------ */
uint32_t oracle_sanitize_expert_ids(
    const int32_t* recv_cnt, int64_t cnt_rank_stride,
    const int32_t* recv_eloc, int64_t eloc_rank_stride,
    int32_t W, int32_t e_local, int32_t K, int64_t max_num_tokens,
    int32_t invalid_id, int32_t* out, int64_t out_rank_stride)
{
    int64_t cap, expert_cap;
    int32_t slots;
    uint32_t err = 0;
    if (oracle_capacities(K, e_local * W, W, max_num_tokens, &cap, &slots,
                          &expert_cap))
        return 0xFFFFFFFFu;
    for (int32_t s = 0; s < W; ++s) {
        int64_t cnt = recv_cnt[s * cnt_rank_stride];
        if (cnt < 0 || cnt > cap) {
            err |= ORACLE_ERR_CNT;
            cnt = cnt < 0 ? 0 : cap;
        }
        for (int64_t slot = 0; slot < cap; ++slot) {
            for (int32_t j = 0; j < slots; ++j) {
                int32_t v = invalid_id;
                if (slot < cnt) {
                    int32_t e = recv_eloc[s * eloc_rank_stride + slot * slots + j];
                    if (e >= e_local)
                        err |= ORACLE_ERR_ELOC;
                    if (e >= 0 && e < e_local)
                        v = e;
                }
                out[s * out_rank_stride + slot * slots + j] = v;
            }
        }
    }
    return err;
}

