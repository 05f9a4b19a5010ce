/*
 * moe_ep.h -- C ABI of the MI355X (gfx950) MoE expert-parallel
 * dispatch/combine layout transform.
 *
 * The operation is the one stated on the vLLM API documentation page
 * "vllm.model_executor.layers.fused_moe.prepare_finalize.alltoall_batched"
 * (class AllToAllBatchedPrepareAndFinalize): a token goes to each
 * destination rank once however many of its experts live there, carrying
 * its local expert ids and router weights as metadata (prepare(), send
 * side); the receive side re-batches rows per local expert
 * (prepare(), receive side); after the experts run, each destination
 * turns the expert rows of each received slot into one weighted row
 * (finalize(), first half) and each source adds up the rows returned for
 * each of its tokens (finalize(), second half). The list of opaque payloads
 * that travel with a token follows the FlashInfer module
 * "flashinfer/comm/trtllm_moe_alltoall.py" (moe_a2a_dispatch: several
 * [T, *] payloads per call, each received as [ep_size, max_tokens, *]).
 *
 * Conventions shared by every call
 *   - Pointers are device pointers unless a comment says host.
 *   - The caller owns every buffer, including the workspace. The library
 *     never allocates, frees, synchronises the host or keeps state between
 *     calls. Work is enqueued on `stream` (a hipStream_t; NULL is the
 *     default stream); outputs are ready when the stream reaches the call;
 *     inputs must stay alive until then.
 *   - Arguments are checked before anything is enqueued; a non-zero status
 *     means nothing was enqueued (except MOE_EP_EHIP, a launch failure).
 *   - Notation: T tokens of this source rank, K picks per token, E experts,
 *     W ranks, e_local = E / W local experts per rank,
 *     cap = max_num_tokens token slots per (source, destination),
 *     slots = min(K, e_local) pick columns per slot,
 *     expert_cap = W * cap rows per local expert
 *     (capacities() on the vLLM page).
 *   - Only valid prefixes are written: send slots [0, send_cnt[d]), expert
 *     rows [0, expert_num_tokens[e]), returned slots [0, recv_cnt[s]).
 *     Tails keep whatever the caller left there. combine_unpack writes
 *     every token row.
 *   - Data errors that the host cannot see without a sync are reported by
 *     OR-ing MOE_EP_ERR_* bits into *err_flags (if non-NULL; the caller
 *     clears it) and have the defined behaviour given with each bit.
 *   - Limits: 1 <= W <= 64, e_local <= 1024, slots <= 64,
 *     n_payloads <= 8, cap <= INT_MAX, H <= INT_MAX, and
 *     W * cap * slots, T * K, T * W < 2^31 (EINVAL otherwise).
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define MOE_EP_API __attribute__((visibility("default")))
#else
#define MOE_EP_API
#endif

/* Status codes. */
#define MOE_EP_OK          0
#define MOE_EP_EINVAL     -1   /* bad pointer, size, stride or limit      */
#define MOE_EP_ECAP       -2   /* T > max_num_tokens                       */
#define MOE_EP_EDTYPE     -3   /* combine data type not supported          */
#define MOE_EP_EALIGN     -4   /* pointer, stride or row not 16-B aligned  */
#define MOE_EP_EWORKSPACE -5   /* workspace missing or too small           */
#define MOE_EP_EHIP       -6   /* a kernel launch failed                    */
#define MOE_EP_ESCRATCH   -7   /* more scratch than moe_ep_dispatch_pack_noalloc
                                  holds (MOE_EP_NOALLOC_SCRATCH_BYTES)      */

/* Combine data types (expert outputs, partials and token outputs). */
#define MOE_EP_BF16 0
#define MOE_EP_F32  1

/* err_flags bits. */
#define MOE_EP_ERR_ID_RANGE 1u  /* topk id >= E: the entry is dropped       */
#define MOE_EP_ERR_PICKS    2u  /* more picks for one (token, dest) than
                                   slots (duplicate ids): extras dropped   */
#define MOE_EP_ERR_ELOC     4u  /* received local id >= e_local: dropped    */
#define MOE_EP_ERR_ROWCAP   8u  /* expert row >= expert_cap: dropped        */
#define MOE_EP_ERR_CNT     16u  /* received count outside [0, cap]: clamped */

#define MOE_EP_MAX_PAYLOADS      8
#define MOE_EP_MAX_WORLD        64
#define MOE_EP_MAX_LOCAL_EXPERTS 1024
#define MOE_EP_MAX_SLOTS        64

/* Device scratch that moe_ep_dispatch_pack_noalloc uses, per GPU. */
#define MOE_EP_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * One payload: every byte of a row is moved as is (bf16, fp8, fp32 scales,
 * int32 ids ...). The leading dimension of src and dst may be strided;
 * rows inside it are dense (row pitch = row_bytes). src, dst, both strides
 * and row_bytes must be multiples of 16 bytes.
 */
typedef struct moe_ep_payload {
    const void* src;       /* device */
    int64_t src_stride;    /* bytes between leading-dim items of src */
    void* dst;             /* device */
    int64_t dst_stride;    /* bytes between leading-dim items of dst */
    int64_t row_bytes;     /* bytes per row, > 0 */
} moe_ep_payload;

/*
 * capacities() of the vLLM page: cap = max_num_tokens,
 * slots = min(K, E / W), expert_cap = max_num_tokens * W. Host only.
 * EINVAL if K <= 0, E <= 0, W <= 0, E % W != 0, max_num_tokens < 0 or
 * max_num_tokens * W does not fit in int64_t.
 */
MOE_EP_API int moe_ep_capacities(int32_t K, int32_t E, int32_t W, int64_t max_num_tokens,
                      int64_t* cap, int32_t* slots, int64_t* expert_cap);

/*
 * Bytes of workspace that moe_ep_dispatch_pack (any T <= max_num_tokens,
 * with or without the per-expert ranks) and moe_ep_expert_batch need for
 * these sizes; one buffer of this size serves both calls when they are
 * ordered on one stream. Each region is
 * padded to 128 bytes, as the FlashInfer module pads its workspace regions
 * (moe_a2a_get_workspace_size_per_rank). Host only.
 */
MOE_EP_API int moe_ep_workspace_bytes(int64_t T, int32_t K, int32_t E, int32_t W,
                           int64_t max_num_tokens, size_t* bytes);

/* Static text for a status code. Host only. */
MOE_EP_API const char* moe_ep_status_string(int status);

/*
 * Dispatch, send side of one source rank (prepare() on the vLLM page:
 * padding filter, destination = floor(id / e_local), one slot per
 * (destination, token) pair in ascending token order, payload scatter,
 * local ids and weights in router order).
 *
 *   topk_ids      int32 [T, K]; a negative id is padding (takes no part).
 *   topk_weights  fp32  [T, K].
 *   payloads      host array of n_payloads descriptors: src [T, row]
 *                 (src_stride = bytes between tokens), dst [W, cap, row]
 *                 (dst_stride = bytes between destination blocks,
 *                 >= cap * row_bytes).
 *   send_cnt      int32 [W] out: slots used per destination.
 *   send_eloc     int32 out: local expert id of pick j of slot (d, s), -1
 *                 for an unused column; destination d's block [cap, slots]
 *                 (dense) at send_eloc + d * meta_rank_stride, so it can be
 *                 aimed at per-destination receive blocks as the payloads
 *                 can.
 *   send_w        fp32 out: its weight, +0.0 unused; same layout and stride.
 *   meta_rank_stride  elements between destination blocks of send_eloc and
 *                 send_w (>= cap * slots; EINVAL otherwise). Elements
 *                 between blocks are not written.
 *   send_rank     int32, nullable, same layout and stride as send_eloc:
 *                 the rank of each used pick column among this source's
 *                 used columns of the same expert on that destination, in
 *                 (slot, column) order; -1 for an unused column. The
 *                 receive side numbers an expert's rows in (source, slot,
 *                 column) order, and within one source that is this order,
 *                 so a row is the counts of the sources before plus the
 *                 rank (moe_ep_expert_batch_ranked).
 *   send_ecnt     int32 [W, e_local], nullable, dense: used pick columns
 *                 per (destination, local expert); every entry is written.
 *                 send_rank and send_ecnt are given together or not at all,
 *                 and need K <= 16 and E <= 4096 (EINVAL otherwise).
 *   token_slot    int32 [T, W] out: slot of token t at destination d, -1
 *                 if none. Context for moe_ep_combine_unpack; keep it.
 *   err_flags     nullable; bits MOE_EP_ERR_ID_RANGE, MOE_EP_ERR_PICKS.
 *   workspace     >= moe_ep_workspace_bytes(...), 16-B aligned.
 */
MOE_EP_API int moe_ep_dispatch_pack(const int32_t* topk_ids, const float* topk_weights,
                         int64_t T, int32_t K, int32_t E, int32_t W,
                         int64_t max_num_tokens,
                         const moe_ep_payload* payloads, int32_t n_payloads,
                         int32_t* send_cnt, int32_t* send_eloc, float* send_w,
                         int64_t meta_rank_stride, int32_t* send_rank, int32_t* send_ecnt,
                         int32_t* token_slot, uint32_t* err_flags, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * moe_ep_dispatch_pack for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. It
 * takes no workspace; the send side's scratch (tile counts, tile offsets
 * and in-tile ranks, the bytes moe_ep_workspace_bytes gives for the send
 * side) lives in a device array of MOE_EP_NOALLOC_SCRATCH_BYTES (8 MiB)
 * that the library holds on each GPU it runs on until the process ends.
 * The call allocates nothing and makes no allocating library call.
 *
 *   - Sizes whose send-side scratch exceeds the array return
 *     MOE_EP_ESCRATCH before anything is enqueued. The scratch is
 *     2 * round_up(ceil(T / 256) * W * 4, 128) + round_up(T * W * 4, 128)
 *     bytes (T <= 256 needs none): T * W up to about 2.08 million (token,
 *     destination) pairs, e.g. T = 65536 at W = 16 or T = 16384 at W = 64.
 *     With send_rank and send_ecnt another round_up(T * K * 4, 128) +
 *     2 * round_up(ceil(T / 256) * E * 4, 128) bytes.
 *   - The stream must belong to the current device (EINVAL otherwise). The
 *     first call on a device looks the array's address up (no allocation);
 *     make it outside graph capture.
 *   - Every call on a GPU shares that GPU's array, and it keeps the last
 *     call's contents. Each call writes every scratch byte it reads before
 *     reading it, so nothing has to be cleared, but calls that overlap on
 *     one GPU (on different streams, or from different host threads) race
 *     on the array: order them.
 * Everything else, and every output, as moe_ep_dispatch_pack.
 */
MOE_EP_API int moe_ep_dispatch_pack_noalloc(const int32_t* topk_ids,
                                            const float* topk_weights, int64_t T,
                                            int32_t K, int32_t E, int32_t W,
                                            int64_t max_num_tokens,
                                            const moe_ep_payload* payloads,
                                            int32_t n_payloads, int32_t* send_cnt,
                                            int32_t* send_eloc, float* send_w,
                                            int64_t meta_rank_stride, int32_t* send_rank,
                                            int32_t* send_ecnt, int32_t* token_slot,
                                            uint32_t* err_flags, void* stream);

/*
 * Dispatch with quantize-on-pack: moe_ep_dispatch_pack, but the bf16 hidden
 * row of each token is quantised once, on the send side, to OCP fp8 E4M3
 * with one fp32 scale per `group` columns, and the codes and scales travel
 * instead of the bf16 row (about half the bytes). The vLLM all2all page's
 * FlashInfer one-sided manager sizes its dispatch for quantised hidden rows
 * plus scale factors; the alltoall_batched page itself supports unquantised
 * MoE only. For each group of a row with amax > 0: scale s = amax / 448
 * and code = e4m3(x / s) (both divisions rounded to fp32 to nearest, the
 * conversion to nearest even: a plain scaled cast); s = 1 when amax = 0.
 * NaN entries do not take part in amax, and every code carries the sign
 * bit of its input (so a NaN input, or an infinite one when the group's
 * amax, and so s, is infinite, gives the NaN code with that sign).
 * Dequantisation is code * scale.
 *
 *   hidden        bf16 [T, H]; hidden_stride = bytes between tokens
 *                 (16-B aligned, >= 2H).
 *   group         32, 64 or 128; H % group == 0.
 *   send_q        e4m3 codes [W, cap, H] (16-B aligned); q_rank_stride =
 *                 bytes between destination blocks (>= cap * H, multiple
 *                 of 16).
 *   send_scale    fp32 [W, cap, Gp] with Gp = H / group rounded up to a
 *                 multiple of 4 (16-byte scale rows, so they batch like any
 *                 payload); columns from H / group on are written +0.0.
 *                 scale_rank_stride = elements between destination blocks
 *                 (>= cap * Gp).
 *   payloads      further payloads moved as is (may be empty).
 * Everything else as moe_ep_dispatch_pack. The receive side batches the
 * codes and the scales as two payloads of moe_ep_expert_batch.
 */
MOE_EP_API int moe_ep_dispatch_pack_fp8(const int32_t* topk_ids, const float* topk_weights,
                                        int64_t T, int32_t K, int32_t E, int32_t W,
                                        int64_t max_num_tokens, const void* hidden,
                                        int64_t hidden_stride, int64_t H, int32_t group,
                                        void* send_q, int64_t q_rank_stride,
                                        float* send_scale, int64_t scale_rank_stride,
                                        const moe_ep_payload* payloads, int32_t n_payloads,
                                        int32_t* send_cnt, int32_t* send_eloc, float* send_w,
                                        int64_t meta_rank_stride, int32_t* send_rank,
                                        int32_t* send_ecnt, int32_t* token_slot,
                                        uint32_t* err_flags, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * Dispatch with 4-bit quantize-on-pack: the FlashInfer one-sided manager on
 * the vLLM all2all page (FlashInferNVLinkOneSidedManager) sizes its dispatch
 * row as H/2 bytes of 4-bit hidden values plus H/16 bytes of fp8 scale
 * factors. Here each bf16 hidden row is quantised once, on the send side,
 * in blocks of 16 columns: amax = max |x|, the scale is the OCP E4M3 code
 * of amax / 6 (fp32 division, then nearest even, saturating at 448), and
 * with s its value each code is the OCP E2M1 code of x / s (the division
 * rounded to fp32; a zero of x's sign when s = 0), to nearest with ties to
 * even, saturating at 6. E2M1
 * magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6. NaN entries do not take part
 * in amax, and every code carries the sign bit of its input (a NaN input
 * gives a zero of its sign). Dequantisation is value(code) * s. Two codes
 * per byte, the even column in the low nibble.
 *
 *   hidden        bf16 [T, H]; hidden_stride = bytes between tokens
 *                 (16-B aligned, >= 2H). H % 32 == 0 (EALIGN otherwise:
 *                 the code row of H/2 bytes is a multiple of 16).
 *   send_q        codes [W, cap, H/2] bytes (16-B aligned); q_rank_stride =
 *                 bytes between destination blocks (>= cap * H/2, multiple
 *                 of 16).
 *   send_scale    E4M3 scale codes [W, cap, Sp] bytes with Sp = H/16 rounded
 *                 up to a multiple of 16; bytes from H/16 on are written
 *                 0x00 (+0.0). scale_rank_stride = bytes between destination
 *                 blocks (>= cap * Sp, multiple of 16; 16-B aligned).
 *   payloads      further payloads moved as is (may be empty).
 * Everything else as moe_ep_dispatch_pack. The receive side batches the
 * codes and the scales as two payloads of moe_ep_expert_batch.
 */
MOE_EP_API int moe_ep_dispatch_pack_fp4(const int32_t* topk_ids, const float* topk_weights,
                                        int64_t T, int32_t K, int32_t E, int32_t W,
                                        int64_t max_num_tokens, const void* hidden,
                                        int64_t hidden_stride, int64_t H,
                                        void* send_q, int64_t q_rank_stride,
                                        void* send_scale, int64_t scale_rank_stride,
                                        const moe_ep_payload* payloads, int32_t n_payloads,
                                        int32_t* send_cnt, int32_t* send_eloc, float* send_w,
                                        int64_t meta_rank_stride, int32_t* send_rank,
                                        int32_t* send_ecnt, int32_t* token_slot,
                                        uint32_t* err_flags, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * Dispatch, receive side of one destination rank (prepare() on the vLLM
 * page after the exchange: a pick (s, slot, j) is valid when
 * slot < recv_cnt[s] and its local id is >= 0; valid picks, taken in
 * (s, slot, j) order, take the next row of their local expert).
 *
 *   recv_cnt      int32, element s at recv_cnt[s * cnt_rank_stride].
 *   recv_eloc     int32, source s block [cap, slots] at
 *                 recv_eloc + s * eloc_rank_stride (elements,
 *                 >= cap * slots).
 *   payloads      src [W, cap, row] (src_stride = bytes between source
 *                 blocks, >= cap * row_bytes), dst [e_local, W*cap, row]
 *                 (dst_stride = bytes between experts,
 *                 >= expert_cap * row_bytes).
 *   expert_num_tokens int32 [e_local] out: rows per local expert.
 *   recv_row      int32 [W, cap, slots] out: expert row of each valid pick,
 *                 -1 for an unused column. Context for combine_reduce.
 *   err_flags     nullable; bits MOE_EP_ERR_ELOC, MOE_EP_ERR_ROWCAP,
 *                 MOE_EP_ERR_CNT.
 */
MOE_EP_API int moe_ep_expert_batch(const int32_t* recv_cnt, int64_t cnt_rank_stride,
                        const int32_t* recv_eloc, int64_t eloc_rank_stride,
                        int32_t W, int32_t e_local, int32_t K,
                        int64_t max_num_tokens,
                        const moe_ep_payload* payloads, int32_t n_payloads,
                        int32_t* expert_num_tokens, int32_t* recv_row,
                        uint32_t* err_flags, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * moe_ep_expert_batch from the sources' per-expert ranks (send_rank and
 * send_ecnt of moe_ep_dispatch_pack, exchanged with the local ids): the row
 * of a valid pick (s, slot, j) of local expert e is
 *   sum over s' < s of recv_ecnt[s', e]  +  recv_rank[s, slot, j],
 * which with metadata from moe_ep_dispatch_pack is the row
 * moe_ep_expert_batch gives (the vLLM alltoall_batched page's (source,
 * slot, column) order); expert_num_tokens[e] = the sum over all sources,
 * clamped to expert_cap. No receive scan runs and no workspace is needed:
 * one kernel moves the rows.
 *
 *   recv_rank     int32, same layout and stride as recv_eloc.
 *   recv_ecnt     int32, source s's [e_local] counts at
 *                 recv_ecnt + s * ecnt_rank_stride (elements, >= e_local).
 *   W * e_local <= 4096 (EINVAL otherwise).
 * Everything else as moe_ep_expert_batch. Data errors: a received local id
 * >= e_local is dropped (MOE_EP_ERR_ELOC); a valid pick whose rank is
 * negative or whose row reaches expert_cap is dropped (MOE_EP_ERR_ROWCAP);
 * counts are clamped to [0, expert_cap]. Rows follow the ranks as received:
 * metadata that did not come from moe_ep_dispatch_pack may give two picks
 * the same row.
 */
MOE_EP_API int moe_ep_expert_batch_ranked(const int32_t* recv_cnt, int64_t cnt_rank_stride,
                                          const int32_t* recv_eloc, const int32_t* recv_rank,
                                          int64_t eloc_rank_stride, const int32_t* recv_ecnt,
                                          int64_t ecnt_rank_stride, int32_t W,
                                          int32_t e_local, int32_t K, int64_t max_num_tokens,
                                          const moe_ep_payload* payloads, int32_t n_payloads,
                                          int32_t* expert_num_tokens, int32_t* recv_row,
                                          uint32_t* err_flags, void* stream);

/*
 * The two halves of moe_ep_expert_batch, for callers that overlap them with
 * the exchange: the plan needs only the counts and local ids (small, sent
 * ahead of the payload rows), the copy needs the payload rows. Arguments
 * mean what they mean for moe_ep_expert_batch.
 *
 * moe_ep_expert_batch_plan: scans the received metadata; writes
 * expert_num_tokens and, in the workspace and recv_row, the row plan.
 * moe_ep_expert_batch_copy: moves every payload row to its expert rows and
 * completes recv_row. It must follow the plan on the same stream with the
 * same metadata, recv_row and workspace (which must not be used by another
 * call in between). plan + copy == moe_ep_expert_batch.
 */
MOE_EP_API int moe_ep_expert_batch_plan(const int32_t* recv_cnt, int64_t cnt_rank_stride,
                                        const int32_t* recv_eloc, int64_t eloc_rank_stride,
                                        int32_t W, int32_t e_local, int32_t K,
                                        int64_t max_num_tokens,
                                        int32_t* expert_num_tokens, int32_t* recv_row,
                                        uint32_t* err_flags, void* workspace,
                                        size_t workspace_bytes, void* stream);

MOE_EP_API int moe_ep_expert_batch_copy(const int32_t* recv_cnt, int64_t cnt_rank_stride,
                                        const int32_t* recv_eloc, int64_t eloc_rank_stride,
                                        int32_t W, int32_t e_local, int32_t K,
                                        int64_t max_num_tokens,
                                        const moe_ep_payload* payloads, int32_t n_payloads,
                                        int32_t* recv_row, uint32_t* err_flags,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * Received expert ids for consumers that read the received slots in place
 * (the [W, cap, row] receive buffers, no expert batching), as the FlashInfer
 * module's moe_a2a_sanitize_expert_ids marks the ids of received entries
 * that are not valid tokens with a sentinel. Every entry of the
 * [W, cap, slots] layout is written: out[s, slot, j] = the local id of pick
 * j when slot < recv_cnt[s] and the id is in [0, e_local), else invalid_id.
 *
 *   recv_cnt, recv_eloc  as for moe_ep_expert_batch.
 *   out           int32; source s block [cap, slots] at
 *                 out + s * out_rank_stride (elements, >= cap * slots).
 *                 May be recv_eloc itself with the same stride (in place);
 *                 otherwise it must not overlap it.
 *   err_flags     nullable; bits MOE_EP_ERR_ELOC, MOE_EP_ERR_CNT.
 */
MOE_EP_API int moe_ep_sanitize_expert_ids(const int32_t* recv_cnt, int64_t cnt_rank_stride,
                                          const int32_t* recv_eloc, int64_t eloc_rank_stride,
                                          int32_t W, int32_t e_local, int32_t K,
                                          int64_t max_num_tokens, int32_t invalid_id,
                                          int32_t* out, int64_t out_rank_stride,
                                          uint32_t* err_flags, void* stream);

/*
 * Combine, on the destination rank (vLLM alltoall_batched page,
 * finalize(): one row per received slot, the weighted sum of its expert
 * rows, so one row per (source, token) pair goes back). For every
 * valid received slot (s, slot) and column h:
 *   acc = +0.0f; for j ascending with recv_row >= 0:
 *     acc = acc + (fp32(Y[e_j, row_j, h]) * w_j)   (product rounded to
 *                                                    fp32, no fused FMA)
 *   ret[s, slot, h] = acc, rounded to bf16 to nearest-even for MOE_EP_BF16.
 *
 *   expert_out    [e_local, W*cap, H] of dtype; expert e starts at
 *                 expert_out + e * expert_stride (elements), rows dense.
 *   recv_w        fp32, same layout and stride as recv_eloc
 *                 (meta_rank_stride elements between sources).
 *   recv_row      the context written by moe_ep_expert_batch.
 *   ret           [W, cap, H] of dtype; source s block at
 *                 ret + s * ret_rank_stride (elements, >= cap * H).
 */
MOE_EP_API int moe_ep_combine_reduce(const void* expert_out, int64_t expert_stride,
                          int32_t dtype, int64_t H,
                          const int32_t* recv_cnt, int64_t cnt_rank_stride,
                          const int32_t* recv_eloc, const float* recv_w,
                          int64_t meta_rank_stride, const int32_t* recv_row,
                          int32_t W, int32_t e_local, int32_t K,
                          int64_t max_num_tokens, void* ret,
                          int64_t ret_rank_stride, void* stream);

/*
 * Combine, on the source rank (vLLM alltoall_batched page, finalize():
 * a token's row adds up what each of its destinations returned).
 * out[t, h] = sum over d ascending with
 * token_slot[t, d] >= 0 of fp32(back[d, token_slot[t, d], h]), from +0.0f,
 * rounded once (bf16 to nearest-even). A token with no slot (padding)
 * gets +0.0. Every row of out is written.
 *
 *   back          [W, cap, H] of dtype; destination d block at
 *                 back + d * back_rank_stride (elements, >= cap * H).
 *   token_slot    the context written by moe_ep_dispatch_pack.
 *   out           [T, H] of dtype, dense.
 */
MOE_EP_API int moe_ep_combine_unpack(const void* back, int64_t back_rank_stride,
                          int32_t dtype, int64_t H, const int32_t* token_slot,
                          int64_t T, int32_t W, int64_t max_num_tokens,
                          void* out, void* stream);

/*
 * Fused combine of the local slice: the rank's own tokens that it also
 * serves as a destination. The FlashInfer module lets the expert kernel
 * write its output straight into the combine's input region to avoid a
 * staging copy; on one rank the same idea removes the partial of the local
 * slice altogether. The destination's reduce skips its own source and the
 * unpack reduces that term from the rank's own expert output. The result is
 * bit-identical to moe_ep_combine_reduce + moe_ep_combine_unpack: the local
 * term is summed over its picks and rounded to the data type exactly as the
 * reduce stores it, then added in its place in the ascending rank order.
 *
 * moe_ep_combine_reduce_peers: moe_ep_combine_reduce for every source except
 * self_src (in [0, W)), whose block of ret is neither read nor written.
 */
MOE_EP_API int moe_ep_combine_reduce_peers(const void* expert_out, int64_t expert_stride,
                          int32_t dtype, int64_t H,
                          const int32_t* recv_cnt, int64_t cnt_rank_stride,
                          const int32_t* recv_eloc, const float* recv_w,
                          int64_t meta_rank_stride, const int32_t* recv_row,
                          int32_t W, int32_t e_local, int32_t K,
                          int64_t max_num_tokens, int32_t self_src, void* ret,
                          int64_t ret_rank_stride, void* stream);

/*
 * moe_ep_combine_unpack_fused: moe_ep_combine_unpack on rank self_rank
 * (in [0, W)) where the term of destination self_rank is not read from back
 * but computed as moe_ep_combine_reduce computes it for received slot
 * token_slot[t, self_rank] of source self_rank:
 *
 *   expert_out, expert_stride   the rank's own expert output, as for
 *                 moe_ep_combine_reduce.
 *   self_eloc, self_w   [cap, slots] received metadata of the rank's own
 *                 source block (the receive view of source self_rank).
 *   self_row      [cap, slots] the moe_ep_expert_batch context of that block.
 *   e_local, K    as for moe_ep_expert_batch.
 * back's block of destination self_rank is not read. Every row of out is
 * written.
 */
MOE_EP_API int moe_ep_combine_unpack_fused(const void* back, int64_t back_rank_stride,
                          int32_t dtype, int64_t H, const int32_t* token_slot,
                          int64_t T, int32_t W, int64_t max_num_tokens,
                          int32_t self_rank, const void* expert_out,
                          int64_t expert_stride, const int32_t* self_eloc,
                          const float* self_w, const int32_t* self_row,
                          int32_t e_local, int32_t K, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EP_H */
