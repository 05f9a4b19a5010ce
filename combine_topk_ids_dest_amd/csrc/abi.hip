// C ABI of the dispatch/combine layout transform: argument checks,
// capacity and workspace queries, and the launch sequence of each call.
// Every check runs before anything is enqueued; no HIP runtime call is made
// unless all checks pass.
#include <limits.h>

#include <mutex>

#include "common.h"

using namespace moe_ep;

// Scratch of moe_ep_dispatch_pack_noalloc: the send side's workspace (tile
// counts, tile offsets, in-tile ranks) in a device array that the library
// holds on every GPU it runs on until the process ends. In host code this
// name is only a stand-in: kernels get the device address that
// hipGetSymbolAddress returns for the current device (scratch_address).
static __device__ __align__(256) uint8_t scratch[MOE_EP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept. The stream must belong to the
// current device: the address is per device.
int scratch_address(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_EP_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_EP_EINVAL;
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MOE_EP_EHIP;
        if (sdev != dev) return MOE_EP_EINVAL;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return MOE_EP_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_EP_OK;
}

constexpr int64_t kI32Max = INT_MAX;

inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

inline bool aligned16(const void* p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// stride >= rows * width (rows, width >= 0), compared without forming the
// product: caller-given sizes may be large enough to overflow it.
inline bool covers(int64_t stride, int64_t rows, int64_t width) {
    if (rows <= 0 || width <= 0) return stride >= 0;
    return stride / width >= rows;
}

// An element stride (eb = 2 or 4 bytes per element) that spans a multiple
// of 16 bytes.
inline bool stride16(int64_t stride, int eb) { return stride % (16 / eb) == 0; }

// Shapes common to every call; fills e_local, cap, slots, expert_cap.
struct Shape {
    int32_t W = 0, e_local = 0, slots = 0;
    int64_t cap = 0, expert_cap = 0;
};

int check_shape(int32_t K, int32_t e_local, int32_t W, int64_t max_num_tokens,
                Shape* sh) {
    // cap <= INT_MAX first (W * cap * slots < 2^31 needs it anyway), so the
    // products below cannot overflow
    if (K <= 0 || W <= 0 || W > MOE_EP_MAX_WORLD || e_local <= 0 ||
        e_local > MOE_EP_MAX_LOCAL_EXPERTS || max_num_tokens < 0 ||
        max_num_tokens > kI32Max)
        return MOE_EP_EINVAL;
    sh->W = W;
    sh->e_local = e_local;
    sh->slots = K < e_local ? K : e_local;
    if (sh->slots > MOE_EP_MAX_SLOTS) return MOE_EP_EINVAL;
    sh->cap = max_num_tokens;
    sh->expert_cap = max_num_tokens * W;
    if ((int64_t)W * sh->cap * sh->slots > kI32Max) return MOE_EP_EINVAL;
    return MOE_EP_OK;
}

// Workspace regions, each padded to 128 bytes.
struct PackWs {
    int64_t ntiles, cnt_off, off_off, rank_off;
    int64_t prank_off, ecnt_off, eoff_off;   // with the per-expert ranks
    int64_t bytes;
};
struct BatchWs { int64_t ntiles, cnt_off, off_off, bytes; };

// Send side: destination tile counts and offsets [tiles][W], in-tile ranks
// [W][T]; with the per-expert ranks also the in-tile ranks of the picks
// [T * K] and expert tile counts and offsets [tiles][E]. (T, W, K and E are
// bounded by the callers' checks, so nothing here overflows.)
PackWs pack_ws(int64_t T, int32_t W, int32_t K, int32_t E, bool ranked) {
    PackWs w;
    w.ntiles = (T + kRouteTile - 1) / kRouteTile;
    const int64_t region = round_up(w.ntiles * W * 4, 128);
    w.cnt_off = 0;
    w.off_off = region;
    w.rank_off = 2 * region;
    w.bytes = w.rank_off + round_up(T * W * 4, 128);
    w.prank_off = w.ecnt_off = w.eoff_off = 0;
    if (ranked) {
        const int64_t eregion = round_up(w.ntiles * E * 4, 128);
        w.prank_off = w.bytes;
        w.ecnt_off = w.prank_off + round_up(T * K * 4, 128);
        w.eoff_off = w.ecnt_off + eregion;
        w.bytes = w.eoff_off + eregion;
    }
    return w;
}

// The per-expert ranks fit their LDS tables for these sizes.
inline bool rank_sizes_ok(int32_t K, int32_t E) { return K <= kRankMaxK && E <= kRankMaxE; }

inline int id_bits(int32_t E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b;
}

BatchWs batch_ws(const Shape& sh) {
    BatchWs w;
    w.ntiles = ((int64_t)sh.W * sh.cap * sh.slots + kBatchTile - 1) / kBatchTile;
    const int64_t region = round_up(w.ntiles * sh.e_local * 4, 128);
    w.cnt_off = 0;
    w.off_off = region;
    w.bytes = 2 * region;
    return w;
}

// Checks the payload descriptors and fills the kernel argument. min_src and
// min_dst are the least leading-dim strides in units of row_bytes.
int check_payloads(const moe_ep_payload* payloads, int32_t n_payloads,
                   int64_t min_src_rows, int64_t min_dst_rows, bool need_ptrs,
                   PayloadSet* P) {
    if (n_payloads < 0 || n_payloads > MOE_EP_MAX_PAYLOADS) return MOE_EP_EINVAL;
    if (n_payloads > 0 && payloads == nullptr) return MOE_EP_EINVAL;
    P->n = n_payloads;
    for (int p = 0; p < MOE_EP_MAX_PAYLOADS; ++p) {
        P->src[p] = nullptr;
        P->dst[p] = nullptr;
        P->src_stride[p] = P->dst_stride[p] = P->row_bytes[p] = 0;
    }
    for (int p = 0; p < n_payloads; ++p) {
        const moe_ep_payload& d = payloads[p];
        if (d.row_bytes <= 0) return MOE_EP_EINVAL;
        if (need_ptrs && (d.src == nullptr || d.dst == nullptr)) return MOE_EP_EINVAL;
        if (d.row_bytes % 16 || d.src_stride % 16 || d.dst_stride % 16 ||
            !aligned16(d.src) || !aligned16(d.dst))
            return MOE_EP_EALIGN;
        if (!covers(d.src_stride, min_src_rows, d.row_bytes) ||
            !covers(d.dst_stride, min_dst_rows, d.row_bytes))
            return MOE_EP_EINVAL;
        P->src[p] = static_cast<const uint8_t*>(d.src);
        P->dst[p] = static_cast<uint8_t*>(d.dst);
        P->src_stride[p] = d.src_stride;
        P->dst_stride[p] = d.dst_stride;
        P->row_bytes[p] = d.row_bytes;
    }
    return MOE_EP_OK;
}

int elem_bytes(int32_t dtype) {
    if (dtype == MOE_EP_BF16) return 2;
    if (dtype == MOE_EP_F32) return 4;
    return 0;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_EP_OK : MOE_EP_EHIP; }

// Checks shared by the receive-side calls; fills sh and the workspace
// layout.
int check_batch(const int32_t* recv_cnt, int64_t cnt_rank_stride,
                const int32_t* recv_eloc, int64_t eloc_rank_stride, int32_t W,
                int32_t e_local, int32_t K, int64_t max_num_tokens,
                const int32_t* recv_row, void* workspace, size_t workspace_bytes,
                Shape* sh, BatchWs* ws) {
    int rc = check_shape(K, e_local, W, max_num_tokens, sh);
    if (rc) return rc;
    if (!recv_cnt || !recv_eloc || !recv_row) return MOE_EP_EINVAL;
    if (cnt_rank_stride < 1 || eloc_rank_stride < sh->cap * sh->slots)
        return MOE_EP_EINVAL;
    *ws = batch_ws(*sh);
    if (ws->bytes > 0 && (!workspace || workspace_bytes < (size_t)ws->bytes))
        return MOE_EP_EWORKSPACE;
    if (workspace && !aligned16(workspace)) return MOE_EP_EALIGN;
    return MOE_EP_OK;
}

int launch_plan(const int32_t* recv_cnt, int64_t cnt_rank_stride,
                const int32_t* recv_eloc, int64_t eloc_rank_stride,
                const Shape& sh, const BatchWs& ws, int32_t* expert_num_tokens,
                int32_t* recv_row, uint32_t* err_flags, void* workspace,
                hipStream_t st) {
    uint8_t* wsb = static_cast<uint8_t*>(workspace);
    int32_t* tile_cnt = reinterpret_cast<int32_t*>(wsb + ws.cnt_off);
    int32_t* tile_off = reinterpret_cast<int32_t*>(wsb + ws.off_off);
    const int32_t clamp = sh.expert_cap < kI32Max ? (int32_t)sh.expert_cap : INT_MAX;
    int rc = hip_status(launch_batch_local(recv_cnt, cnt_rank_stride, recv_eloc,
                                           eloc_rank_stride, sh.W, sh.e_local,
                                           sh.slots, sh.cap, (int)ws.ntiles,
                                           recv_row, tile_cnt, err_flags, st));
    if (rc) return rc;
    return hip_status(launch_column_scan(tile_cnt, (int)ws.ntiles, sh.e_local,
                                         tile_off, expert_num_tokens, clamp, st));
}

int launch_copy(const int32_t* recv_cnt, int64_t cnt_rank_stride,
                const int32_t* recv_eloc, int64_t eloc_rank_stride,
                const Shape& sh, const BatchWs& ws, const PayloadSet& P,
                int32_t* recv_row, uint32_t* err_flags, void* workspace,
                hipStream_t st) {
    uint8_t* wsb = static_cast<uint8_t*>(workspace);
    const int32_t* tile_off = reinterpret_cast<const int32_t*>(wsb + ws.off_off);
    return hip_status(launch_batch_copy(recv_cnt, cnt_rank_stride, recv_eloc,
                                        eloc_rank_stride, sh.W, sh.e_local,
                                        sh.slots, sh.cap, tile_off, nullptr, 0, nullptr,
                                        nullptr, 0, nullptr, 0, recv_row, P, err_flags, st));
}

}  // namespace

extern "C" {

int moe_ep_capacities(int32_t K, int32_t E, int32_t W, int64_t max_num_tokens,
                      int64_t* cap, int32_t* slots, int64_t* expert_cap) {
    if (!cap || !slots || !expert_cap) return MOE_EP_EINVAL;
    if (K <= 0 || E <= 0 || W <= 0 || E % W != 0 || max_num_tokens < 0 ||
        max_num_tokens > INT64_MAX / W)   // expert_cap would overflow
        return MOE_EP_EINVAL;
    const int32_t e_local = E / W;
    *cap = max_num_tokens;
    *slots = K < e_local ? K : e_local;
    *expert_cap = max_num_tokens * W;
    return MOE_EP_OK;
}

int moe_ep_workspace_bytes(int64_t T, int32_t K, int32_t E, int32_t W,
                           int64_t max_num_tokens, size_t* bytes) {
    if (!bytes || E <= 0 || W <= 0 || E % W != 0 || T < 0) return MOE_EP_EINVAL;
    if (T > max_num_tokens) return MOE_EP_ECAP;
    Shape sh;
    const int rc = check_shape(K, E / W, W, max_num_tokens, &sh);
    if (rc) return rc;
    // the send side with the per-expert ranks where they are supported
    const int64_t a = pack_ws(max_num_tokens, W, K, E, rank_sizes_ok(K, E)).bytes;
    const int64_t b = batch_ws(sh).bytes;
    *bytes = (size_t)(a > b ? a : b);
    return MOE_EP_OK;
}

const char* moe_ep_status_string(int status) {
    switch (status) {
        case MOE_EP_OK: return "ok";
        case MOE_EP_EINVAL: return "invalid argument";
        case MOE_EP_ECAP: return "more tokens than max_num_tokens";
        case MOE_EP_EDTYPE: return "unsupported combine data type";
        case MOE_EP_EALIGN: return "pointer, stride or row not 16-byte aligned";
        case MOE_EP_EWORKSPACE: return "workspace missing or too small";
        case MOE_EP_EHIP: return "HIP kernel launch failed";
        case MOE_EP_ESCRATCH:
            return "sizes need more scratch than the no-allocation entry point holds";
        default: return "unknown status";
    }
}

int moe_ep_combine_unpack_fused(const void* back, int64_t back_rank_stride,
                                int32_t dtype, int64_t H, const int32_t* token_slot,
                                int64_t T, int32_t W, int64_t max_num_tokens,
                                int32_t self_rank, const void* expert_out,
                                int64_t expert_stride, const int32_t* self_eloc,
                                const float* self_w, const int32_t* self_row,
                                int32_t e_local, int32_t K, void* out, void* stream) {
    Shape sh;
    int rc = check_shape(K, e_local, W, max_num_tokens, &sh);
    if (rc) return rc;
    if (T < 0 || H <= 0 || H > kI32Max || self_rank < 0 || self_rank >= W)
        return MOE_EP_EINVAL;
    const int eb = elem_bytes(dtype);
    if (eb == 0) return MOE_EP_EDTYPE;
    if (T > max_num_tokens) return MOE_EP_ECAP;
    if (T * W > kI32Max) return MOE_EP_EINVAL;
    if (T > 0 && (!back || !token_slot || !out || !expert_out || !self_eloc ||
                  !self_w || !self_row))
        return MOE_EP_EINVAL;
    if (!covers(back_rank_stride, max_num_tokens, H) ||
        !covers(expert_stride, sh.expert_cap, H))
        return MOE_EP_EINVAL;
    if ((H * eb) % 16 || !stride16(back_rank_stride, eb) || !stride16(expert_stride, eb) ||
        !aligned16(back) || !aligned16(out) || !aligned16(expert_out))
        return MOE_EP_EALIGN;
    return hip_status(launch_combine_unpack_fused(
        back, back_rank_stride, dtype, H, token_slot, T, W, sh.cap, self_rank,
        expert_out, expert_stride, self_eloc, self_w, self_row, e_local, sh.slots,
        out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

int dispatch(const int32_t* topk_ids, const float* topk_weights, int64_t T,
             int32_t K, int32_t E, int32_t W, int64_t max_num_tokens,
             const moe_ep_payload* payloads, int32_t n_payloads,
             const QuantArgs* quant, int32_t* send_cnt, int32_t* send_eloc,
             float* send_w, int64_t meta_rank_stride, int32_t* send_rank,
             int32_t* send_ecnt, int32_t* token_slot, uint32_t* err_flags,
             void* workspace, size_t workspace_bytes, void* stream,
             bool use_scratch = false) {
    if (E <= 0 || W <= 0 || E % W != 0 || T < 0) return MOE_EP_EINVAL;
    Shape sh;
    int rc = check_shape(K, E / W, W, max_num_tokens, &sh);
    if (rc) return rc;
    if (T > max_num_tokens) return MOE_EP_ECAP;
    if (T * K > kI32Max || T * W > kI32Max) return MOE_EP_EINVAL;
    if (!send_cnt || !send_eloc || !send_w) return MOE_EP_EINVAL;
    // destination blocks of the metadata: at least dense, and the offset of
    // the last block must fit in int64_t
    if (meta_rank_stride < sh.cap * sh.slots || meta_rank_stride > INT64_MAX / W)
        return MOE_EP_EINVAL;
    // the per-expert ranks: both outputs or neither, within their limits
    const bool ranked = send_rank != nullptr || send_ecnt != nullptr;
    if (ranked && (!send_rank || !send_ecnt || !rank_sizes_ok(K, E))) return MOE_EP_EINVAL;
    if (T > 0 && (!topk_ids || !topk_weights || !token_slot)) return MOE_EP_EINVAL;
    PayloadSet P;
    rc = check_payloads(payloads, n_payloads, 1, sh.cap, T > 0, &P);
    if (rc) return rc;
    if (quant && quant->mode == 1) {
        const QuantArgs& Q = *quant;
        if (Q.group != 32 && Q.group != 64 && Q.group != 128) return MOE_EP_EINVAL;
        if (Q.H <= 0 || Q.H > kI32Max || Q.H % Q.group) return MOE_EP_EINVAL;
        if (T > 0 && (!Q.src || !Q.q || !Q.s)) return MOE_EP_EINVAL;
        if (!covers(Q.src_stride, 2, Q.H) || !covers(Q.q_stride, sh.cap, Q.H) ||
            !covers(Q.s_stride, sh.cap, Q.s_pitch))
            return MOE_EP_EINVAL;
        if (!aligned16(Q.src) || Q.src_stride % 16 || (reinterpret_cast<uintptr_t>(Q.q) & 15) ||
            Q.q_stride % 16 || (reinterpret_cast<uintptr_t>(Q.s) & 3))
            return MOE_EP_EALIGN;
    } else if (quant) {
        const QuantArgs& Q = *quant;
        if (Q.H <= 0 || Q.H > kI32Max) return MOE_EP_EINVAL;
        if (T > 0 && (!Q.src || !Q.q || !Q.s)) return MOE_EP_EINVAL;
        if (!covers(Q.src_stride, 2, Q.H) || !covers(Q.q_stride, sh.cap, Q.H / 2) ||
            !covers(Q.s_stride, sh.cap, Q.s_pitch))
            return MOE_EP_EINVAL;
        // code rows of H/2 bytes, like every travelling row, are 16-byte multiples
        if (Q.H % 32 || !aligned16(Q.src) || Q.src_stride % 16 || !aligned16(Q.q) ||
            Q.q_stride % 16 || !aligned16(Q.s) || Q.s_stride % 16)
            return MOE_EP_EALIGN;
    }
    const PackWs ws = pack_ws(T, W, K, E, ranked);
    // one tile of tokens needs no workspace (the pack routes by itself)
    const bool own_route = T > 0 && T <= kRouteTile;
    if (use_scratch) {
        if (ws.bytes > (int64_t)MOE_EP_NOALLOC_SCRATCH_BYTES) return MOE_EP_ESCRATCH;
    } else {
        if (ws.bytes > 0 && (!workspace || workspace_bytes < (size_t)ws.bytes))
            return MOE_EP_EWORKSPACE;
        if (workspace && !aligned16(workspace)) return MOE_EP_EALIGN;
    }

    hipStream_t st = static_cast<hipStream_t>(stream);
    if (use_scratch && !own_route) {
        rc = scratch_address(st, &workspace);
        if (rc) return rc;
    }
    uint8_t* wsb = static_cast<uint8_t*>(workspace);
    int32_t* tile_cnt = reinterpret_cast<int32_t*>(wsb + ws.cnt_off);
    int32_t* tile_off = reinterpret_cast<int32_t*>(wsb + ws.off_off);
    int32_t* rank = reinterpret_cast<int32_t*>(wsb + ws.rank_off);
    RankArgs R{};
    if (ranked) {
        R.send_rank = send_rank;
        R.send_ecnt = send_ecnt;
        R.nbits = id_bits(E);
    }

    // One tile of tokens (decode-sized batches): pack_copy routes by itself
    // and writes send_cnt (and, ranked, the ranks and send_ecnt); no
    // separate routing launch.
    if (own_route)
        return hip_status(launch_pack_copy(topk_ids, topk_weights, T, K, E,
                                           sh.e_local, W, sh.slots, sh.cap, nullptr,
                                           token_slot, nullptr, nullptr, send_cnt, P,
                                           quant, send_eloc, send_w, meta_rank_stride,
                                           ranked ? &R : nullptr, err_flags, st));
    int32_t* prank = ranked ? reinterpret_cast<int32_t*>(wsb + ws.prank_off) : nullptr;
    int32_t* ecnt_tile = ranked ? reinterpret_cast<int32_t*>(wsb + ws.ecnt_off) : nullptr;
    int32_t* eoff_tile = ranked ? reinterpret_cast<int32_t*>(wsb + ws.eoff_off) : nullptr;
    rc = hip_status(launch_route_local(topk_ids, T, K, E, sh.e_local, W, sh.slots,
                                       rank, tile_cnt, prank, ecnt_tile, R.nbits,
                                       err_flags, st));
    if (rc) return rc;
    // Few tiles (or none): pack_copy sums the tile counts itself; the scan
    // kernels still run for T = 0 so that send_cnt (and send_ecnt) are
    // written.
    const bool fused = ws.ntiles > 0 && ws.ntiles <= kPackFuseTiles;
    if (!fused) {
        rc = hip_status(launch_column_scan(tile_cnt, (int)ws.ntiles, W, tile_off,
                                           send_cnt, INT_MAX, st));
        if (rc) return rc;
        if (ranked) {
            rc = hip_status(launch_column_scan(ecnt_tile, (int)ws.ntiles, E, eoff_tile,
                                               send_ecnt, INT_MAX, st));
            if (rc) return rc;
        }
    }
    if (ranked) {
        R.prank = prank;
        R.ecnt_tile = ecnt_tile;
        R.eoff_tile = fused ? nullptr : eoff_tile;
    }
    return hip_status(launch_pack_copy(topk_ids, topk_weights, T, K, E,
                                       sh.e_local, W, sh.slots, sh.cap, rank,
                                       token_slot, fused ? tile_cnt : nullptr,
                                       tile_off, send_cnt, P, quant, send_eloc,
                                       send_w, meta_rank_stride, ranked ? &R : nullptr,
                                       err_flags, st));
}

}  // namespace

extern "C" {

int moe_ep_dispatch_pack(const int32_t* topk_ids, const float* topk_weights,
                         int64_t T, int32_t K, int32_t E, int32_t W,
                         int64_t max_num_tokens,
                         const moe_ep_payload* payloads, int32_t n_payloads,
                         int32_t* send_cnt, int32_t* send_eloc, float* send_w,
                         int64_t meta_rank_stride, int32_t* send_rank, int32_t* send_ecnt,
                         int32_t* token_slot, uint32_t* err_flags, void* workspace,
                         size_t workspace_bytes, void* stream) {
    return dispatch(topk_ids, topk_weights, T, K, E, W, max_num_tokens, payloads,
                    n_payloads, nullptr, send_cnt, send_eloc, send_w, meta_rank_stride,
                    send_rank, send_ecnt, token_slot, err_flags, workspace,
                    workspace_bytes, stream);
}

int moe_ep_dispatch_pack_noalloc(const int32_t* topk_ids, const float* topk_weights,
                                 int64_t T, int32_t K, int32_t E, int32_t W,
                                 int64_t max_num_tokens,
                                 const moe_ep_payload* payloads, int32_t n_payloads,
                                 int32_t* send_cnt, int32_t* send_eloc, float* send_w,
                                 int64_t meta_rank_stride, int32_t* send_rank,
                                 int32_t* send_ecnt, int32_t* token_slot,
                                 uint32_t* err_flags, void* stream) {
    return dispatch(topk_ids, topk_weights, T, K, E, W, max_num_tokens, payloads,
                    n_payloads, nullptr, send_cnt, send_eloc, send_w, meta_rank_stride,
                    send_rank, send_ecnt, token_slot, err_flags, nullptr, 0, stream, true);
}

int moe_ep_dispatch_pack_fp8(const int32_t* topk_ids, const float* topk_weights,
                             int64_t T, int32_t K, int32_t E, int32_t W,
                             int64_t max_num_tokens, const void* hidden,
                             int64_t hidden_stride, int64_t H, int32_t group,
                             void* send_q, int64_t q_rank_stride,
                             float* send_scale, int64_t scale_rank_stride,
                             const moe_ep_payload* payloads, int32_t n_payloads,
                             int32_t* send_cnt, int32_t* send_eloc, float* send_w,
                             int64_t meta_rank_stride, int32_t* send_rank,
                             int32_t* send_ecnt, int32_t* token_slot, uint32_t* err_flags,
                             void* workspace, size_t workspace_bytes, void* stream) {
    QuantArgs Q;
    Q.src = static_cast<const uint8_t*>(hidden);
    Q.src_stride = hidden_stride;
    Q.q = static_cast<uint8_t*>(send_q);
    Q.q_stride = q_rank_stride;
    Q.s = reinterpret_cast<uint8_t*>(send_scale);
    // floats -> bytes; a stride whose byte count overflows becomes -1,
    // which the stride check rejects
    Q.s_stride = scale_rank_stride < 0 || scale_rank_stride > INT64_MAX / 4
                     ? -1 : scale_rank_stride * 4;
    Q.H = H;
    Q.group = group;
    Q.n_scales = group > 0 ? H / group : 0;
    Q.s_pitch = (Q.n_scales + 3) / 4 * 4 * 4;
    Q.mode = 1;
    return dispatch(topk_ids, topk_weights, T, K, E, W, max_num_tokens, payloads,
                    n_payloads, &Q, send_cnt, send_eloc, send_w, meta_rank_stride,
                    send_rank, send_ecnt, token_slot, err_flags, workspace,
                    workspace_bytes, stream);
}

int moe_ep_dispatch_pack_fp4(const int32_t* topk_ids, const float* topk_weights,
                             int64_t T, int32_t K, int32_t E, int32_t W,
                             int64_t max_num_tokens, const void* hidden,
                             int64_t hidden_stride, int64_t H, void* send_q,
                             int64_t q_rank_stride, void* send_scale,
                             int64_t scale_rank_stride,
                             const moe_ep_payload* payloads, int32_t n_payloads,
                             int32_t* send_cnt, int32_t* send_eloc, float* send_w,
                             int64_t meta_rank_stride, int32_t* send_rank,
                             int32_t* send_ecnt, int32_t* token_slot, uint32_t* err_flags,
                             void* workspace, size_t workspace_bytes, void* stream) {
    QuantArgs Q;
    Q.src = static_cast<const uint8_t*>(hidden);
    Q.src_stride = hidden_stride;
    Q.q = static_cast<uint8_t*>(send_q);
    Q.q_stride = q_rank_stride;
    Q.s = static_cast<uint8_t*>(send_scale);
    Q.s_stride = scale_rank_stride;
    Q.H = H;
    Q.group = 16;
    Q.n_scales = H / 16;
    Q.s_pitch = (Q.n_scales + 15) / 16 * 16;
    Q.mode = 2;
    return dispatch(topk_ids, topk_weights, T, K, E, W, max_num_tokens, payloads,
                    n_payloads, &Q, send_cnt, send_eloc, send_w, meta_rank_stride,
                    send_rank, send_ecnt, token_slot, err_flags, workspace,
                    workspace_bytes, stream);
}

int moe_ep_expert_batch_plan(const int32_t* recv_cnt, int64_t cnt_rank_stride,
                             const int32_t* recv_eloc, int64_t eloc_rank_stride,
                             int32_t W, int32_t e_local, int32_t K,
                             int64_t max_num_tokens, int32_t* expert_num_tokens,
                             int32_t* recv_row, uint32_t* err_flags,
                             void* workspace, size_t workspace_bytes,
                             void* stream) {
    Shape sh;
    BatchWs ws;
    int rc = check_batch(recv_cnt, cnt_rank_stride, recv_eloc, eloc_rank_stride,
                         W, e_local, K, max_num_tokens, recv_row, workspace,
                         workspace_bytes, &sh, &ws);
    if (rc) return rc;
    if (!expert_num_tokens) return MOE_EP_EINVAL;
    return launch_plan(recv_cnt, cnt_rank_stride, recv_eloc, eloc_rank_stride, sh,
                       ws, expert_num_tokens, recv_row, err_flags, workspace,
                       static_cast<hipStream_t>(stream));
}

int moe_ep_expert_batch_copy(const int32_t* recv_cnt, int64_t cnt_rank_stride,
                             const int32_t* recv_eloc, int64_t eloc_rank_stride,
                             int32_t W, int32_t e_local, int32_t K,
                             int64_t max_num_tokens,
                             const moe_ep_payload* payloads, int32_t n_payloads,
                             int32_t* recv_row, uint32_t* err_flags,
                             void* workspace, size_t workspace_bytes,
                             void* stream) {
    Shape sh;
    BatchWs ws;
    int rc = check_batch(recv_cnt, cnt_rank_stride, recv_eloc, eloc_rank_stride,
                         W, e_local, K, max_num_tokens, recv_row, workspace,
                         workspace_bytes, &sh, &ws);
    if (rc) return rc;
    PayloadSet P;
    rc = check_payloads(payloads, n_payloads, sh.cap, sh.expert_cap, true, &P);
    if (rc) return rc;
    return launch_copy(recv_cnt, cnt_rank_stride, recv_eloc, eloc_rank_stride, sh,
                       ws, P, recv_row, err_flags, workspace,
                       static_cast<hipStream_t>(stream));
}

int moe_ep_expert_batch(const int32_t* recv_cnt, int64_t cnt_rank_stride,
                        const int32_t* recv_eloc, int64_t eloc_rank_stride,
                        int32_t W, int32_t e_local, int32_t K,
                        int64_t max_num_tokens,
                        const moe_ep_payload* payloads, int32_t n_payloads,
                        int32_t* expert_num_tokens, int32_t* recv_row,
                        uint32_t* err_flags, void* workspace,
                        size_t workspace_bytes, void* stream) {
    Shape sh;
    BatchWs ws;
    int rc = check_batch(recv_cnt, cnt_rank_stride, recv_eloc, eloc_rank_stride,
                         W, e_local, K, max_num_tokens, recv_row, workspace,
                         workspace_bytes, &sh, &ws);
    if (rc) return rc;
    if (!expert_num_tokens) return MOE_EP_EINVAL;
    PayloadSet P;
    rc = check_payloads(payloads, n_payloads, sh.cap, sh.expert_cap, true, &P);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // Few tiles: no column_scan; the copy sums the tile offsets and writes
    // expert_num_tokens (the result is the same as plan + copy).
    if (ws.ntiles > 0 && ws.ntiles <= kBatchFuseTiles) {
        uint8_t* wsb = static_cast<uint8_t*>(workspace);
        int32_t* tile_cnt = reinterpret_cast<int32_t*>(wsb + ws.cnt_off);
        const int32_t clamp = sh.expert_cap < kI32Max ? (int32_t)sh.expert_cap : INT_MAX;
        rc = hip_status(launch_batch_local(recv_cnt, cnt_rank_stride, recv_eloc,
                                           eloc_rank_stride, sh.W, sh.e_local, sh.slots,
                                           sh.cap, (int)ws.ntiles, recv_row, tile_cnt,
                                           err_flags, st));
        if (rc) return rc;
        return hip_status(launch_batch_copy(recv_cnt, cnt_rank_stride, recv_eloc,
                                            eloc_rank_stride, sh.W, sh.e_local, sh.slots,
                                            sh.cap, nullptr, tile_cnt, (int)ws.ntiles,
                                            nullptr, nullptr, 0, expert_num_tokens, clamp,
                                            recv_row, P, err_flags, st));
    }
    rc = launch_plan(recv_cnt, cnt_rank_stride, recv_eloc, eloc_rank_stride, sh, ws,
                     expert_num_tokens, recv_row, err_flags, workspace, st);
    if (rc) return rc;
    return launch_copy(recv_cnt, cnt_rank_stride, recv_eloc, eloc_rank_stride, sh, ws,
                       P, recv_row, err_flags, workspace, st);
}

int moe_ep_expert_batch_ranked(const int32_t* recv_cnt, int64_t cnt_rank_stride,
                               const int32_t* recv_eloc, const int32_t* recv_rank,
                               int64_t eloc_rank_stride, const int32_t* recv_ecnt,
                               int64_t ecnt_rank_stride, int32_t W, int32_t e_local,
                               int32_t K, int64_t max_num_tokens,
                               const moe_ep_payload* payloads, int32_t n_payloads,
                               int32_t* expert_num_tokens, int32_t* recv_row,
                               uint32_t* err_flags, void* stream) {
    Shape sh;
    int rc = check_shape(K, e_local, W, max_num_tokens, &sh);
    if (rc) return rc;
    if (!recv_cnt || !recv_eloc || !recv_rank || !recv_ecnt || !expert_num_tokens ||
        !recv_row)
        return MOE_EP_EINVAL;
    // the ranks come from packs limited to E = W * e_local <= kRankMaxE; the
    // receive side takes the same limit, so the form has one domain
    if (!rank_sizes_ok(1, W * e_local)) return MOE_EP_EINVAL;
    if (cnt_rank_stride < 1 || eloc_rank_stride < sh.cap * sh.slots ||
        ecnt_rank_stride < e_local)
        return MOE_EP_EINVAL;
    PayloadSet P;
    rc = check_payloads(payloads, n_payloads, sh.cap, sh.expert_cap, true, &P);
    if (rc) return rc;
    const int32_t clamp = sh.expert_cap < kI32Max ? (int32_t)sh.expert_cap : INT_MAX;
    return hip_status(launch_batch_copy(recv_cnt, cnt_rank_stride, recv_eloc,
                                        eloc_rank_stride, sh.W, sh.e_local, sh.slots,
                                        sh.cap, nullptr, nullptr, 0, recv_rank, recv_ecnt,
                                        ecnt_rank_stride, expert_num_tokens, clamp,
                                        recv_row, P, err_flags,
                                        static_cast<hipStream_t>(stream)));
}

int moe_ep_sanitize_expert_ids(const int32_t* recv_cnt, int64_t cnt_rank_stride,
                               const int32_t* recv_eloc, int64_t eloc_rank_stride,
                               int32_t W, int32_t e_local, int32_t K,
                               int64_t max_num_tokens, int32_t invalid_id,
                               int32_t* out, int64_t out_rank_stride,
                               uint32_t* err_flags, void* stream) {
    Shape sh;
    int rc = check_shape(K, e_local, W, max_num_tokens, &sh);
    if (rc) return rc;
    if (!recv_cnt || !recv_eloc || !out) return MOE_EP_EINVAL;
    if (cnt_rank_stride < 1 || eloc_rank_stride < sh.cap * sh.slots ||
        out_rank_stride < sh.cap * sh.slots)
        return MOE_EP_EINVAL;
    if (out == recv_eloc && out_rank_stride != eloc_rank_stride) return MOE_EP_EINVAL;
    return hip_status(launch_sanitize_ids(recv_cnt, cnt_rank_stride, recv_eloc,
                                          eloc_rank_stride, W, e_local, sh.slots,
                                          sh.cap, invalid_id, out, out_rank_stride,
                                          err_flags, static_cast<hipStream_t>(stream)));
}

static int combine_reduce(const void* expert_out, int64_t expert_stride,
                          int32_t dtype, int64_t H,
                          const int32_t* recv_cnt, int64_t cnt_rank_stride,
                          const int32_t* recv_eloc, const float* recv_w,
                          int64_t meta_rank_stride, const int32_t* recv_row,
                          int32_t W, int32_t e_local, int32_t K,
                          int64_t max_num_tokens, void* ret,
                          int64_t ret_rank_stride, int32_t skip_src, void* stream) {
    Shape sh;
    int rc = check_shape(K, e_local, W, max_num_tokens, &sh);
    if (rc) return rc;
    const int eb = elem_bytes(dtype);
    if (eb == 0) return MOE_EP_EDTYPE;
    if (H <= 0 || H > kI32Max) return MOE_EP_EINVAL;
    if (!expert_out || !recv_cnt || !recv_eloc || !recv_w || !recv_row || !ret)
        return MOE_EP_EINVAL;
    if (cnt_rank_stride < 1 || meta_rank_stride < sh.cap * sh.slots ||
        !covers(expert_stride, sh.expert_cap, H) || !covers(ret_rank_stride, sh.cap, H))
        return MOE_EP_EINVAL;
    if ((H * eb) % 16 || !stride16(expert_stride, eb) || !stride16(ret_rank_stride, eb) ||
        !aligned16(expert_out) || !aligned16(ret))
        return MOE_EP_EALIGN;
    return hip_status(launch_combine_reduce(
        expert_out, expert_stride, dtype, H, recv_cnt, cnt_rank_stride,
        recv_eloc, recv_w, meta_rank_stride, recv_row, W, e_local, sh.slots,
        sh.cap, ret, ret_rank_stride, skip_src, static_cast<hipStream_t>(stream)));
}

int moe_ep_combine_reduce(const void* expert_out, int64_t expert_stride,
                          int32_t dtype, int64_t H,
                          const int32_t* recv_cnt, int64_t cnt_rank_stride,
                          const int32_t* recv_eloc, const float* recv_w,
                          int64_t meta_rank_stride, const int32_t* recv_row,
                          int32_t W, int32_t e_local, int32_t K,
                          int64_t max_num_tokens, void* ret,
                          int64_t ret_rank_stride, void* stream) {
    return combine_reduce(expert_out, expert_stride, dtype, H, recv_cnt,
                          cnt_rank_stride, recv_eloc, recv_w, meta_rank_stride,
                          recv_row, W, e_local, K, max_num_tokens, ret,
                          ret_rank_stride, -1, stream);
}

int moe_ep_combine_reduce_peers(const void* expert_out, int64_t expert_stride,
                                int32_t dtype, int64_t H,
                                const int32_t* recv_cnt, int64_t cnt_rank_stride,
                                const int32_t* recv_eloc, const float* recv_w,
                                int64_t meta_rank_stride, const int32_t* recv_row,
                                int32_t W, int32_t e_local, int32_t K,
                                int64_t max_num_tokens, int32_t self_src, void* ret,
                                int64_t ret_rank_stride, void* stream) {
    if (W > 0 && (self_src < 0 || self_src >= W)) return MOE_EP_EINVAL;
    return combine_reduce(expert_out, expert_stride, dtype, H, recv_cnt,
                          cnt_rank_stride, recv_eloc, recv_w, meta_rank_stride,
                          recv_row, W, e_local, K, max_num_tokens, ret,
                          ret_rank_stride, self_src, stream);
}

int moe_ep_combine_unpack(const void* back, int64_t back_rank_stride,
                          int32_t dtype, int64_t H, const int32_t* token_slot,
                          int64_t T, int32_t W, int64_t max_num_tokens,
                          void* out, void* stream) {
    if (W <= 0 || W > MOE_EP_MAX_WORLD || T < 0 || max_num_tokens < 0 ||
        max_num_tokens > kI32Max || H <= 0 || H > kI32Max)
        return MOE_EP_EINVAL;
    const int eb = elem_bytes(dtype);
    if (eb == 0) return MOE_EP_EDTYPE;
    if (T > max_num_tokens) return MOE_EP_ECAP;
    if (T * W > kI32Max) return MOE_EP_EINVAL;
    if (T > 0 && (!back || !token_slot || !out)) return MOE_EP_EINVAL;
    if (!covers(back_rank_stride, max_num_tokens, H)) return MOE_EP_EINVAL;
    if ((H * eb) % 16 || !stride16(back_rank_stride, eb) || !aligned16(back) ||
        !aligned16(out))
        return MOE_EP_EALIGN;
    return hip_status(launch_combine_unpack(back, back_rank_stride, dtype, H,
                                            token_slot, T, W, max_num_tokens, out,
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"
