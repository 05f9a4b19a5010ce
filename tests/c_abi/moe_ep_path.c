/*
 * The whole dispatch/combine path for W logical ranks on one GPU through
 * the C ABI of libmoe_ep.so alone: plain C99, HIP runtime calls for device
 * memory and copies, no torch and no Python. tests/test_gpu_c_abi.py runs it
 * on seeded inputs and compares what it writes with the oracle.
 *
 * The exchanges of the vLLM alltoall_batched page (prepare(): rows, counts
 * and metadata to their destinations; finalize(): partials back to their
 * sources) are rank-stride views of buffers laid out [source][destination]
 * and [destination][source]. The experts are the identity: expert e's output
 * rows are its batched input rows.
 *
 * usage: moe_ep_path <in.bin> <out.bin>
 *   in.bin   int64 T, H, E, K, W, max_num_tokens; then per source s:
 *            int32 topk_ids[T*K], float topk_weights[T*K],
 *            uint16 hidden[T*H] (bf16 bits)
 *   out.bin  per source s: int32 send_cnt[W], int32 token_slot[T*W],
 *            uint16 out[T*H];
 *            per destination r: int32 expert_num_tokens[e_local];
 *            uint32 err_flags
 * Exit status 0 on success; otherwise a message names the failing call.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_ep.h"

static void fail(const char* what, const char* why) {
    fprintf(stderr, "moe_ep_path: %s: %s\n", what, why);
    exit(1);
}

static void check_hip(hipError_t e, const char* what) {
    if (e != hipSuccess) fail(what, hipGetErrorString(e));
}

static void check(int status, const char* what) {
    if (status != MOE_EP_OK) fail(what, moe_ep_status_string(status));
}

static void* dev_alloc(size_t bytes, const char* what) {
    void* p = NULL;
    check_hip(hipMalloc(&p, bytes > 0 ? bytes : 16), what);
    return p;
}

static void read_exact(FILE* f, void* p, size_t bytes) {
    if (bytes && fread(p, 1, bytes, f) != bytes) fail("read", "input file too short");
}

static void write_exact(FILE* f, const void* p, size_t bytes) {
    if (bytes && fwrite(p, 1, bytes, f) != bytes) fail("write", "output file");
}

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s <in.bin> <out.bin>\n", argv[0]);
        return 2;
    }
    FILE* in = fopen(argv[1], "rb");
    if (!in) fail("open", argv[1]);
    int64_t hdr[6];
    read_exact(in, hdr, sizeof hdr);
    const int64_t T = hdr[0], H = hdr[1];
    const int32_t E = (int32_t)hdr[2], K = (int32_t)hdr[3], W = (int32_t)hdr[4];
    const int64_t max_num_tokens = hdr[5];

    int64_t cap = 0, expert_cap = 0;
    int32_t slots = 0;
    check(moe_ep_capacities(K, E, W, max_num_tokens, &cap, &slots, &expert_cap),
          "moe_ep_capacities");
    const int32_t e_local = E / W;
    size_t ws_bytes = 0;
    check(moe_ep_workspace_bytes(T, K, E, W, max_num_tokens, &ws_bytes),
          "moe_ep_workspace_bytes");

    /* host inputs, per source */
    const size_t n_tk = (size_t)(T * K), n_th = (size_t)(T * H);
    int32_t* h_ids = malloc(sizeof(int32_t) * n_tk * W + 1);
    float* h_wts = malloc(sizeof(float) * n_tk * W + 1);
    uint16_t* h_hid = malloc(sizeof(uint16_t) * n_th * W + 1);
    if (!h_ids || !h_wts || !h_hid) fail("malloc", "inputs");
    for (int32_t s = 0; s < W; ++s) {
        read_exact(in, h_ids + s * n_tk, sizeof(int32_t) * n_tk);
        read_exact(in, h_wts + s * n_tk, sizeof(float) * n_tk);
        read_exact(in, h_hid + s * n_th, sizeof(uint16_t) * n_th);
    }
    fclose(in);

    /* device buffers; [src][dst] for what the packs write, [dst][src] for
       what the reduces write */
    const int64_t row = 2 * H;                              /* bf16 row bytes */
    const int64_t meta_block = cap * slots;                 /* elements */
    int32_t* ids = dev_alloc(sizeof(int32_t) * n_tk * W, "ids");
    float* wts = dev_alloc(sizeof(float) * n_tk * W, "weights");
    uint8_t* hidden = dev_alloc((size_t)row * T * W, "hidden");
    uint8_t* send = dev_alloc((size_t)row * cap * W * W, "send");
    int32_t* send_cnt = dev_alloc(sizeof(int32_t) * W * W, "send_cnt");
    int32_t* send_eloc = dev_alloc(sizeof(int32_t) * meta_block * W * W, "send_eloc");
    float* send_w = dev_alloc(sizeof(float) * meta_block * W * W, "send_w");
    int32_t* token_slot = dev_alloc(sizeof(int32_t) * T * W * W, "token_slot");
    uint8_t* batch = dev_alloc((size_t)row * expert_cap * e_local * W, "expert batch");
    int32_t* expert_num_tokens = dev_alloc(sizeof(int32_t) * e_local * W, "expert_num_tokens");
    int32_t* recv_row = dev_alloc(sizeof(int32_t) * meta_block * W * W, "recv_row");
    uint8_t* ret = dev_alloc((size_t)row * cap * W * W, "ret");
    uint8_t* out = dev_alloc((size_t)row * T * W, "out");
    uint32_t* err = dev_alloc(sizeof(uint32_t), "err_flags");
    void* ws = dev_alloc(ws_bytes, "workspace");
    check_hip(hipMemcpy(ids, h_ids, sizeof(int32_t) * n_tk * W, hipMemcpyHostToDevice), "copy ids");
    check_hip(hipMemcpy(wts, h_wts, sizeof(float) * n_tk * W, hipMemcpyHostToDevice), "copy weights");
    check_hip(hipMemcpy(hidden, h_hid, (size_t)row * T * W, hipMemcpyHostToDevice), "copy hidden");
    check_hip(hipMemset(err, 0, sizeof(uint32_t)), "clear err_flags");
    void* stream = NULL;   /* the null stream: every call in order */

    /* dispatch, send side of every source */
    for (int32_t s = 0; s < W; ++s) {
        moe_ep_payload p;
        p.src = hidden + (size_t)s * T * row;
        p.src_stride = row;
        p.dst = send + (size_t)s * W * cap * row;
        p.dst_stride = cap * row;
        p.row_bytes = row;
        check(moe_ep_dispatch_pack(ids + s * n_tk, wts + s * n_tk, T, K, E, W, max_num_tokens,
                                   &p, 1, send_cnt + s * W, send_eloc + (size_t)s * W * meta_block,
                                   send_w + (size_t)s * W * meta_block, meta_block, NULL, NULL,
                                   token_slot + (size_t)s * T * W, err, ws, ws_bytes, stream),
              "moe_ep_dispatch_pack");
    }
    /* receive side and combine reduce of every destination: source s's block
       for destination r is [s][r] of the send-side buffers */
    for (int32_t r = 0; r < W; ++r) {
        moe_ep_payload p;
        p.src = send + (size_t)r * cap * row;
        p.src_stride = W * cap * row;
        p.dst = batch + (size_t)r * e_local * expert_cap * row;
        p.dst_stride = expert_cap * row;
        p.row_bytes = row;
        int32_t* rrow = recv_row + (size_t)r * W * meta_block;
        check(moe_ep_expert_batch(send_cnt + r, W, send_eloc + (size_t)r * meta_block,
                                  W * meta_block, W, e_local, K, max_num_tokens, &p, 1,
                                  expert_num_tokens + r * e_local, rrow, err, ws, ws_bytes,
                                  stream),
              "moe_ep_expert_batch");
        check(moe_ep_combine_reduce(batch + (size_t)r * e_local * expert_cap * row,
                                    expert_cap * H, MOE_EP_BF16, H, send_cnt + r, W,
                                    send_eloc + (size_t)r * meta_block,
                                    send_w + (size_t)r * meta_block, W * meta_block, rrow, W,
                                    e_local, K, max_num_tokens,
                                    ret + (size_t)r * W * cap * row, cap * H, stream),
              "moe_ep_combine_reduce");
    }
    /* combine unpack of every source: destination d's partial for source s
       is [d][s] of ret */
    for (int32_t s = 0; s < W; ++s) {
        check(moe_ep_combine_unpack(ret + (size_t)s * cap * row, W * cap * H, MOE_EP_BF16, H,
                                    token_slot + (size_t)s * T * W, T, W, max_num_tokens,
                                    out + (size_t)s * T * row, stream),
              "moe_ep_combine_unpack");
    }
    check_hip(hipDeviceSynchronize(), "synchronize");

    /* results */
    int32_t* h_cnt = malloc(sizeof(int32_t) * W * W + 1);
    int32_t* h_slot = malloc(sizeof(int32_t) * T * W * W + 1);
    uint16_t* h_out = malloc((size_t)row * T * W + 1);
    int32_t* h_ent = malloc(sizeof(int32_t) * e_local * W + 1);
    uint32_t h_err = 0;
    if (!h_cnt || !h_slot || !h_out || !h_ent) fail("malloc", "outputs");
    check_hip(hipMemcpy(h_cnt, send_cnt, sizeof(int32_t) * W * W, hipMemcpyDeviceToHost), "copy send_cnt");
    check_hip(hipMemcpy(h_slot, token_slot, sizeof(int32_t) * T * W * W, hipMemcpyDeviceToHost), "copy token_slot");
    check_hip(hipMemcpy(h_out, out, (size_t)row * T * W, hipMemcpyDeviceToHost), "copy out");
    check_hip(hipMemcpy(h_ent, expert_num_tokens, sizeof(int32_t) * e_local * W, hipMemcpyDeviceToHost), "copy expert_num_tokens");
    check_hip(hipMemcpy(&h_err, err, sizeof(uint32_t), hipMemcpyDeviceToHost), "copy err_flags");
    FILE* o = fopen(argv[2], "wb");
    if (!o) fail("open", argv[2]);
    for (int32_t s = 0; s < W; ++s) {
        write_exact(o, h_cnt + s * W, sizeof(int32_t) * W);
        write_exact(o, h_slot + (size_t)s * T * W, sizeof(int32_t) * T * W);
        write_exact(o, h_out + (size_t)s * T * H, (size_t)row * T);
    }
    write_exact(o, h_ent, sizeof(int32_t) * e_local * W);
    write_exact(o, &h_err, sizeof h_err);
    fclose(o);

    hipFree(ids); hipFree(wts); hipFree(hidden); hipFree(send); hipFree(send_cnt);
    hipFree(send_eloc); hipFree(send_w); hipFree(token_slot); hipFree(batch);
    hipFree(expert_num_tokens); hipFree(recv_row); hipFree(ret); hipFree(out); hipFree(err);
    hipFree(ws);
    free(h_ids); free(h_wts); free(h_hid); free(h_cnt); free(h_slot); free(h_out); free(h_ent);
    printf("moe_ep_path: T=%lld H=%lld E=%d K=%d W=%d ok\n", (long long)T, (long long)H, E, K, W);
    return 0;
}
