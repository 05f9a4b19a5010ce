"""The path inside a small MoE layer: dispatch, a real expert (one bf16
linear map per expert, torch matmul on the batched rows), combine; the
output compared with a plain fp32 evaluation of sum_k w_k * expert_k(x) for
every token. The tolerance is that of bf16 inputs and bf16 expert outputs
(the layout transform itself is checked bit for bit elsewhere)."""
import numpy as np
import pytest
import torch

import workloads as wl
from combine_topk_ids_dest_amd.emulate import LogicalEP
from parity import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("W,E,K,T,H", [(4, 16, 2, 64, 128), (8, 64, 6, 100, 256)])
def test_moe_layer_matches_dense_evaluation(W, E, K, T, H):
    w = wl.WORKLOADS[1].scaled(W=W, E=E, K=K, T=T, cap=T, H=H, pad_frac=0.05)
    say(f"[moe layer] W={W} E={E} K={K} T={T} H={H}")
    g = torch.Generator().manual_seed(5)
    experts = (torch.randn(E, H, H, generator=g) / H ** 0.5).to(torch.bfloat16)
    srcs = [wl.routing(w, s, 1) for s in range(W)]
    xs = [wl.hidden_bf16(w, s, 1) for s in range(W)]
    ep = LogicalEP(T, H, E, K, W, T, [2 * H], torch.bfloat16, "cuda")
    for s in range(W):
        ep.set_source(s, srcs[s][0], srcs[s][1], [xs[s].view(np.uint8).reshape(T, 2 * H)])
        ep.pack(s)
    dev_experts = experts.cuda()
    el = ep.e_local
    for r in range(W):
        ep.batch(r)
        counts = ep.expert_num_tokens[r].cpu().tolist()
        for e in range(el):
            n = counts[e]
            if n:
                rows = ep.b[0][e, :n].view(torch.bfloat16).reshape(n, H).contiguous()
                ep.Y[e, :n] = rows @ dev_experts[r * el + e].contiguous()
        ep.reduce(r)
    for s in range(W):
        ep.unpack(s)
    torch.cuda.synchronize()
    assert int(ep.err.item()) == 0

    ef = experts.float()
    for s in range(W):
        ids, wts = srcs[s]
        x = torch.from_numpy(wl.bf16_bits_to_f32(xs[s]))
        ref = torch.zeros(T, H)
        for t in range(T):
            for k in range(K):
                if ids[t, k] >= 0:
                    ref[t] += float(wts[t, k]) * (x[t] @ ef[ids[t, k]])
        got = ep.out[s].float().cpu()
        pad = (ids < 0).all(axis=1)
        assert torch.equal(got[torch.from_numpy(pad)], torch.zeros(int(pad.sum()), H))
        scale = ref.abs().max().item()
        err = (got - ref).abs().max().item()
        assert err <= 2e-2 * scale, (s, err, scale)


def test_moe_layer_on_the_non_batched_receive_buffers():
    """The same layer without the expert batching: a consumer reads the
    received [W, cap, H] rows in place, takes the expert ids that
    moe_ep_sanitize_expert_ids leaves (-1 for every entry that is not a
    valid pick), weights and sums its experts per received slot into the
    return buffer, and moe_ep_combine_unpack finishes the combine."""
    from combine_topk_ids_dest_amd import binding as B

    W, E, K, T, H = 4, 16, 3, 80, 128
    w = wl.WORKLOADS[1].scaled(W=W, E=E, K=K, T=T, cap=T, H=H, pad_frac=0.05)
    say(f"[moe layer, non-batched] W={W} E={E} K={K} T={T} H={H}")
    g = torch.Generator().manual_seed(6)
    experts = (torch.randn(E, H, H, generator=g) / H ** 0.5).to(torch.bfloat16)
    srcs = [wl.routing(w, s, 2) for s in range(W)]
    xs = [wl.hidden_bf16(w, s, 2) for s in range(W)]
    ep = LogicalEP(T, H, E, K, W, T, [2 * H], torch.bfloat16, "cuda", fill=0xFF)
    for s in range(W):
        ep.set_source(s, srcs[s][0], srcs[s][1], [xs[s].view(np.uint8).reshape(T, 2 * H)])
        ep.pack(s)
    el, sl = ep.e_local, ep.slots
    dev_experts = experts.cuda().float()
    ids = torch.empty(W, T, sl, dtype=torch.int32, device="cuda")
    for r in range(W):
        B.moe_ep_sanitize_expert_ids(ep.send_cnt[:, r], ep.send_eloc[:, r], W, el, K, T,
                                     -1, ids, ep.err)
        rows = ep.send[0][:, r].view(torch.bfloat16).float()          # [W, cap, H]
        wts = ep.send_w[:, r]                                          # [W, cap, slots]
        acc = torch.zeros(W, T, H, device="cuda")
        for j in range(sl):
            for e in range(el):
                m = ids[:, :, j] == e
                if bool(m.any()):
                    y = (rows[m].to(torch.bfloat16).float() @ dev_experts[r * el + e])
                    y = y.to(torch.bfloat16).float()
                    acc[m] += wts[:, :, j][m][:, None] * y
        cnt = ep.send_cnt[:, r].cpu().tolist()
        for s in range(W):
            ep.ret[r, s, :cnt[s]] = acc[s, :cnt[s]].to(torch.bfloat16)
    for s in range(W):
        ep.unpack(s)
    torch.cuda.synchronize()
    assert int(ep.err.item()) == 0

    ef = experts.float()
    for s in range(W):
        sid, swt = srcs[s]
        x = torch.from_numpy(wl.bf16_bits_to_f32(xs[s]))
        ref = torch.zeros(T, H)
        for t in range(T):
            for k in range(K):
                if sid[t, k] >= 0:
                    ref[t] += float(swt[t, k]) * (x[t] @ ef[sid[t, k]])
        got = ep.out[s].float().cpu()
        assert (got - ref).abs().max().item() <= 2e-2 * ref.abs().max().item()
