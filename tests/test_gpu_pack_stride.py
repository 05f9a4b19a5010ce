"""GPU: the pack's metadata rank stride. send_eloc / send_w may have their
destination blocks further apart than cap * slots (so they can point at
per-destination receive blocks, as the payloads can); every valid entry
must equal the oracle's, and neither the slots past a destination's count
nor the elements between blocks may be written. Through the C ABI for the
plain, fp8 and 4-bit packs, with the pack's own routing (T <= 256) and with
the routing kernel (T > 256)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from combine_topk_ids_dest_amd import binding as B
from parity import say

pytestmark = pytest.mark.gpu

PAD = 37
ELOC_FILL = -12345
W_FILL = 0x7FBADBAD        # a NaN pattern no pack writes


@pytest.mark.parametrize("mode", ["plain", "fp8", "fp4"])
@pytest.mark.parametrize("T", [200, 600])
def test_pack_metadata_rank_stride_leaves_the_pad(mode, T):
    w = wl.WORKLOADS[1].scaled(W=4, E=16, K=4, T=T, cap=T + 40, H=128, pad_frac=0.05)
    say(f"[pack meta stride] {mode} T={T} pad={PAD}")
    ids, wts = wl.routing(w, 0, 51)
    hidden = wl.hidden_bf16(w, 0, 51)                         # uint16 [T, H]
    slots = min(w.K, w.e_local)
    block = w.cap * slots
    dev = torch.device("cuda")
    eloc_base = torch.full((w.W, block + PAD), ELOC_FILL, dtype=torch.int32, device=dev)
    w_base = torch.full((w.W, block + PAD), W_FILL, dtype=torch.int32, device=dev)
    send_eloc = eloc_base[:, :block].view(w.W, w.cap, slots)
    send_w = w_base.view(torch.float32)[:, :block].view(w.W, w.cap, slots)
    assert send_eloc.stride(0) == block + PAD
    d_ids = torch.from_numpy(ids).to(dev)
    d_wts = torch.from_numpy(wts).to(dev)
    d_hidden = torch.from_numpy(hidden.view(np.int16)).to(dev).view(torch.bfloat16)
    send_cnt = torch.full((w.W,), -1, dtype=torch.int32, device=dev)
    token_slot = torch.empty((w.T, w.W), dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.empty(max(B.moe_ep_workspace_bytes(w.T, w.K, w.E, w.W, w.cap), 16),
                     dtype=torch.uint8, device=dev)
    if mode == "plain":
        dst = torch.full((w.W, w.cap, 2 * w.H), 0xFF, dtype=torch.uint8, device=dev)
        B.moe_ep_dispatch_pack(d_ids, d_wts, w.E, w.W, w.cap,
                               [(d_hidden.view(torch.uint8), dst)], send_cnt, send_eloc,
                               send_w, token_slot, err, ws)
        exp = oracle.dispatch_pack(ids, wts, w.E, w.W, w.cap,
                                   [hidden.view(np.uint8).reshape(w.T, 2 * w.H)])
        got_rows = [dst]
    elif mode == "fp8":
        G = B.scale_pitch(w.H, 32)
        q = torch.full((w.W, w.cap, w.H), 0xFF, dtype=torch.uint8, device=dev)
        sc = torch.full((w.W, w.cap, G), float("nan"), dtype=torch.float32, device=dev)
        B.moe_ep_dispatch_pack_fp8(d_ids, d_wts, w.E, w.W, w.cap, d_hidden, 32, q, sc, [],
                                   send_cnt, send_eloc, send_w, token_slot, err, ws)
        exp = oracle.dispatch_pack_fp8(ids, wts, w.E, w.W, w.cap, hidden, 32)
        got_rows = [q, sc.view(torch.uint8).view(w.W, w.cap, 4 * G)]
    else:
        q = torch.full((w.W, w.cap, w.H // 2), 0xFF, dtype=torch.uint8, device=dev)
        sc = torch.full((w.W, w.cap, B.fp4_scale_pitch(w.H)), 0xFF, dtype=torch.uint8,
                        device=dev)
        B.moe_ep_dispatch_pack_fp4(d_ids, d_wts, w.E, w.W, w.cap, d_hidden, q, sc, [],
                                   send_cnt, send_eloc, send_w, token_slot, err, ws)
        exp = oracle.dispatch_pack_fp4(ids, wts, w.E, w.W, w.cap, hidden)
        got_rows = [q, sc]
    torch.cuda.synchronize()
    assert np.array_equal(send_cnt.cpu().numpy(), exp["send_cnt"])
    assert np.array_equal(token_slot.cpu().numpy(), exp["token_slot"])
    ge = eloc_base.cpu().numpy()
    gw = w_base.cpu().numpy()
    for d in range(w.W):
        c = int(exp["send_cnt"][d])
        assert np.array_equal(ge[d, :c * slots].reshape(c, slots), exp["send_eloc"][d, :c])
        assert np.array_equal(gw[d, :c * slots].reshape(c, slots).view(np.uint32),
                              exp["send_w"][d, :c].view(np.uint32))
        assert (ge[d, c * slots:] == ELOC_FILL).all(), f"eloc tail or pad of {d} written"
        assert (gw[d, c * slots:] == W_FILL).all(), f"weight tail or pad of {d} written"
        for p, g in enumerate(got_rows):
            assert np.array_equal(g[d, :c].cpu().numpy(), exp["send"][p][d, :c]), \
                f"payload {p} of destination {d}"
    assert int(err.item()) == exp["err"]
