"""GPU: moe_ep_dispatch_pack_noalloc (the pack for callers that cannot
allocate; its workspace is the library's own device scratch) writes exactly
what moe_ep_dispatch_pack writes with a caller workspace. Two calls in a row
on the one scratch array, the second with fewer tokens, each compared byte
for byte with the pack on the same inputs; the outputs also agree with the
oracle. A third call with more than 64 routing tiles uses the scratch's tile
offset region as well, and a fourth (one tile of tokens) needs none."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from combine_topk_ids_dest_amd import binding as B
from parity import say

pytestmark = pytest.mark.gpu

FILL = 0xFF


def _buffers(w, slots, dev):
    return dict(
        send=torch.full((w.W, w.cap, 2 * w.H), FILL, dtype=torch.uint8, device=dev),
        send_cnt=torch.full((w.W,), -1, dtype=torch.int32, device=dev),
        send_eloc=torch.full((w.W, w.cap, slots), -3, dtype=torch.int32, device=dev),
        send_w=torch.full((w.W, w.cap, slots), float("nan"), device=dev),
        token_slot=torch.full((w.T, w.W), -5, dtype=torch.int32, device=dev),
        err=torch.zeros(1, dtype=torch.int32, device=dev))


def _one(w, salt, ranked=False):
    dev = torch.device("cuda")
    slots = min(w.K, w.e_local)
    ids, wts = wl.routing(w, 0, salt)
    hidden = wl.hidden_bf16(w, 0, salt)
    d_ids = torch.from_numpy(ids).to(dev)
    d_wts = torch.from_numpy(wts).to(dev)
    src = torch.from_numpy(hidden.view(np.uint8).reshape(w.T, 2 * w.H)).to(dev)
    a = _buffers(w, slots, dev)
    b = _buffers(w, slots, dev)
    for x in (a, b):
        x["send_rank"] = torch.full((w.W, w.cap, slots), -7, dtype=torch.int32, device=dev)
        x["send_ecnt"] = torch.full((w.W, w.e_local), -7, dtype=torch.int32, device=dev)
    rk = lambda x: dict(send_rank=x["send_rank"], send_ecnt=x["send_ecnt"]) if ranked else {}
    ws = torch.empty(max(B.moe_ep_workspace_bytes(w.T, w.K, w.E, w.W, w.cap), 16),
                     dtype=torch.uint8, device=dev)
    B.moe_ep_dispatch_pack(d_ids, d_wts, w.E, w.W, w.cap, [(src, a["send"])], a["send_cnt"],
                           a["send_eloc"], a["send_w"], a["token_slot"], a["err"], ws, **rk(a))
    B.moe_ep_dispatch_pack_noalloc(d_ids, d_wts, w.E, w.W, w.cap, [(src, b["send"])],
                                   b["send_cnt"], b["send_eloc"], b["send_w"],
                                   b["token_slot"], b["err"], **rk(b))
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), k
    exp = oracle.dispatch_pack(ids, wts, w.E, w.W, w.cap,
                               [hidden.view(np.uint8).reshape(w.T, 2 * w.H)])
    assert np.array_equal(b["send_cnt"].cpu().numpy(), exp["send_cnt"])
    assert np.array_equal(b["token_slot"].cpu().numpy(), exp["token_slot"])
    ge = b["send_eloc"].cpu().numpy()
    gs = b["send"].cpu().numpy()
    for d in range(w.W):
        c = int(exp["send_cnt"][d])
        assert np.array_equal(ge[d, :c], exp["send_eloc"][d, :c])
        assert np.array_equal(gs[d, :c], exp["send"][0][d, :c])
    assert int(b["err"].item()) == exp["err"]
    if ranked:
        er = oracle.pick_ranks(exp["send_cnt"], exp["send_eloc"], w.e_local)
        assert np.array_equal(b["send_ecnt"].cpu().numpy(), er["send_ecnt"])
        gr = b["send_rank"].cpu().numpy()
        for d in range(w.W):
            c = int(exp["send_cnt"][d])
            assert np.array_equal(gr[d, :c], er["send_rank"][d, :c])


def test_noalloc_pack_matches_the_pack_on_successive_calls():
    base = wl.WORKLOADS[2]
    first = base.scaled(W=8, E=64, K=6, T=3000, cap=3000, H=256)
    second = base.scaled(W=8, E=64, K=6, T=700, cap=800, H=256)
    third = base.scaled(W=4, E=16, K=4, T=17000, cap=17000, H=64)
    decode = base.scaled(W=8, E=64, K=6, T=100, cap=128, H=256)   # no scratch needed
    for i, w in enumerate((first, second, third, decode)):
        say(f"[noalloc] call {i}: T={w.T} W={w.W} E={w.E} K={w.K} H={w.H}")
        _one(w, 60 + i)
    # with the per-expert ranks (their tables in the scratch as well)
    for i, w in enumerate((second, first, third, decode)):
        say(f"[noalloc ranked] call {i}: T={w.T} W={w.W} E={w.E} K={w.K} H={w.H}")
        _one(w, 70 + i, ranked=True)
