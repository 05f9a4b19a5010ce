"""GPU parity of moe_ep_sanitize_expert_ids (through the C ABI) with the
oracle: bit-exact on every entry of the [W, cap, slots] layout, out of place
and in place, on seeded garbage (ids and counts out of range) and on the
receive buffers of the whole path."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from combine_topk_ids_dest_amd import binding as B
from combine_topk_ids_dest_amd.emulate import LogicalEP
from parity import say

pytestmark = pytest.mark.gpu

W1, W2, W4 = wl.WORKLOADS[1], wl.WORKLOADS[2], wl.WORKLOADS[4]

SHAPES = {
    # (W, e_local, K, cap)
    "tiny": (4, 2, 2, 16),
    "dsv3_full": (8, 32, 8, 4096),
    "decode_full": (32, 8, 8, 128),
    "w64_ragged": (64, 2, 4, 97),
    "k1": (3, 5, 1, 1000),
    "e_local_1": (8, 1, 2, 300),
}


def _garbage(W, e_local, K, cap, seed):
    rng = np.random.default_rng(seed)
    slots = min(K, e_local)
    cnt = rng.integers(0, cap + 1, W).astype(np.int32)
    cnt[0] = cap
    if W > 2:
        cnt[1] = cap + 5            # clamped
        cnt[2] = -2                 # clamped to 0
    eloc = rng.integers(-2, e_local + 2, (W, cap, slots)).astype(np.int32)
    return cnt, eloc


@pytest.mark.parametrize("name", sorted(SHAPES))
@pytest.mark.parametrize("in_place", [False, True])
def test_sanitize_garbage(name, in_place):
    W, e_local, K, cap = SHAPES[name]
    say(f"[sanitize] {name} in_place={in_place}")
    cnt, eloc = _garbage(W, e_local, K, cap, seed=sorted(SHAPES).index(name))
    exp = oracle.sanitize_expert_ids(cnt, eloc, W, e_local, K, cap, -77)
    slots = min(K, e_local)
    # rank stride padded past cap * slots to check the stride is honoured
    pad = 5
    d_cnt = torch.from_numpy(np.repeat(cnt[:, None], 3, 1)).cuda()[:, 0]
    d_eloc = torch.full((W, cap * slots + pad), 12345, dtype=torch.int32, device="cuda")
    d_eloc[:, :cap * slots] = torch.from_numpy(eloc.reshape(W, -1)).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    if in_place:
        out = d_eloc
    else:
        out = torch.full((W, cap * slots + 3), 54321, dtype=torch.int32, device="cuda")
    B.moe_ep_sanitize_expert_ids(d_cnt, d_eloc[:, :cap * slots], W, e_local, K, cap,
                                 -77, out[:, :cap * slots], err)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got[:, :cap * slots].reshape(W, cap, slots), exp["ids"])
    tail = 12345 if in_place else 54321
    assert (got[:, cap * slots:] == tail).all(), "wrote past the rank block"
    assert int(err.item()) == exp["err"]


@pytest.mark.parametrize("w", [W1, W4, W2.scaled(T=300, cap=320, H=256)],
                         ids=["tiny", "decode", "dsv3_small"])
def test_sanitize_received_ids_of_the_path(w):
    """In place on the receive buffers the pack wrote: equal to the oracle
    run on the oracle's own pack outputs, for every destination."""
    say(f"[sanitize path] {w.name} W={w.W}")
    srcs = [wl.routing(w, s, 31) for s in range(w.W)]
    packs = [oracle.dispatch_pack(ids, wts, w.E, w.W, w.cap) for ids, wts in srcs]
    ep = LogicalEP(w.T, w.H, w.E, w.K, w.W, w.cap, [2 * w.H], torch.bfloat16, "cuda")
    for s, (ids, wts) in enumerate(srcs):
        ep.set_source(s, ids, wts, [wl.hidden_bf16(w, s, 31).view(np.uint8)
                                    .reshape(w.T, 2 * w.H)])
        ep.pack(s)
    for r in range(w.W):
        cnt = np.stack([p["send_cnt"][r] for p in packs]).astype(np.int32)
        eloc = np.stack([p["send_eloc"][r] for p in packs])
        exp = oracle.sanitize_expert_ids(cnt, eloc, w.W, w.e_local, w.K, w.cap, -1)
        view = ep.send_eloc[:, r]
        B.moe_ep_sanitize_expert_ids(ep.send_cnt[:, r], view, w.W, w.e_local, w.K,
                                     w.cap, -1, view, ep.err)
        torch.cuda.synchronize()
        assert np.array_equal(view.cpu().numpy(), exp["ids"]), f"dst {r}"
    assert int(ep.err.item()) == 0
