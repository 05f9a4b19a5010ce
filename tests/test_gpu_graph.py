"""A whole step (every call of the path for all logical ranks) captured in a
HIP graph and replayed gives, on every replay, the same bytes as the eager
step. The library makes no allocation, memset or host synchronisation, so it
is capturable; the test replays several times with eager work and
synchronisations in between."""
import numpy as np
import pytest
import torch

import workloads as wl
from combine_topk_ids_dest_amd.emulate import LogicalEP
from parity import say

pytestmark = pytest.mark.gpu


def _setup(w, seed, **mode):
    srcs = [wl.routing(w, s, seed) for s in range(w.W)]
    pls = [wl.payloads(w, s, seed, ids=srcs[s][0], wts=srcs[s][1]) for s in range(w.W)]
    ep = LogicalEP(w.T, w.H, w.E, w.K, w.W, w.cap, [p.shape[1] for p in pls[0]],
                   torch.bfloat16, "cuda", fill=0xFF, **mode)
    for s in range(w.W):
        ep.set_source(s, srcs[s][0], srcs[s][1], pls[s])
    wl.expert_outputs_device(ep.Y, seed=3000 + seed)
    return ep


def _outputs(ep):
    ranks = [ep.send_rank, ep.send_ecnt] if ep.ranked else []
    return [x.clone() for x in [ep.send_cnt, ep.token_slot, ep.send_eloc,
                                ep.expert_num_tokens, ep.recv_row, ep.out] + ranks] + \
           [x.clone() for x in ep.send]


SMALL_DSV3 = dict(T=600, cap=640, H=1024)
CASES = [
    (4, None, {}, False),
    (1, None, {}, False),
    (2, SMALL_DSV3, {}, False),
    # the other forms of the path: quantised packs and the fused local combine
    (2, SMALL_DSV3, dict(quant_group=128), False),
    (4, None, dict(quant_fp4=True), False),
    (2, SMALL_DSV3, {}, True),
    # the senders' per-expert ranks and the ranked receive side, counted by
    # the pack itself (one tile) and by the routing kernel (three tiles)
    (4, None, dict(ranked=True), False),
    (2, SMALL_DSV3, dict(ranked=True), False),
]


@pytest.mark.parametrize("wid,scale,mode,fused", CASES)
def test_graph_replay_matches_eager(wid, scale, mode, fused):
    w = wl.WORKLOADS[wid] if scale is None else wl.WORKLOADS[wid].scaled(**scale)
    say(f"[graph] {w.name} T={w.T} W={w.W} {mode} fused={fused}")
    ep = _setup(w, 1, **mode)
    ep.step(fused_local=fused)
    torch.cuda.synchronize()
    eager = _outputs(ep)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ep.step(fused_local=fused)    # warm the prepared calls on this stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        ep.step(fused_local=fused)
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work between replays: scribble over the outputs that the
        # path writes in full (tails of the others are never written)
        ep.out.view(torch.uint8).fill_(0xAB)
        ep.token_slot.fill_(-9)
        ep.send_cnt.fill_(-9)
        ep.expert_num_tokens.fill_(-9)
        if ep.ranked:
            ep.send_ecnt.fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(ep)
        for a, b in zip(eager, got):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}"
    assert int(ep.err.item()) == 0
