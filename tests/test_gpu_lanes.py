"""The emulated step with the logical ranks spread over several HIP streams
(lanes, each with its own workspace and expert-batch buffer) writes the same
bytes as the one-stream step, eagerly and from one HIP graph per phase and
lane (each captured on a single stream) replayed on the lanes' streams.
Capturing a whole step over several streams in one graph crashed the
process when the capture ended; that case is switched off (the step raises
under capture) and its test is skipped."""
import pytest
import torch

import workloads as wl
from combine_topk_ids_dest_amd.emulate import LogicalEP
from parity import say

pytestmark = pytest.mark.gpu


def _setup(w, seed, lanes, **mode):
    srcs = [wl.routing(w, s, seed) for s in range(w.W)]
    pls = [wl.payloads(w, s, seed, ids=srcs[s][0], wts=srcs[s][1]) for s in range(w.W)]
    ep = LogicalEP(w.T, w.H, w.E, w.K, w.W, w.cap, [p.shape[1] for p in pls[0]],
                   torch.bfloat16, "cuda", fill=0xFF, lanes=lanes, **mode)
    for s in range(w.W):
        ep.set_source(s, srcs[s][0], srcs[s][1], pls[s])
    wl.expert_outputs_device(ep.Y, seed=3000 + seed)
    ep.share_expert_outputs()
    return ep


def _outputs(ep):
    """Every output of the step except the expert-batch buffers."""
    return [x.clone() for x in (ep.send_cnt, ep.token_slot, ep.send_eloc, ep.send_w,
                                ep.expert_num_tokens, ep.recv_row, ep.ret, ep.out)] + \
           [x.clone() for x in ep.send]


def _last_batch(ep):
    """Valid rows of the last destination's expert batch (in the buffer of
    its lane)."""
    r = ep.W - 1
    ent = ep.expert_num_tokens[r].tolist()
    return [torch.cat([b[e, :ent[e]] for e in range(ep.e_local)]).clone()
            for b in ep.b_lanes[r % ep.lanes]]


def _same(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"{what}: output {i}"


SMALL_DSV3 = dict(T=600, cap=640, H=1024)
CASES = [
    (1, None, 4, {}, False),
    (2, SMALL_DSV3, 4, {}, False),
    (2, SMALL_DSV3, 3, {}, True),                      # W = 8 not a multiple of 3
    (2, SMALL_DSV3, 2, dict(quant_group=128), False),
    (4, None, 4, dict(quant_fp4=True), False),         # W = 32 ranks over 4 lanes
    (3, dict(T=1000, cap=1000, H=512), 8, {}, False),  # one lane per rank
]


@pytest.mark.parametrize("wid,scale,lanes,mode,fused", CASES)
def test_lanes_match_one_stream(wid, scale, lanes, mode, fused):
    w = wl.WORKLOADS[wid] if scale is None else wl.WORKLOADS[wid].scaled(**scale)
    say(f"[lanes] {w.name} T={w.T} W={w.W} lanes={lanes} {mode} fused={fused}")
    one = _setup(w, 2, 1, **mode)
    one.step(fused_local=fused)
    torch.cuda.synchronize()
    ref, ref_b = _outputs(one), _last_batch(one)
    assert int(one.err.item()) == 0
    del one

    ep = _setup(w, 2, lanes, **mode)
    streams = [torch.cuda.Stream() for _ in range(lanes)]
    ep.step(fused_local=fused, streams=streams)
    torch.cuda.synchronize()
    _same(ref, _outputs(ep), "eager")
    _same(ref_b, _last_batch(ep), "eager batch")
    assert int(ep.err.item()) == 0


@pytest.mark.parametrize("wid,scale,lanes,mode,fused", CASES)
def test_lane_graphs_match_one_stream(wid, scale, lanes, mode, fused):
    w = wl.WORKLOADS[wid] if scale is None else wl.WORKLOADS[wid].scaled(**scale)
    say(f"[lane graphs] {w.name} T={w.T} W={w.W} lanes={lanes} {mode} fused={fused}")
    one = _setup(w, 3, 1, **mode)
    one.step(fused_local=fused)
    torch.cuda.synchronize()
    ref, ref_b = _outputs(one), _last_batch(one)
    del one

    ep = _setup(w, 3, lanes, **mode)
    streams = [torch.cuda.Stream() for _ in range(lanes)]
    ep.capture_lane_graphs(fused_local=fused)
    for rep in range(3):
        # eager work between replays: scribble over what the step writes
        ep.out.view(torch.uint8).fill_(0xAB)
        ep.ret.view(torch.uint8).fill_(0xCD)
        ep.token_slot.fill_(-9)
        ep.send_cnt.fill_(-9)
        ep.expert_num_tokens.fill_(-9)
        torch.cuda.synchronize()
        ep.step_graphs(streams)
        torch.cuda.synchronize()
        got = _outputs(ep)
        _same([x for i, x in enumerate(ref) if i != 6],
              [x for i, x in enumerate(got) if i != 6], f"replay {rep}")
        valid = _valid_ret_rows(ep, fused)
        assert torch.equal(ref[6].view(torch.uint8)[valid], got[6].view(torch.uint8)[valid])
        _same(ref_b, _last_batch(ep), f"replay {rep} batch")
    assert int(ep.err.item()) == 0


def _valid_ret_rows(ep, fused):
    """Boolean [W, W, cap] mask of the ret rows the reduce writes (the
    peers-only reduce of the fused combine leaves a rank's own block)."""
    cnt = ep.send_cnt.t()     # [dest, src]
    slot = torch.arange(ep.cap, device=cnt.device)
    valid = slot[None, None, :] < cnt[:, :, None]
    if fused:
        eye = torch.eye(ep.W, dtype=torch.bool, device=cnt.device)
        valid &= ~eye[:, :, None]
    return valid


def test_lanes_argument_checks():
    w = wl.WORKLOADS[1]
    with pytest.raises(ValueError):
        LogicalEP(w.T, w.H, w.E, w.K, w.W, w.cap, [2 * w.H], torch.bfloat16, "cuda",
                  lanes=w.W + 1)
    ep = LogicalEP(w.T, w.H, w.E, w.K, w.W, w.cap, [2 * w.H], torch.bfloat16, "cuda",
                   lanes=2)
    with pytest.raises(ValueError):
        ep.step(streams=[torch.cuda.Stream()])


@pytest.mark.skip(reason="capturing a step over several streams crashed the process at "
                         "the end of the capture (segmentation fault in capture_end); "
                         "the emulation refuses such a capture until the cause is known")
@pytest.mark.parametrize("wid,scale,lanes,mode,fused", CASES[:2])
def test_lanes_graph_replay(wid, scale, lanes, mode, fused):
    w = wl.WORKLOADS[wid] if scale is None else wl.WORKLOADS[wid].scaled(**scale)
    one = _setup(w, 2, 1, **mode)
    one.step(fused_local=fused)
    torch.cuda.synchronize()
    ref = _outputs(one)
    del one
    ep = _setup(w, 2, lanes, **mode)
    streams = [torch.cuda.Stream() for _ in range(lanes)]
    # the same step captured once and replayed, with eager work between
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ep.step(fused_local=fused, streams=streams)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        ep.step(fused_local=fused, streams=streams)
    torch.cuda.synchronize()
    for rep in range(3):
        ep.out.view(torch.uint8).fill_(0xAB)
        ep.ret.view(torch.uint8).fill_(0xCD)
        ep.token_slot.fill_(-9)
        ep.send_cnt.fill_(-9)
        ep.expert_num_tokens.fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(ep)
        # ret is written only at valid slots: compare those rows
        _same([x for i, x in enumerate(ref) if i != 6],
              [x for i, x in enumerate(got) if i != 6], f"replay {rep}")
        valid = _valid_ret_rows(ep, fused)
        assert torch.equal(ref[6].view(torch.uint8)[valid], got[6].view(torch.uint8)[valid])
    assert int(ep.err.item()) == 0
