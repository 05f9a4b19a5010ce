"""GPU parity at the full sizes of the five workloads, in the launch
configuration that bench.py times (LogicalEP calls on W logical ranks, and
the whole step over the HIP streams bench.py spreads the ranks over).
Integer outputs are compared whole; every valid payload byte is compared on
the device with the source row the oracle's slot and row maps name; the
combine is compared element by element on column windows the oracle
computes exactly."""
import gc

import pytest
import torch

import bench
import workloads as wl
from parity import SENTINEL, check_lanes_step, run_fullsize, say, snapshot_step

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_fullsize(wid):
    w = wl.WORKLOADS[wid]
    say(f"[fullsize] start {w.name}")
    ep = run_fullsize(w)
    lanes = bench.auto_lanes(w, ep.row_bytes)
    if lanes > 1:
        ref = snapshot_step(ep)
        del ep
        gc.collect()                 # contiguous blocks go with their last reference
        torch.cuda.empty_cache()
        check_lanes_step(w, ref, lanes)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_fullsize_ranked(wid):
    """The packs with per-expert ranks and the ranked receive side at full
    size (ranks and counts against the oracle's, rows and every batched byte
    as in test_fullsize), and the whole step over the lanes bench.py uses."""
    w = wl.WORKLOADS[wid]
    say(f"[fullsize ranked] start {w.name}")
    ep = run_fullsize(w, ranked=True)
    lanes = bench.auto_lanes(w, ep.row_bytes)
    if lanes > 1:
        ref = snapshot_step(ep)
        del ep
        gc.collect()
        torch.cuda.empty_cache()
        check_lanes_step(w, ref, lanes, ranked=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wid", [2, 5])
def test_fullsize_fp8_pack(wid):
    """Quantize-on-pack at the DeepSeek-V3 and multi-payload shapes."""
    w = wl.WORKLOADS[wid]
    say(f"[fullsize fp8] start {w.name}")
    run_fullsize(w, fp8_group=128)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wid", [2, 5])
def test_fullsize_fp4_pack(wid):
    """4-bit quantize-on-pack at the DeepSeek-V3 and multi-payload shapes."""
    w = wl.WORKLOADS[wid]
    say(f"[fullsize fp4] start {w.name}")
    run_fullsize(w, fp4=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wid,mode", [(2, "fp8"), (4, "fp4")])
def test_fullsize_ranked_quantised(wid, mode):
    """The quantising packs with the per-expert ranks and the ranked receive
    side at full size: DS-V3 with fp8 (the routing kernel's ranks) and
    decode with 4-bit codes (the pack counts the ranks itself)."""
    w = wl.WORKLOADS[wid]
    say(f"[fullsize ranked {mode}] start {w.name}")
    if mode == "fp8":
        run_fullsize(w, fp8_group=128, ranked=True)
    else:
        run_fullsize(w, fp4=True, ranked=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wid", [2, 3, 4])
def test_fullsize_fused_local_combine(wid):
    """The fused combine of each rank's local slice at full size (the shared
    expert output stands in for every rank's own, as in bench.py): out
    bit-identical to the unfused path checked above, and the own block of
    ret neither read (it is overwritten with NaN bytes first) nor written."""
    w = wl.WORKLOADS[wid]
    say(f"[fullsize fused] start {w.name}")
    ep = run_fullsize(w)
    out_ref = ep.out.clone()
    ep.out.view(torch.uint8).fill_(SENTINEL)
    for r in range(w.W):
        ep.ret[r, r].view(torch.uint8).fill_(SENTINEL)
    for r in range(w.W):
        ep.reduce_peers(r)
    for s in range(w.W):
        ep.unpack_fused(s)
    torch.cuda.synchronize()
    assert torch.equal(ep.out.view(torch.uint8), out_ref.view(torch.uint8))
    for r in range(w.W):
        assert bool((ep.ret[r, r].view(torch.uint8) == SENTINEL).all())
    say(f"[fullsize fused] {w.name}: ok")
