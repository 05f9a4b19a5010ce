"""Physically contiguous device blocks (devmem.empty_contiguous) hold what
is written to them, work under the library's kernels, go back to the device
when their last tensor is gone, and are what the full-size emulation uses
for its large buffers."""
import gc

import pytest
import torch

import workloads as wl
from combine_topk_ids_dest_amd import devmem
from combine_topk_ids_dest_amd.emulate import CONTIGUOUS_MIN_BYTES, LogicalEP

pytestmark = pytest.mark.gpu


def test_contiguous_block_round_trip_and_release():
    n = 1 << 30
    ref = torch.randint(0, 256, (4, n // 4), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    t = devmem.empty_contiguous((4, n // 4), torch.uint8, "cuda")
    assert t is not None, "the device granted no contiguous block of 1 GiB"
    assert t.shape == (4, n // 4) and t.dtype == torch.uint8 and t.is_cuda
    assert t.data_ptr() % 256 == 0
    slack = 16 << 20                   # the free-memory figure is not byte-exact
    assert free0 - torch.cuda.mem_get_info()[0] >= n - slack
    t.copy_(ref)
    assert torch.equal(t, ref)
    f = t.view(torch.float32)          # other dtypes view the same bytes
    assert f.shape == (4, n // 16)
    assert torch.equal(f.view(torch.uint8), ref)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    del t, f
    gc.collect()
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] - free1 >= n - slack, "block not returned"


def test_fullsize_emulation_gets_contiguous_buffers():
    """At the DeepSeek-V3 shape the send, expert-batch, expert-output and
    return buffers are contiguous blocks; the smaller ones (sources,
    outputs, metadata) are not."""
    w = wl.WORKLOADS[2]
    ep = LogicalEP(w.T, w.H, w.E, w.K, w.W, w.cap, [2 * w.H], torch.bfloat16, "cuda")
    nbytes = lambda x: x.numel() * x.element_size()
    big = [ep.send[0], ep.b[0], ep.Y, ep.ret]
    assert all(nbytes(x) >= CONTIGUOUS_MIN_BYTES for x in big)
    assert nbytes(ep.src[0]) < CONTIGUOUS_MIN_BYTES and nbytes(ep.out) < CONTIGUOUS_MIN_BYTES
    assert ep.contiguous_bytes == sum(nbytes(x) for x in big)
    del ep
    gc.collect()
    torch.cuda.empty_cache()


def test_no_contiguous_when_switched_off():
    w = wl.WORKLOADS[2]
    ep = LogicalEP(w.T, w.H, w.E, w.K, w.W, w.cap, [2 * w.H], torch.bfloat16, "cuda",
                   contiguous=False)
    assert ep.contiguous_bytes == 0
    del ep
    gc.collect()
    torch.cuda.empty_cache()


def test_refused_block_falls_back_and_leaves_no_error():
    """A block the device cannot grant (1 PiB) gives None, and the runtime's
    last error is cleared, so the library's next launches do not report it;
    the emulation then takes its buffers from torch."""
    assert devmem.empty_contiguous((1 << 50,), torch.uint8, "cuda") is None
    w = wl.WORKLOADS[1]
    ep = LogicalEP(w.T, w.H, w.E, w.K, w.W, w.cap, [2 * w.H], torch.bfloat16, "cuda")
    for s in range(w.W):
        ids, wts = wl.routing(w, s)
        ep.set_source(s, ids, wts, wl.payloads(w, s, ids=ids, wts=wts))
    ep.step()                          # raises MoeEpError on a stale launch error
    torch.cuda.synchronize()
    assert int(ep.err.item()) == 0
    assert int(ep.send_cnt.sum().item()) > 0
