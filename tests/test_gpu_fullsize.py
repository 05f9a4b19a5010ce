"""GPU parity at the full sizes of the five workloads, in the launch
configuration that bench.py times (LogicalEP calls on W logical ranks).
Integer outputs are compared whole; every valid payload byte is compared on
the device with the source row the oracle's slot and row maps name; the
combine is compared element by element on column windows the oracle
computes exactly."""
import pytest

import workloads as wl
from parity import run_fullsize, say

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_fullsize(wid):
    w = wl.WORKLOADS[wid]
    say(f"[fullsize] start {w.name}")
    run_fullsize(w)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wid", [2, 5])
def test_fullsize_fp8_pack(wid):
    """Quantize-on-pack at the DeepSeek-V3 and multi-payload shapes."""
    w = wl.WORKLOADS[wid]
    say(f"[fullsize fp8] start {w.name}")
    run_fullsize(w, fp8_group=128)
