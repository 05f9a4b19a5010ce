"""Host-side logic without a GPU: the binding's layout checks (no library
call is made; CPU tensors only stand in for shapes and strides), the
benchmark's algorithmic byte model on a hand-counted case, the rule that a
counter summary taken on other kernel sources is not used, and the lanes
the benchmark picks per workload."""
import os
import shutil

import numpy as np
import pytest
import torch

import bench
import workloads as wl
from combine_topk_ids_dest_amd import binding as B


def test_scale_pitches():
    assert B.scale_pitch(7168, 128) == 56 and B.scale_pitch(7168, 32) == 224
    assert B.scale_pitch(1024 + 128, 128) == 12          # 9 scales -> 12 floats
    assert B.fp4_scale_pitch(7168) == 448 and B.fp4_scale_pitch(544) == 48


def test_payload_descriptors_and_layout_checks():
    src = torch.zeros(10, 64, dtype=torch.uint8)
    dst = torch.zeros(4, 16, 64, dtype=torch.uint8)
    arr = B._payload_array([(src, dst)], 1, 2)
    assert arr[0].row_bytes == 64 and arr[0].src_stride == 64 and arr[0].dst_stride == 16 * 64
    with pytest.raises(ValueError):                      # rows differ in size
        B._payload_array([(src, torch.zeros(4, 16, 32, dtype=torch.uint8))], 1, 2)
    with pytest.raises(ValueError):                      # a gap inside a row block
        B._payload_array([(src, torch.zeros(4, 16, 128, dtype=torch.uint8)[:, :, :64])], 1, 2)
    with pytest.raises(ValueError):
        B._payload_array([(src, dst)] * (B.MAX_PAYLOADS + 1), 1, 2)
    # a strided leading dim is allowed: a rank view of a [W_src, W_dst, ...] buffer
    big = torch.zeros(3, 4, 16, 64, dtype=torch.uint8)
    arr = B._payload_array([(src, big[:, 1])], 1, 2)
    assert arr[0].dst_stride == 4 * 16 * 64


def test_byte_model_hand_counted():
    """W = 2 ranks, E = 2 (e_local = 1), T = 3 tokens, K = 2, P = Hb = 32 B,
    slots = 1.
    Source 0 sends 2 slots to rank 0 and 1 to rank 1 (U = 3); source 1
    sends 1 and 2 (U = 3). Rank r receives S = 3 slots holding R = 4 and 2
    expert rows."""
    w = wl.WORKLOADS[1].scaled(T=3, H=16, E=2, K=2, W=2, cap=3)
    send_cnt = np.array([[2, 1], [1, 2]])
    ent = np.array([[3, 1], [1, 1]])                     # rows per local expert
    bm = bench.byte_model(w, [32], 1, send_cnt, ent, routed=[3, 2])
    assert bm["pack"] == [8 * 3 * 2 + 3 * 32 + 3 * 32 + 3 * 1 * 8 + 4 * 2,
                          8 * 3 * 2 + 2 * 32 + 3 * 32 + 3 * 1 * 8 + 4 * 2]
    assert bm["batch_plan"] == [4 * 2 + 3 * 1 * 4 + 4 * 1] * 2     # e_local = 1
    assert bm["batch_copy"] == [3 * 32 + 4 * 32, 3 * 32 + 2 * 32]
    assert bm["reduce"] == [4 * 32 + 3 * 1 * 8 + 3 * 32, 2 * 32 + 3 * 8 + 3 * 32]
    assert bm["unpack"] == [3 * 32 + 3 * 32] * 2
    # fused local slice: rank r's own slots (send_cnt[r, r]) and rows
    bmf = bench.byte_model(w, [32], 1, send_cnt, ent, routed=[3, 2], r_own=[2, 2])
    assert bmf["reduce_peers"] == [(4 - 2) * 32 + (3 - 2) * (8 + 32),
                                   (2 - 2) * 32 + (3 - 2) * (8 + 32)]
    assert bmf["unpack_fused"] == [(3 - 2) * 32 + 2 * 32 + 2 * 8 + 3 * 32,
                                   (3 - 2) * 32 + 2 * 32 + 2 * 8 + 3 * 32]


def test_counter_summary_of_other_sources_is_ignored(tmp_path, monkeypatch):
    kern = "batch_copy_kernel"
    prof = tmp_path / "profiles"
    prof.mkdir()
    pkg = tmp_path / "combine_topk_ids_dest_amd"
    shutil.copytree(os.path.join(bench.ROOT, "combine_topk_ids_dest_amd", "csrc"), pkg / "csrc")
    shutil.copy(os.path.join(bench.ROOT, "combine_topk_ids_dest_amd", "build.py"), pkg)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.source_digest(kern)
    (prof / f"{kern}.w.pmc.txt").write_text(
        f"traffic_bytes_per_launch: 123\nsource_sha256: {digest}\n")
    assert bench.read_traffic(kern, "w") == 123.0
    with open(pkg / "csrc" / "batch.hip", "a") as f:
        f.write("\n// changed\n")
    assert bench.read_traffic(kern, "w") is None         # the kernel changed since
    assert bench.read_traffic(kern, "other") is None     # no summary at all


def test_auto_lanes_per_workload():
    """--lanes auto: 2 lanes, 1 for a tiny step, and no more lanes than
    there are ranks or than fit the lanes' expert-batch and bf16
    expert-output buffers in LANE_MEMORY_BYTES (the multi-payload rows are
    21,792 B)."""
    W = wl.WORKLOADS
    assert bench.auto_lanes(W[1], [2 * W[1].H]) == 1
    assert bench.auto_lanes(W[2], [2 * W[2].H]) == 2
    assert bench.auto_lanes(W[3], [2 * W[3].H]) == 2
    assert bench.auto_lanes(W[4], [2 * W[4].H]) == 2
    rows5 = [2 * W[5].H, W[5].H, 4 * 56, 32, 32]
    per_lane = W[5].e_local * W[5].W * W[5].cap * (sum(rows5) + 2 * W[5].H)
    assert bench.auto_lanes(W[5], rows5) == bench.LANE_MEMORY_BYTES // per_lane == 2
    # quantised rows are smaller, so more lanes would fit
    assert bench.auto_lanes(W[5], rows5, fp8_group=128) == 2
    assert bench.auto_lanes(W[5], rows5, fp4=True) == 2
    assert bench.lanes_that_fit(W[5], rows5, None, True, 4) == 3
    # never more lanes than ranks
    assert bench.lanes_that_fit(W[1], [2 * W[1].H], None, False, 16) == W[1].W


def test_emulation_is_freed_by_reference_count():
    """Contiguous device blocks are returned when their last tensor goes, so
    the emulation object must hold no reference cycle that would keep its
    buffers until a garbage collection; the block allocator declines
    non-GPU devices (the caller then allocates from torch)."""
    import weakref

    import torch

    from combine_topk_ids_dest_amd import devmem
    from combine_topk_ids_dest_amd.emulate import LogicalEP
    w = wl.WORKLOADS[1]
    ep = LogicalEP(w.T, w.H, w.E, w.K, w.W, w.cap, [2 * w.H], torch.bfloat16, "cpu")
    assert ep.contiguous_bytes == 0
    ref = weakref.ref(ep)
    del ep
    assert ref() is None
    assert devmem.empty_contiguous((4, 4), torch.uint8, "cpu") is None


def test_prepared_calls_take_gpu_tensors_only():
    """The library takes device pointers only: a call prepared on host
    tensors is refused before any pointer reaches it."""
    import torch
    back = torch.zeros(4, 16, 256, dtype=torch.bfloat16)
    token_slot = torch.zeros(8, 4, dtype=torch.int32)
    out = torch.zeros(8, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="one GPU"):
        B.prepare_combine_unpack(back, token_slot, 16, out)
    with pytest.raises(ValueError, match="one GPU"):
        B.moe_ep_combine_unpack(back, token_slot, 16, out)
    assert list(B._tensors((1, [back, (None, out)], token_slot))) == [back, out, token_slot]
