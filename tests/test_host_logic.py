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


def _send_side_tensors(T=8, K=2, W=4, cap=8, slots=2, row=64):
    z = torch.zeros
    return dict(
        topk_ids=z(T, K, dtype=torch.int32), topk_weights=z(T, K),
        payloads=[(z(T, row, dtype=torch.uint8), z(W, cap, row, dtype=torch.uint8))],
        send_cnt=z(W, dtype=torch.int32), send_eloc=z(W, cap, slots, dtype=torch.int32),
        send_w=z(W, cap, slots), token_slot=z(T, W, dtype=torch.int32),
        err_flags=z(1, dtype=torch.int32), workspace=z(4096, dtype=torch.uint8))


def _pack_call(t, E=8, W=4, cap=8):
    return B.prepare_dispatch_pack(t["topk_ids"], t["topk_weights"], E, W, cap,
                                   t["payloads"], t["send_cnt"], t["send_eloc"],
                                   t["send_w"], t["token_slot"], t["err_flags"],
                                   t["workspace"])


def test_binding_checks_pack_shapes_before_the_device():
    """Every tensor of a pack call is checked against T, K, W, cap and slots
    (the C ABI sees pointers only, so a short buffer would be written out of
    bounds on the device). Correct shapes on host tensors reach the one-GPU
    check; each wrong one is refused before it."""
    with pytest.raises(ValueError, match="one GPU"):
        _pack_call(_send_side_tensors())
    z = torch.zeros
    wrong = {
        "topk_weights": z(8, 3),
        "send_cnt": z(3, dtype=torch.int32),
        "send_eloc": z(4, 7, 2, dtype=torch.int32),
        "send_w": z(4, 8, 2, dtype=torch.float64),
        "token_slot": z(8, 3, dtype=torch.int32),
        "err_flags": z(0, dtype=torch.int32),
        "payloads": [(z(7, 64, dtype=torch.uint8), z(4, 8, 64, dtype=torch.uint8))],
    }
    for name, bad in wrong.items():
        t = _send_side_tensors()
        t[name] = bad
        with pytest.raises(ValueError) as e:
            _pack_call(t)
        assert "one GPU" not in str(e.value), name
    t = _send_side_tensors()
    t["payloads"] = [(z(8, 64, dtype=torch.uint8), z(4, 7, 64, dtype=torch.uint8))]
    with pytest.raises(ValueError, match="at least"):
        _pack_call(t)
    # a padded metadata rank stride is accepted when both arrays share it
    base_e = z(4, 16 + 5, dtype=torch.int32)
    base_w = z(4, 16 + 5)
    t = _send_side_tensors()
    t["send_eloc"] = base_e[:, :16].view(4, 8, 2)
    t["send_w"] = base_w[:, :16].view(4, 8, 2)
    with pytest.raises(ValueError, match="one GPU"):
        _pack_call(t)
    t["send_w"] = z(4, 8, 2)
    with pytest.raises(ValueError, match="share a rank stride"):
        _pack_call(t)


def test_binding_checks_quantised_pack_shapes():
    t = _send_side_tensors(row=64)
    z = torch.zeros
    hidden = z(8, 32, dtype=torch.bfloat16)
    args = lambda q, sc: (t["topk_ids"], t["topk_weights"], 8, 4, 8, hidden, 32, q, sc,
                          [], t["send_cnt"], t["send_eloc"], t["send_w"],
                          t["token_slot"], t["err_flags"], t["workspace"])
    with pytest.raises(ValueError, match="one GPU"):
        B.prepare_dispatch_pack_fp8(*args(z(4, 8, 32, dtype=torch.uint8), z(4, 8, 4)))
    for q, sc in ((z(4, 8, 31, dtype=torch.uint8), z(4, 8, 4)),
                  (z(4, 7, 32, dtype=torch.uint8), z(4, 8, 4)),
                  (z(4, 8, 32, dtype=torch.uint8), z(4, 8, 3)),
                  (z(4, 8, 32, dtype=torch.int32), z(4, 8, 4))):
        with pytest.raises(ValueError) as e:
            B.prepare_dispatch_pack_fp8(*args(q, sc))
        assert "one GPU" not in str(e.value)
    fp4 = lambda q, sc: B.prepare_dispatch_pack_fp4(
        t["topk_ids"], t["topk_weights"], 8, 4, 8, hidden, q, sc, [], t["send_cnt"],
        t["send_eloc"], t["send_w"], t["token_slot"], t["err_flags"], t["workspace"])
    with pytest.raises(ValueError, match="one GPU"):
        fp4(z(4, 8, 16, dtype=torch.uint8), z(4, 8, 16, dtype=torch.uint8))
    for q, sc in ((z(4, 8, 8, dtype=torch.uint8), z(4, 8, 16, dtype=torch.uint8)),
                  (z(4, 7, 16, dtype=torch.uint8), z(4, 8, 16, dtype=torch.uint8)),
                  (z(4, 8, 16, dtype=torch.uint8), z(4, 8, 2, dtype=torch.uint8))):
        with pytest.raises(ValueError) as e:
            fp4(q, sc)
        assert "one GPU" not in str(e.value)


def test_binding_checks_receive_and_combine_shapes():
    """Batch, sanitise, reduce and unpack calls: counts, local ids, rows,
    expert batches and outputs against W, e_local, cap, slots and H."""
    z = torch.zeros
    W, el, K, cap, H = 4, 2, 2, 8, 32
    ecap = W * cap
    ok = dict(cnt=z(W, dtype=torch.int32), eloc=z(W, cap, 2, dtype=torch.int32),
              pl=[(z(W, cap, 64, dtype=torch.uint8), z(el, ecap, 64, dtype=torch.uint8))],
              ent=z(el, dtype=torch.int32), row=z(W, cap, 2, dtype=torch.int32),
              err=z(1, dtype=torch.int32), ws=z(4096, dtype=torch.uint8))

    def batch(d):
        return B.prepare_expert_batch(d["cnt"], d["eloc"], W, el, K, cap, d["pl"],
                                      d["ent"], d["row"], d["err"], d["ws"])

    with pytest.raises(ValueError, match="one GPU"):
        batch(ok)
    for k, bad in (("cnt", z(W - 1, dtype=torch.int32)),
                   ("eloc", z(W, cap - 1, 2, dtype=torch.int32)),
                   ("ent", z(el + 1, dtype=torch.int32)),
                   ("row", z(W, cap, 1, dtype=torch.int32)),
                   ("pl", [(z(W, cap, 64, dtype=torch.uint8),
                            z(el, ecap - 1, 64, dtype=torch.uint8))]),
                   ("pl", [(z(W - 1, cap, 64, dtype=torch.uint8),
                            z(el, ecap, 64, dtype=torch.uint8))])):
        d = dict(ok)
        d[k] = bad
        with pytest.raises(ValueError) as e:
            batch(d)
        assert "one GPU" not in str(e.value), k
    with pytest.raises(ValueError) as e:
        B.prepare_sanitize_expert_ids(ok["cnt"], ok["eloc"], W, el, K, cap, -1,
                                      z(W, cap, 3, dtype=torch.int32), None)
    assert "one GPU" not in str(e.value)

    Y = z(el, ecap, H, dtype=torch.bfloat16)
    wts = z(W, cap, 2)
    ret = z(W, cap, H, dtype=torch.bfloat16)

    def reduce(Y=Y, wts=wts, ret=ret, row=ok["row"]):
        return B.prepare_combine_reduce(Y, ok["cnt"], ok["eloc"], wts, row, W, el, K,
                                        cap, ret)

    with pytest.raises(ValueError, match="one GPU"):
        reduce()
    for kw in (dict(Y=z(el, ecap - 1, H, dtype=torch.bfloat16)),
               dict(Y=z(el - 1, ecap, H, dtype=torch.bfloat16)),
               dict(wts=z(W, cap, 1)),
               dict(ret=z(W, cap, H - 8, dtype=torch.bfloat16)),
               dict(ret=z(W, cap - 1, H, dtype=torch.bfloat16)),
               dict(row=z(W, cap - 1, 2, dtype=torch.int32))):
        with pytest.raises(ValueError) as e:
            reduce(**kw)
        assert "one GPU" not in str(e.value), kw
    T = 6
    ts = z(T, W, dtype=torch.int32)
    out = z(T, H, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="one GPU"):
        B.prepare_combine_unpack(ret, ts, cap, out)
    for b, t_, o in ((z(W, cap - 1, H, dtype=torch.bfloat16), ts, out),
                     (ret, z(T, W + 1, dtype=torch.int32), out),
                     (ret, ts, z(T - 1, H, dtype=torch.bfloat16)),
                     (ret, ts, z(T, H + 8, dtype=torch.bfloat16))):
        with pytest.raises(ValueError) as e:
            B.prepare_combine_unpack(b, t_, cap, o)
        assert "one GPU" not in str(e.value)
    own = dict(e=z(cap, 2, dtype=torch.int32), w=z(cap, 2), r=z(cap, 2, dtype=torch.int32))
    with pytest.raises(ValueError, match="one GPU"):
        B.prepare_combine_unpack_fused(ret, ts, cap, 0, Y, own["e"], own["w"], own["r"],
                                       el, K, out)
    with pytest.raises(ValueError) as e:
        B.prepare_combine_unpack_fused(ret, ts, cap, 0, Y, own["e"], own["w"],
                                       z(cap - 1, 2, dtype=torch.int32), el, K, out)
    assert "one GPU" not in str(e.value)


def test_bench_receive_form():
    """--receive auto takes the sender-ranked receive side for batches of one
    routing tile (decode, tiny) and the receiver's scan above."""
    W = wl.WORKLOADS
    assert bench.receive_ranked("auto", W[1].T) and bench.receive_ranked("auto", W[4].T)
    assert not any(bench.receive_ranked("auto", W[i].T) for i in (2, 3, 5))
    assert bench.receive_ranked("auto", 256) and not bench.receive_ranked("auto", 257)
    assert bench.receive_ranked("ranked", 4096) and not bench.receive_ranked("scan", 64)
    # auto keeps the scan where the ranked form does not apply
    assert not bench.receive_ranked("auto", 64, K=64, E=128)
    assert not bench.receive_ranked("auto", 64, K=8, E=8192)


def test_bench_refuses_more_than_one_gpu():
    """The bench measures one GPU (the W ranks are logical partitions of it):
    --gpus above 1 exits with a message before touching any device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus must be 1" in r.stderr


def test_bench_roofline_call_skips_the_receive_plan():
    """The roofline names the call with the most time among those that move
    rows; the receive plan (index data only) never is that call."""
    import bench
    assert bench.roofline_call({"pack": 11.5, "batch_plan": 12.0, "batch_copy": 9.0,
                                "reduce": 11.0, "unpack": 7.0}) == "pack"
    assert bench.roofline_call({"pack": 1.0, "batch": 3.0, "reduce": 2.0}) == "batch"
    assert bench.roofline_call({"batch_plan": 1.0}) == "batch_plan"
