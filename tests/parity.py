"""Helpers of the GPU parity tests: run the HIP path through the C ABI on W
logical ranks and compare it with the CPU oracle on the same seeded inputs.

Bar: bit-exact for counts, slots, local ids, weights, rows and every payload
byte; combine within 2 bf16 ulp per element (ordered-integer distance on the
bit patterns, +0 and -0 both 0), or 1e-5 relative on the fp32 path. Tails
(slots past the count, rows past expert_num_tokens) are pre-filled with 0xFF
bytes (NaN in bf16/fp32) and must come back untouched.
"""
from __future__ import annotations

import sys
from typing import List

import numpy as np
import torch

import oracle
import workloads as wl
from combine_topk_ids_dest_amd.emulate import LogicalEP

SENTINEL = 0xFF
BF16_ULP_TOL = 2
F32_REL_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_ulp_dist(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a.view(np.uint16)) - ordered(b.view(np.uint16)))


def assert_combine_close(got: np.ndarray, exp: np.ndarray, what: str):
    if exp.dtype == np.uint16:
        d = bf16_ulp_dist(got, exp)
        assert d.max(initial=0) <= BF16_ULP_TOL, \
            f"{what}: max bf16 ulp distance {d.max()} at {np.unravel_index(d.argmax(), d.shape)}"
    else:
        tol = F32_REL_TOL * np.maximum(np.abs(exp), 1e-30)
        bad = ~(np.abs(got - exp) <= tol)
        assert not bad.any(), f"{what}: {bad.sum()} fp32 elements out of tolerance"


def inputs(w: wl.Workload, salt: int = 0, f32_hidden: bool = False):
    srcs = [wl.routing(w, s, salt) for s in range(w.W)]
    pls = []
    for s, (ids, wts) in enumerate(srcs):
        if f32_hidden:
            pls.append([wl.hidden_f32(w, s, salt).view(np.uint8).reshape(w.T, 4 * w.H)])
        else:
            pls.append(wl.payloads(w, s, salt, ids=ids, wts=wts))
    return srcs, pls


def expert_out_host(w: wl.Workload, r: int, counts, salt: int, f32: bool):
    """Y of destination r as [e_local, rows, H] with rows = max(counts):
    drawn rows in each expert's valid prefix, 0xFF bytes (NaN) after it."""
    rows = int(np.max(counts, initial=0))
    if f32:
        blocks = wl.expert_outputs_f32(w, r, counts, salt)
        Y = np.full((w.e_local, rows, w.H), np.nan, np.float32)
    else:
        blocks = wl.expert_outputs_bf16(w, r, counts, salt)
        Y = np.full((w.e_local, rows, w.H), 0xFFFF, np.uint16)
    for e, blk in enumerate(blocks):
        Y[e, :len(blk)] = blk
    return Y


def assert_bytes_equal(got: np.ndarray, exp: np.ndarray, what: str):
    """Byte arrays equal; on a mismatch the message names the first few
    differing positions with both values."""
    if np.array_equal(got, exp):
        return
    bad = np.argwhere(got != exp)
    shown = ", ".join(f"{tuple(int(i) for i in ix)}: got {int(got[tuple(ix)]):#x} "
                      f"want {int(exp[tuple(ix)]):#x}" for ix in bad[:6])
    raise AssertionError(f"{what}: {len(bad)} bytes differ; first {shown}")


def check_pick_ranks(ep, packs, w):
    """The packs' per-expert ranks and counts (ranked form) against the
    oracle's, computed from the oracle's own pack outputs: valid slots and
    every count bit-exact, slots past the count untouched."""
    g_rank = ep.send_rank.cpu().numpy()
    g_ecnt = ep.send_ecnt.cpu().numpy()
    for s in range(w.W):
        exp = oracle.pick_ranks(packs[s]["send_cnt"], packs[s]["send_eloc"], w.e_local)
        assert np.array_equal(g_ecnt[s], exp["send_ecnt"]), f"send_ecnt src {s}"
        for d in range(w.W):
            c = int(packs[s]["send_cnt"][d])
            assert np.array_equal(g_rank[s, d, :c], exp["send_rank"][d, :c]), \
                f"send_rank {s}->{d}"
            assert (g_rank[s, d, c:].view(np.uint32) == 0xFFFFFFFF).all(), \
                f"send_rank tail {s}->{d} written"


def run_full_parity(w: wl.Workload, salt: int = 0, f32: bool = False,
                    srcs=None, pls=None, corrupt_cnt=None, split_batch=False,
                    fp8_group=None, fused_local=False, fp4=False, ranked=False):
    """Whole path on W logical ranks, every output compared element by
    element with the oracle. ranked: the packs also write the per-expert
    ranks (checked against the oracle's) and the receive side is the
    ranked batch (its rows checked against the oracle's scanned batch).
    Returns (ep, oracle result)."""
    if srcs is None:
        srcs, pls = inputs(w, salt, f32_hidden=f32)
    ids_l = [s[0] for s in srcs]
    wts_l = [s[1] for s in srcs]
    Ys = {}

    def yfn(r, b):
        Ys[r] = expert_out_host(w, r, b["expert_num_tokens"], salt, f32)
        return Ys[r]

    # oracle side (host only)
    if fp4:
        packs = [oracle.dispatch_pack_fp4(
            ids_l[s], wts_l[s], w.E, w.W, w.cap,
            pls[s][0].view(np.uint16).reshape(w.T, w.H), pls[s][1:])
            for s in range(w.W)]
    elif fp8_group is None:
        packs = [oracle.dispatch_pack(ids_l[s], wts_l[s], w.E, w.W, w.cap, pls[s])
                 for s in range(w.W)]
    else:
        packs = [oracle.dispatch_pack_fp8(
            ids_l[s], wts_l[s], w.E, w.W, w.cap,
            pls[s][0].view(np.uint16).reshape(w.T, w.H), fp8_group, pls[s][1:])
            for s in range(w.W)]
    send_cnt = np.stack([p["send_cnt"] for p in packs]) if w.W else None
    send_eloc = np.stack([p["send_eloc"] for p in packs])
    send_w = np.stack([p["send_w"] for p in packs])
    if corrupt_cnt is not None:
        s_c, r_c, v_c = corrupt_cnt
        send_cnt = send_cnt.copy()
        send_cnt[s_c, r_c] = v_c
    n_pl = len(packs[0]["send"])
    batches, rets = [], []
    for r in range(w.W):
        recv_pl = [oracle.stack_ranks([packs[s]["send"][p][r] for s in range(w.W)],
                                      min_rows=w.cap if corrupt_cnt else 0)
                   for p in range(n_pl)]
        b = oracle.expert_batch(np.ascontiguousarray(send_cnt[:, r]),
                                np.ascontiguousarray(send_eloc[:, r]), w.W,
                                w.e_local, w.K, w.cap, recv_pl)
        batches.append(b)
        Y = yfn(r, b)
        rets.append(oracle.combine_reduce(
            Y, np.ascontiguousarray(send_cnt[:, r]),
            np.ascontiguousarray(send_eloc[:, r]),
            np.ascontiguousarray(send_w[:, r]), b["recv_row"], w.W, w.e_local,
            w.K, w.cap)["ret"])
    outs = []
    for s in range(w.W):
        back = oracle.stack_ranks([rets[d][s] for d in range(w.W)])
        outs.append(oracle.combine_unpack(back, packs[s]["token_slot"]))

    # GPU side, through the C ABI
    row_bytes = [p.shape[1] * p.itemsize for p in pls[0]]
    dt = torch.float32 if f32 else torch.bfloat16
    ep = LogicalEP(w.T, w.H, w.E, w.K, w.W, w.cap, row_bytes, dt, "cuda",
                   fill=SENTINEL, quant_group=fp8_group, quant_fp4=fp4, ranked=ranked)
    for s in range(w.W):
        ep.set_source(s, ids_l[s], wts_l[s], pls[s])
    for s in range(w.W):
        ep.pack(s)
    torch.cuda.synchronize()
    if ranked:
        check_pick_ranks(ep, packs, w)
    g_cnt = ep.send_cnt.cpu().numpy()
    g_eloc = ep.send_eloc.cpu().numpy()
    g_w = ep.send_w.cpu().numpy()
    g_ts = ep.token_slot.cpu().numpy()
    g_send = [x.cpu().numpy() for x in ep.send]
    exp_err = 0
    for s in range(w.W):
        p = packs[s]
        exp_err |= p["err"]
        assert np.array_equal(g_cnt[s], p["send_cnt"]), f"send_cnt src {s}"
        assert np.array_equal(g_ts[s], p["token_slot"]), f"token_slot src {s}"
        for d in range(w.W):
            c = int(p["send_cnt"][d])
            assert np.array_equal(g_eloc[s, d, :c], p["send_eloc"][d, :c]), f"eloc {s}->{d}"
            assert np.array_equal(g_w[s, d, :c].view(np.uint32),
                                  p["send_w"][d, :c].view(np.uint32)), f"w {s}->{d}"
            assert (g_eloc[s, d, c:].view(np.uint32) == 0xFFFFFFFF).all(), "eloc tail written"
            for q in range(n_pl):
                assert_bytes_equal(g_send[q][s, d, :c], p["send"][q][d, :c],
                                   f"payload {q} {s}->{d}")
                assert (g_send[q][s, d, c:] == SENTINEL).all(), f"payload {q} tail written"

    if corrupt_cnt is not None:
        s_c, r_c, v_c = corrupt_cnt
        ep.send_cnt[s_c, r_c] = v_c

    for r in range(w.W):
        if split_batch:
            ep.batch_plan(r)
            ep.batch_copy(r)
        else:
            ep.batch(r)
        Yd = torch.from_numpy(Ys[r].view(np.int16) if not f32 else Ys[r])
        ep.Y.view(torch.uint8).fill_(SENTINEL)
        ep.Y[:, :Ys[r].shape[1]].copy_(Yd.view(dt) if not f32 else Yd)
        if fused_local:
            ep.reduce_peers(r)
        else:
            ep.reduce(r)
        torch.cuda.synchronize()
        b = batches[r]
        exp_err |= b["err"]
        ent = ep.expert_num_tokens[r].cpu().numpy()
        assert np.array_equal(ent, b["expert_num_tokens"]), f"expert_num_tokens dst {r}"
        rr = ep.recv_row[r].cpu().numpy()
        cnt = np.clip(send_cnt[:, r], 0, w.cap)
        for s in range(w.W):
            c = int(cnt[s])
            assert np.array_equal(rr[s, :c], b["recv_row"][s, :c]), f"recv_row {s}->{r}"
            assert (rr[s, c:].view(np.uint32) == 0xFFFFFFFF).all(), "recv_row tail written"
        for q in range(n_pl):
            gb = ep.b[q].cpu().numpy()
            for e in range(w.e_local):
                n = int(ent[e])
                assert np.array_equal(gb[e, :n], b["b"][q][e, :n]), f"batched payload {q} e{e} dst {r}"
                assert (gb[e, n:] == SENTINEL).all(), f"batched tail written e{e}"
            ep.b[q].fill_(SENTINEL)
        gret = ep.ret[r].cpu()
        gret = gret.view(torch.int16).numpy().view(np.uint16) if not f32 else gret.numpy()
        for s in range(w.W):
            c = int(cnt[s])
            if fused_local and s == r:
                assert (gret[s].view(np.uint8) == SENTINEL).all(), "own block of ret written"
                continue
            assert_combine_close(gret[s, :c], rets[r][s, :c], f"ret {s}->{r}")
            tail = gret[s, c:]
            assert (tail.view(np.uint8) == SENTINEL).all(), "ret tail written"

    for s in range(w.W):
        if fused_local:
            # rank s's own expert output, as its reduce saw it
            Yown = torch.empty_like(ep.Y)
            Yown.view(torch.uint8).fill_(SENTINEL)
            Yd = torch.from_numpy(Ys[s].view(np.int16) if not f32 else Ys[s])
            Yown[:, :Ys[s].shape[1]].copy_(Yd.view(dt) if not f32 else Yd)
            ep.unpack_fused(s, Y=Yown)
            torch.cuda.synchronize()
            del Yown
        else:
            ep.unpack(s)
    torch.cuda.synchronize()
    gout = ep.out.cpu()
    gout = gout.view(torch.int16).numpy().view(np.uint16) if not f32 else gout.numpy()
    for s in range(w.W):
        assert_combine_close(gout[s], outs[s], f"out src {s}")
    assert int(ep.err.item()) == exp_err, f"err flags {ep.err.item()} vs {exp_err}"
    return ep, dict(packs=packs, batches=batches, rets=rets, outs=outs)


# ---------------------------------------------------------------------------
# Full workload sizes (the launch configuration bench.py times)
# ---------------------------------------------------------------------------

def column_windows(nbytes: int, width: int = 64):
    """Byte windows of a row: the start, the middle, the end, and in every
    4 KiB pass of 256 lanes x 16 B one window across its start and one in
    its middle (16-byte aligned), so each vector pass of every kernel is
    compared."""
    starts = {0, (nbytes // 2) // 16 * 16, nbytes - width}
    for k in range(0, nbytes, 4096):
        starts.add(max(0, k - width // 2))
        starts.add(k + 2048)
    out = []
    for s in sorted(starts):
        s = max(0, min(s, nbytes - width)) // 16 * 16
        out.extend(range(s, min(nbytes, s + width)))
    return np.array(sorted(set(out)), dtype=np.int64)


def run_fullsize(w: wl.Workload, seed: int = 0, fp8_group=None, fp4=False, ranked=False):
    """Whole path at full size. Every integer output and every valid payload
    byte is compared; the combine is compared on column windows that the
    oracle computes exactly (the reduction is independent per column). With
    fp8_group the pack quantises payload 0; the oracle quantises the same
    rows and its codes and scales are the expected rows. ranked: the packs'
    per-expert ranks are compared too and the receive side is the ranked
    batch."""
    dev = torch.device("cuda")
    say(f"[fullsize] {w.name}: generating inputs")
    srcs = [wl.routing(w, s, seed) for s in range(w.W)]
    pls = [wl.payloads(w, s, seed, ids=srcs[s][0], wts=srcs[s][1]) for s in range(w.W)]
    row_bytes = [p.shape[1] for p in pls[0]]
    ep = LogicalEP(w.T, w.H, w.E, w.K, w.W, w.cap, row_bytes, torch.bfloat16, dev,
                   fill=SENTINEL, quant_group=fp8_group, quant_fp4=fp4, ranked=ranked)
    n_pl = len(ep.send)
    for s in range(w.W):
        ep.set_source(s, srcs[s][0], srcs[s][1], pls[s])
    if fp4:
        say(f"[fullsize] {w.name}: oracle 4-bit quantisation")
        qs, ss = [], []
        for s in range(w.W):
            q, sc = oracle.quantize_fp4(pls[s][0].view(np.uint16).reshape(w.T, w.H))
            scp = np.zeros((w.T, oracle.fp4_scale_pitch(w.H)), np.uint8)
            scp[:, :sc.shape[1]] = sc
            qs.append(torch.from_numpy(q))
            ss.append(torch.from_numpy(scp))
        exp_src = [torch.stack(qs).to(dev), torch.stack(ss).to(dev)] + ep.src[1:]
    elif fp8_group is None:
        exp_src = ep.src
    else:
        say(f"[fullsize] {w.name}: oracle quantisation")
        qs, ss = [], []
        for s in range(w.W):
            q, sc = oracle.quantize_fp8(pls[s][0].view(np.uint16).reshape(w.T, w.H), fp8_group)
            Gp = (sc.shape[1] + 3) // 4 * 4
            scp = np.zeros((w.T, Gp), np.float32)
            scp[:, :sc.shape[1]] = sc
            qs.append(torch.from_numpy(q))
            ss.append(torch.from_numpy(scp.view(np.uint8).reshape(w.T, -1)))
        exp_src = [torch.stack(qs).to(dev), torch.stack(ss).to(dev)] + ep.src[1:]
    wl.expert_outputs_device(ep.Y, seed=2000 + w.wid)
    # the expert outputs are an input of the combine; the oracle gets a host
    # copy of the column windows it checks
    hcols = column_windows(w.H * 2) // 2
    hcols = np.unique(hcols)
    say(f"[fullsize] {w.name}: oracle metadata")
    packs = [oracle.dispatch_pack(srcs[s][0], srcs[s][1], w.E, w.W, w.cap)
             for s in range(w.W)]
    send_cnt = np.stack([p["send_cnt"] for p in packs])
    send_eloc = np.stack([p["send_eloc"] for p in packs])
    send_w = np.stack([p["send_w"] for p in packs])
    batches = [oracle.expert_batch(np.ascontiguousarray(send_cnt[:, r]),
                                   np.ascontiguousarray(send_eloc[:, r]), w.W,
                                   w.e_local, w.K, w.cap) for r in range(w.W)]
    maxn = max(int(b["expert_num_tokens"].max(initial=0)) for b in batches)
    Ysub = ep.Y[:, :max(maxn, 1)][:, :, torch.from_numpy(hcols).to(dev)].contiguous()
    Ysub = Ysub.cpu().view(torch.int16).numpy().view(np.uint16)

    say(f"[fullsize] {w.name}: pack on the GPU")
    for s in range(w.W):
        ep.pack(s)
    torch.cuda.synchronize()
    assert np.array_equal(ep.send_cnt.cpu().numpy(), send_cnt), "send_cnt"
    assert np.array_equal(ep.token_slot.cpu().numpy(),
                          np.stack([p["token_slot"] for p in packs])), "token_slot"
    g_eloc = ep.send_eloc.cpu().numpy()
    g_w = ep.send_w.cpu().numpy()
    for s in range(w.W):
        for d in range(w.W):
            c = int(send_cnt[s, d])
            assert np.array_equal(g_eloc[s, d, :c], send_eloc[s, d, :c]), f"eloc {s}->{d}"
            assert np.array_equal(g_w[s, d, :c].view(np.uint32),
                                  send_w[s, d, :c].view(np.uint32)), f"w {s}->{d}"
    if ranked:
        check_pick_ranks(ep, packs, w)
    # every valid payload byte: send[s, d, slot] is the source row of the
    # token the oracle put in that slot
    tok_of = {}
    for s in range(w.W):
        ts = packs[s]["token_slot"]
        for d in range(w.W):
            toks = np.nonzero(ts[:, d] >= 0)[0]
            order = np.argsort(ts[toks, d], kind="stable")
            tok_of[(s, d)] = toks[order]
            idx = torch.from_numpy(tok_of[(s, d)]).to(dev)
            c = len(idx)
            for p in range(n_pl):
                exp = exp_src[p][s].index_select(0, idx)
                assert torch.equal(ep.send[p][s, d, :c], exp), f"payload {p} {s}->{d}"
                assert bool((ep.send[p][s, d, c:] == SENTINEL).all()), f"payload {p} tail {s}->{d}"

    say(f"[fullsize] {w.name}: batch + reduce on the GPU")
    rets_sub = []
    src_flat = [x.reshape(w.W * w.T, -1) for x in exp_src]
    for r in range(w.W):
        for p in range(n_pl):
            ep.b[p].fill_(SENTINEL)
        ep.batch(r)
        ep.reduce(r)
        torch.cuda.synchronize()
        b = batches[r]
        ent = ep.expert_num_tokens[r].cpu().numpy()
        assert np.array_equal(ent, b["expert_num_tokens"]), f"expert_num_tokens {r}"
        rr = ep.recv_row[r].cpu().numpy()
        e_all, row_all, src_all = [], [], []
        for s in range(w.W):
            c = int(send_cnt[s, r])
            assert np.array_equal(rr[s, :c], b["recv_row"][s, :c]), f"recv_row {s}->{r}"
            rows = b["recv_row"][s, :c]                       # [c, slots]
            m = rows >= 0
            e_all.append(send_eloc[s, r, :c][m])
            row_all.append(rows[m])
            src_all.append(np.broadcast_to((s * w.T + tok_of[(s, r)])[:, None], rows.shape)[m])
        e_all = np.concatenate(e_all) if e_all else np.zeros(0, np.int32)
        row_all = np.concatenate(row_all) if row_all else np.zeros(0, np.int32)
        src_all = np.concatenate(src_all) if src_all else np.zeros(0, np.int64)
        for e in range(w.e_local):
            n = int(ent[e])
            sel = e_all == e
            order = np.argsort(row_all[sel], kind="stable")
            assert np.array_equal(row_all[sel][order], np.arange(n))
            idx = torch.from_numpy(src_all[sel][order].astype(np.int64)).to(dev)
            for p in range(n_pl):
                assert torch.equal(ep.b[p][e, :n], src_flat[p].index_select(0, idx)), \
                    f"batched payload {p} e{e} dst {r}"
                assert bool((ep.b[p][e, n:] == SENTINEL).all()), f"batched tail e{e} dst {r}"
        # combine reduce on the column windows
        exp_ret = oracle.combine_reduce(
            Ysub, np.ascontiguousarray(send_cnt[:, r]),
            np.ascontiguousarray(send_eloc[:, r]), np.ascontiguousarray(send_w[:, r]),
            b["recv_row"], w.W, w.e_local, w.K, w.cap)["ret"]
        rets_sub.append(exp_ret)
        gret = ep.ret[r][:, :, torch.from_numpy(hcols).to(dev)].cpu()
        gret = gret.view(torch.int16).numpy().view(np.uint16)
        for s in range(w.W):
            c = int(send_cnt[s, r])
            assert_combine_close(gret[s, :c], exp_ret[s, :c], f"ret {s}->{r}")
            assert bool((ep.ret[r][s, c:].view(torch.uint8) == SENTINEL).all()), "ret tail"

    say(f"[fullsize] {w.name}: unpack on the GPU")
    for s in range(w.W):
        ep.unpack(s)
    torch.cuda.synchronize()
    gout = ep.out[:, :, torch.from_numpy(hcols).to(dev)].cpu()
    gout = gout.view(torch.int16).numpy().view(np.uint16)
    for s in range(w.W):
        back = oracle.stack_ranks([rets_sub[d][s] for d in range(w.W)])
        exp_out = oracle.combine_unpack(back, packs[s]["token_slot"])
        assert_combine_close(gout[s], exp_out, f"out src {s}")
        pad = (srcs[s][0] < 0).all(axis=1)
        if pad.any():
            pidx = torch.from_numpy(np.nonzero(pad)[0]).to(dev)
            assert bool((ep.out[s].index_select(0, pidx).view(torch.int16) == 0).all()), \
                "padding rows must be +0.0"
    assert int(ep.err.item()) == 0
    say(f"[fullsize] {w.name}: ok")
    return ep


STEP_OUTPUTS = ("send_cnt", "token_slot", "send_eloc", "send_w", "expert_num_tokens",
                "recv_row", "ret", "out")


def snapshot_step(ep):
    """Device copies of every output of a step, and the valid rows of the
    last destination's expert batch."""
    names = STEP_OUTPUTS + (("send_rank", "send_ecnt") if ep.ranked else ())
    snap = {n: getattr(ep, n).clone() for n in names}
    snap["send"] = [x.clone() for x in ep.send]
    r = ep.W - 1
    ent = ep.expert_num_tokens[r].tolist()
    snap["b_last"] = [torch.cat([b[e, :ent[e]] for e in range(ep.e_local)])
                      for b in ep.b_lanes[r % ep.lanes]]
    return snap


def check_lanes_step(w: wl.Workload, ref, lanes: int, seed: int = 0, ranked: bool = False):
    """The whole step as bench.py times it, with the ranks over `lanes` HIP
    streams, on the inputs of run_fullsize: every output byte equals the
    one-stream outputs in `ref` (snapshot_step of the path that run_fullsize
    checked against the oracle)."""
    say(f"[fullsize] {w.name}: whole step over {lanes} lanes (ranked={ranked})")
    srcs = [wl.routing(w, s, seed) for s in range(w.W)]
    pls = [wl.payloads(w, s, seed, ids=srcs[s][0], wts=srcs[s][1]) for s in range(w.W)]
    ep = LogicalEP(w.T, w.H, w.E, w.K, w.W, w.cap, [p.shape[1] for p in pls[0]],
                   torch.bfloat16, torch.device("cuda"), fill=SENTINEL, lanes=lanes,
                   ranked=ranked)
    for s in range(w.W):
        ep.set_source(s, srcs[s][0], srcs[s][1], pls[s])
    wl.expert_outputs_device(ep.Y, seed=2000 + w.wid)
    ep.share_expert_outputs()
    streams = [torch.cuda.Stream() for _ in range(lanes)]
    ep.step(streams=streams)
    torch.cuda.synchronize()
    got = snapshot_step(ep)
    for n in STEP_OUTPUTS + (("send_rank", "send_ecnt") if ranked else ()):
        assert torch.equal(got[n].view(torch.uint8), ref[n].view(torch.uint8)), f"lanes: {n}"
    for p, (a, b) in enumerate(zip(got["send"], ref["send"])):
        assert torch.equal(a, b), f"lanes: send payload {p}"
    for p, (a, b) in enumerate(zip(got["b_last"], ref["b_last"])):
        assert torch.equal(a, b), f"lanes: batch of the last destination, payload {p}"
    assert int(ep.err.item()) == 0
    say(f"[fullsize] {w.name}: {lanes} lanes ok")
