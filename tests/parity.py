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


def run_full_parity(w: wl.Workload, salt: int = 0, f32: bool = False,
                    srcs=None, pls=None, corrupt_cnt=None):
    """Whole path on W logical ranks, every output compared element by
    element with the oracle. Returns (ep, oracle result)."""
    if srcs is None:
        srcs, pls = inputs(w, salt, f32_hidden=f32)
    ids_l = [s[0] for s in srcs]
    wts_l = [s[1] for s in srcs]
    Ys = {}

    def yfn(r, b):
        Ys[r] = expert_out_host(w, r, b["expert_num_tokens"], salt, f32)
        return Ys[r]

    # oracle side (host only)
    packs = [oracle.dispatch_pack(ids_l[s], wts_l[s], w.E, w.W, w.cap, pls[s])
             for s in range(w.W)]
    send_cnt = np.stack([p["send_cnt"] for p in packs]) if w.W else None
    send_eloc = np.stack([p["send_eloc"] for p in packs])
    send_w = np.stack([p["send_w"] for p in packs])
    if corrupt_cnt is not None:
        s_c, r_c, v_c = corrupt_cnt
        send_cnt = send_cnt.copy()
        send_cnt[s_c, r_c] = v_c
    n_pl = len(pls[0])
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
                   fill=SENTINEL)
    for s in range(w.W):
        ep.set_source(s, ids_l[s], wts_l[s], pls[s])
    for s in range(w.W):
        ep.pack(s)
    torch.cuda.synchronize()
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
                assert np.array_equal(g_send[q][s, d, :c], p["send"][q][d, :c]), \
                    f"payload {q} {s}->{d}"
                assert (g_send[q][s, d, c:] == SENTINEL).all(), f"payload {q} tail written"

    if corrupt_cnt is not None:
        s_c, r_c, v_c = corrupt_cnt
        ep.send_cnt[s_c, r_c] = v_c

    for r in range(w.W):
        ep.batch(r)
        Yd = torch.from_numpy(Ys[r].view(np.int16) if not f32 else Ys[r])
        ep.Y.view(torch.uint8).fill_(SENTINEL)
        ep.Y[:, :Ys[r].shape[1]].copy_(Yd.view(dt) if not f32 else Yd)
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
            assert_combine_close(gret[s, :c], rets[r][s, :c], f"ret {s}->{r}")
            tail = gret[s, c:]
            assert (tail.view(np.uint8) == SENTINEL).all(), "ret tail written"

    for s in range(w.W):
        ep.unpack(s)
    torch.cuda.synchronize()
    gout = ep.out.cpu()
    gout = gout.view(torch.int16).numpy().view(np.uint16) if not f32 else gout.numpy()
    for s in range(w.W):
        assert_combine_close(gout[s], outs[s], f"out src {s}")
    assert int(ep.err.item()) == exp_err, f"err flags {ep.err.item()} vs {exp_err}"
    return ep, dict(packs=packs, batches=batches, rets=rets, outs=outs)
