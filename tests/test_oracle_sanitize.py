"""Pins of the oracle's received-id sanitiser (FlashInfer module,
moe_a2a_sanitize_expert_ids: ids of received entries that are not valid
tokens become a sentinel) against a hand example and against a brute-force
construction from the routing with Python sets and sorts."""
import numpy as np
import pytest

import oracle
import workloads as wl


def test_sanitize_hand_example():
    # W=3 sources, e_local=2, K=2 -> slots 2; max_num_tokens 4 -> cap 4.
    cnt = np.array([2, 0, 5], np.int32)                  # 5 > cap: clamped, bit 4
    eloc = np.array([
        [[0, 1], [1, -1], [0, 0], [1, 1]],               # rows 2, 3 are stale
        [[1, 1], [0, 0], [1, 0], [0, 1]],                # no valid row
        [[1, 3], [-1, 0], [0, 1], [1, 0]],               # 3 >= e_local: bit 2
    ], np.int32)
    r = oracle.sanitize_expert_ids(cnt, eloc, 3, 2, 2, 4, 99)
    assert r["err"] == oracle.ERR_CNT | oracle.ERR_ELOC
    assert r["ids"].tolist() == [
        [[0, 1], [1, 99], [99, 99], [99, 99]],
        [[99, 99], [99, 99], [99, 99], [99, 99]],
        [[1, 99], [99, 0], [0, 1], [1, 0]],
    ]
    # a negative count clamps to 0; ids in rows past the count are not read
    r = oracle.sanitize_expert_ids(np.array([-3, 1, 0], np.int32), eloc, 3, 2, 2, 4, -1)
    assert r["err"] == oracle.ERR_CNT
    assert (r["ids"][0] == -1).all() and r["ids"][1, 0].tolist() == [1, 1]


def _brute_received_ids(srcs, E, W, d, cap, slots, invalid):
    """Received ids on rank d written from the definition: the tokens of each
    source with a pick on d, ascending; each row holds that token's local ids
    on d in router order, then the sentinel; rows past the count hold only
    the sentinel."""
    e_local = E // W
    out = np.full((W, cap, slots), invalid, np.int32)
    for s, ids in enumerate(srcs):
        toks = sorted(t for t in range(ids.shape[0])
                      if any(0 <= i < E and i // e_local == d for i in ids[t]))
        for r, t in enumerate(toks):
            loc = [int(i) - d * e_local for i in ids[t] if 0 <= i < E and i // e_local == d]
            out[s, r, :len(loc)] = loc
    return out


@pytest.mark.parametrize("W,E,K", [(2, 8, 2), (4, 8, 3), (3, 3, 1), (4, 16, 4)])
def test_sanitize_matches_brute_force_from_routing(W, E, K):
    rng = np.random.default_rng(1000 * W + 10 * E + K)
    T = cap = 9
    e_local = E // W
    slots = min(K, e_local)
    srcs = []
    for s in range(W):
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
        ids[rng.random(T) < 0.2] = -1                    # padding rows
        srcs.append(ids)
    packs = [oracle.dispatch_pack(ids, np.ones(ids.shape, np.float32), E, W, cap)
             for ids in srcs]
    for d in range(W):
        cnt = np.array([p["send_cnt"][d] for p in packs], np.int32)
        eloc = np.stack([p["send_eloc"][d] for p in packs])
        got = oracle.sanitize_expert_ids(cnt, eloc, W, e_local, K, cap, -9)
        assert got["err"] == 0
        np.testing.assert_array_equal(
            got["ids"], _brute_received_ids(srcs, E, W, d, cap, slots, -9))


@pytest.mark.parametrize("wid", [1, 4])
def test_sanitize_keeps_exactly_the_picks_the_batch_places(wid):
    """Valid entries are exactly those the expert batch gives a row, and keep
    their id; on a workload's real routing (sizes scaled for the CPU)."""
    w = wl.WORKLOADS[wid]
    if wid == 1:
        w = w.scaled(T=300, cap=300)
    d = w.W // 2
    cnt, eloc = [], []
    for s in range(w.W):
        ids, wts = wl.routing(w, s, 0)
        p = oracle.dispatch_pack(ids, wts, w.E, w.W, w.cap)
        cnt.append(p["send_cnt"][d])
        eloc.append(p["send_eloc"][d])
    cnt = np.array(cnt, np.int32)
    eloc = np.stack(eloc)
    got = oracle.sanitize_expert_ids(cnt, eloc, w.W, w.e_local, w.K, w.cap, -1)
    assert got["err"] == 0
    b = oracle.expert_batch(cnt, eloc, w.W, w.e_local, w.K, w.cap)
    valid = b["recv_row"] >= 0
    ids = got["ids"]
    assert np.array_equal(ids >= 0, valid)
    assert np.array_equal(ids[valid], eloc[valid])
