"""Pins of the CPU oracle to facts other than itself (runs without a GPU).

Sources of truth, none of which is the oracle's own code:
  * hand-worked examples in tests/golden/ (derived by hand from the method
    on the vLLM "alltoall_batched" documentation page, each step cited);
  * brute force over micro shapes against independent set/sort/dictionary
    formulations (tests/brute.py);
  * closed forms and special cases that reduce to a textbook operation
    (stream compaction, stable counting sort, a rank-major concatenation);
  * invariants the page states (each token sent once per destination,
    padding never sent and its output zero, counts = unique pairs, a round
    trip with identity experts returns the input).
"""
import itertools
import json
import os

import numpy as np
import pytest

import brute
import oracle
import workloads as wl

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bf16(vals):
    return wl.f32_to_bf16_bits(np.asarray(vals, np.float32))


def _hex(s):
    return int(s, 16)


def _f32_from_hex(h):
    return np.array([_hex(h)], np.uint32).view(np.float32)[0]


# --------------------------------------------------------------------------
# Hand-worked golden examples
# --------------------------------------------------------------------------

def test_capacities_match_page_definition():
    # capacities(): (max_num_tokens, min(topk, e_local), max_num_tokens * W)
    assert oracle.capacities(8, 256, 8, 4096) == (4096, 8, 32768)
    assert oracle.capacities(2, 8, 8, 8192) == (8192, 1, 65536)
    assert oracle.capacities(8, 256, 32, 128) == (128, 8, 4096)
    assert oracle.capacities(3, 6, 3, 5) == (5, 2, 15)


def test_golden_pack():
    g = _gold("worked_example.json")["pack"]
    ids = np.array(g["topk_ids"], np.int32)
    wts = np.array(g["topk_weights"], np.float32)
    rows = np.array(g["payload_rows"], np.int32)
    r = oracle.dispatch_pack(ids, wts, g["E"], g["W"], g["max_num_tokens"],
                             [rows])
    assert (r["cap"], r["slots"]) == (g["expect_cap"], g["expect_slots"])
    assert r["err"] == 0
    assert r["send_cnt"].tolist() == g["send_cnt"]
    assert r["token_slot"].tolist() == g["token_slot"]
    for d in range(g["W"]):
        c = g["send_cnt"][d]
        assert r["send_eloc"][d, :c].tolist() == g["send_eloc"][d]
        assert r["send_w"][d, :c].tolist() == g["send_w"][d]
        got_rows = r["send"][0][d, :c].view(np.int32)
        assert got_rows.tolist() == [g["payload_rows"][t]
                                     for t in g["send_tokens"][d]]


def test_golden_batch():
    g = _gold("worked_example.json")["batch"]
    W, el, K, cap = g["W"], g["e_local"], g["K"], g["max_num_tokens"]
    cnt = np.array(g["recv_cnt"], np.int32)
    eloc = np.array(g["recv_eloc"], np.int32)
    pay = np.zeros((W, cap, 1), np.int32)
    for s in range(W):
        for slot in range(cap):
            pay[s, slot, 0] = 100 * s + slot
    r = oracle.expert_batch(cnt, eloc, W, el, K, cap, [pay])
    assert r["err"] == 0
    assert r["expert_num_tokens"].tolist() == g["expert_num_tokens"]
    for s in range(W):
        c = g["recv_cnt"][s]
        assert r["recv_row"][s, :c].tolist() == g["recv_row_valid"][s]
    b = r["b"][0].view(np.int32)
    for e in range(el):
        n = g["expert_num_tokens"][e]
        assert b[e, :n, 0].tolist() == [100 * s + slot for s, slot in
                                        g["batched_sources"][e]]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_golden_reduce(dtype):
    G = _gold("worked_example.json")
    g, gb = G["reduce"], G["batch"]
    W, el, K, cap = gb["W"], gb["e_local"], gb["K"], gb["max_num_tokens"]
    cnt = np.array(gb["recv_cnt"], np.int32)
    eloc = np.array(gb["recv_eloc"], np.int32)
    rows = oracle.expert_batch(cnt, eloc, W, el, K, cap)["recv_row"]
    Y = np.array(g["Y"], np.float32)
    Y = _bf16(Y) if dtype == "bf16" else Y
    w = np.array(g["recv_w"], np.float32)
    ret = oracle.combine_reduce(Y, cnt, eloc, w, rows, W, el, K, cap)["ret"]
    for s in range(W):
        c = gb["recv_cnt"][s]
        exp = np.array(g["ret_valid"][s], np.float32).reshape(c, 2)
        if dtype == "bf16":
            assert np.array_equal(ret[s, :c], _bf16(exp))
        else:
            assert np.array_equal(ret[s, :c], exp)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_reduce_sums_start_at_positive_zero(dtype):
    """The page's finalize() adds the weighted rows into a zeroed output, so
    each slot's sum starts at +0.0 (reading A11): a slot whose only product
    is -0.0, and a slot with no valid pick, both give +0.0 (bits 0), while
    a negative product stays negative. W = 1, e_local = 1, K = 1, cap 4."""
    cnt = np.array([4], np.int32)
    eloc = np.array([[[0], [-1], [0], [0]]], np.int32)
    w = np.array([[[1.0], [1.0], [0.0], [0.5]]], np.float32)
    rows = np.array([[[0], [-1], [1], [2]]], np.int32)
    Yf = np.array([[[-0.0, 2.0], [-1.0, -0.0], [-3.0, 0.0]]], np.float32)
    Y = _bf16(Yf) if dtype == "bf16" else Yf
    ret = oracle.combine_reduce(Y, cnt, eloc, w, rows, 1, 1, 1, 4)["ret"]
    # slot 0: -0.0 * 1 = -0.0, +0.0 + -0.0 = +0.0; 2.0
    # slot 1: no valid pick: +0.0, +0.0
    # slot 2: -1.0 * 0.0 = -0.0 -> +0.0; -0.0 * 0.0 = -0.0 -> +0.0
    # slot 3: -3.0 * 0.5 = -1.5; 0.0
    exp = np.array([[[0.0, 2.0], [0.0, 0.0], [0.0, 0.0], [-1.5, 0.0]]], np.float32)
    exp = _bf16(exp) if dtype == "bf16" else exp
    got = ret.view(np.uint16 if dtype == "bf16" else np.uint32)
    want = exp.view(np.uint16 if dtype == "bf16" else np.uint32)
    assert np.array_equal(got, want), (got, want)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_golden_unpack(dtype):
    G = _gold("worked_example.json")
    g = G["unpack"]
    ts = np.array(G["pack"]["token_slot"], np.int32)
    back = np.array(g["back"], np.float32)
    back = _bf16(back) if dtype == "bf16" else back
    out = oracle.combine_unpack(back, ts)
    exp = np.array(g["out"], np.float32)
    if dtype == "bf16":
        assert np.array_equal(out, _bf16(exp))
        assert out[1].tolist() == g["out_bits_padding_row"]
    else:
        assert np.array_equal(out, exp)
        assert out[1].view(np.uint32).tolist() == g["out_bits_padding_row"]


def test_golden_bf16_rounding():
    g = _gold("rounding.json")["bf16_rne"]
    for fx, bx in g["cases_f32_hex_to_bf16_hex"]:
        assert oracle.round_bf16(float(_f32_from_hex(fx))) == _hex(bx), fx
        assert oracle.round_bf16_bits(_hex(fx)) == _hex(bx), fx


def test_golden_bf16_nan():
    g = _gold("rounding.json")["bf16_nan"]
    for fx, bx in g["cases_f32_hex_to_bf16_hex"]:
        assert oracle.round_bf16_bits(_hex(fx)) == _hex(bx), fx


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_golden_products_rounded_before_add(dtype):
    g = _gold("rounding.json")["no_fma"]
    # one destination, W=1, e_local=2, K=2 (slots 2), cap=1, one slot with
    # picks on experts 0 and 1, each at row 0
    cnt = np.array([1], np.int32)
    eloc = np.array([[[0, 1]]], np.int32)
    w = np.array([[[_f32_from_hex(h) for h in g["w_f32_hex"]]]], np.float32)
    rows = oracle.expert_batch(cnt, eloc, 1, 2, 2, 1)["recv_row"]
    ybits = np.array([_hex(h) for h in g["y_bf16_hex"]], np.uint16)
    if dtype == "bf16":
        Y = ybits.reshape(2, 1, 1)
        ret = oracle.combine_reduce(Y, cnt, eloc, w, rows, 1, 2, 2, 1)["ret"]
        assert int(ret[0, 0, 0]) == _hex(g["expect_ret_bf16_hex"])
    else:
        Y = wl.bf16_bits_to_f32(ybits).reshape(2, 1, 1)
        ret = oracle.combine_reduce(Y, cnt, eloc, w, rows, 1, 2, 2, 1)["ret"]
        assert int(ret.view(np.uint32)[0, 0, 0]) == _hex(g["expect_ret_f32_hex"])


def test_rounding_against_exact_rationals():
    """bf16 rounding of the oracle vs exact rational rounding, on random and
    boundary fp32 values."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0x00800000, 0x7F000000, size=4000, dtype=np.uint64)
    bits = np.concatenate([bits, bits | 0x80000000]).astype(np.uint32)
    # exact ties and their neighbours
    base = rng.integers(0x0100, 0x7E00, size=500).astype(np.uint32) << 16
    bits = np.concatenate([bits, base | 0x8000, base | 0x7FFF, base | 0x8001])
    for b in bits:
        x = np.array([b], np.uint32).view(np.float32)[0]
        assert oracle.round_bf16(float(x)) == brute.bf16_rne_from_fraction(x)


# --------------------------------------------------------------------------
# Brute force over micro shapes
# --------------------------------------------------------------------------

def _check_pack_against_sets(ids, wts, E, W, cap):
    T, K = ids.shape
    pay = np.arange(T * 2, dtype=np.int32).reshape(T, 2) * 7 + 1
    r = oracle.dispatch_pack(ids, wts, E, W, cap, [pay])
    cnt, slot, picks, err = brute.pack_sets(ids, wts, E, W)
    assert r["err"] == err
    assert r["send_cnt"].tolist() == cnt
    slots = r["slots"]
    for t in range(T):
        for d in range(W):
            if (d, t) in slot:
                sl = slot[(d, t)]
                assert r["token_slot"][t, d] == sl
                lst = picks[(d, t)]
                exp_e = [e for e, _ in lst] + [-1] * (slots - len(lst))
                exp_w = [w for _, w in lst] + [0.0] * (slots - len(lst))
                assert r["send_eloc"][d, sl].tolist() == exp_e
                assert r["send_w"][d, sl].tolist() == \
                    [float(np.float32(x)) for x in exp_w]
                assert np.array_equal(r["send"][0][d, sl].view(np.int32), pay[t])
            else:
                assert r["token_slot"][t, d] == -1
    return r


@pytest.mark.parametrize("W,K", [(1, 1), (1, 2), (2, 1), (2, 2), (4, 1), (4, 2)])
def test_pack_exhaustive_micro(W, K):
    """Every id tuple over T=3 tokens, E=4, ids in {-1,0,1,2,3} (duplicates
    and partial padding included), against the set-based formulation."""
    E, T = 4, 3
    vals = [-1, 0, 1, 2, 3]
    wts = (np.arange(T * K, dtype=np.float32).reshape(T, K) + 1) / 8
    per_tok = list(itertools.product(vals, repeat=K))
    for combo in itertools.product(per_tok, repeat=T):
        ids = np.array(combo, np.int32).reshape(T, K)
        _check_pack_against_sets(ids, wts, E, W, cap=T)


def test_pack_random_micro_with_range_errors():
    rng = np.random.default_rng(11)
    for _ in range(1500):
        W = int(rng.choice([1, 2, 3, 4, 6]))
        el = int(rng.integers(1, 4))
        E = W * el
        K = int(rng.integers(1, 5))
        T = int(rng.integers(0, 7))
        ids = rng.integers(-2, E + 2, size=(T, K)).astype(np.int32)
        wts = rng.standard_normal((T, K)).astype(np.float32)
        _check_pack_against_sets(ids, wts, E, W, cap=T + int(rng.integers(0, 3)))


def test_batch_random_micro_against_sorted_entries():
    rng = np.random.default_rng(12)
    for _ in range(1500):
        W = int(rng.integers(1, 5))
        el = int(rng.integers(1, 5))
        K = int(rng.integers(1, 5))
        cap = int(rng.integers(0, 5))
        slots = min(K, el)
        cnt = rng.integers(0, cap + 1, size=W).astype(np.int32)
        eloc = rng.integers(-1, el, size=(W, cap, slots)).astype(np.int32)
        pay = rng.integers(0, 1 << 30, size=(W, cap, 3)).astype(np.int32)
        r = oracle.expert_batch(cnt, eloc, W, el, K, cap, [pay])
        recv = [(int(cnt[s]), eloc[s].tolist()) for s in range(W)]
        row, n = brute.batch_sorted(recv, el, W * cap)
        n_valid = sum(int((eloc[s, :cnt[s]] >= 0).sum()) for s in range(W))
        assert r["err"] == (oracle.ERR_ROWCAP if len(row) < n_valid else 0)
        assert r["expert_num_tokens"].tolist() == n
        b = r["b"][0].view(np.int32)
        for s in range(W):
            for slot in range(int(cnt[s])):
                for j in range(slots):
                    key = (s, slot, j)
                    if key in row:
                        assert r["recv_row"][s, slot, j] == row[key]
                        assert np.array_equal(b[eloc[s, slot, j], row[key]],
                                              pay[s, slot])
                    else:
                        assert r["recv_row"][s, slot, j] == -1


def _dense_combine_reference(ids_l, wts_l, E, W, Ys, rowmap):
    """Per-token dense formulation: out[t] = sum over destinations d in
    ascending order of RNE(sum over the token's picks on d, in router order,
    of fp32(w) * fp32(Y[e, row])), with the row found through a dictionary
    keyed by (source, token, expert). The gather/all-reduce managers on the
    vLLM all2all page compute the same sum densely."""
    e_local = E // W
    outs = []
    for s, (ids, wts) in enumerate(zip(ids_l, wts_l)):
        T, K = ids.shape
        H = Ys[0].shape[2]
        out = np.zeros((T, H), np.uint16)
        for t in range(T):
            for h in range(H):
                acc = np.float32(0.0)
                for d in range(W):
                    part = np.float32(0.0)
                    hit = False
                    for k in range(K):
                        e = int(ids[t, k])
                        if e < 0 or e // e_local != d:
                            continue
                        hit = True
                        el = e - d * e_local
                        row = rowmap[(s, t, e)]
                        y = brute.bf16_to_f32(Ys[d][el, row, h])
                        part = np.float32(part + np.float32(y * wts[t, k]))
                    if hit:
                        acc = np.float32(acc + brute.bf16_to_f32(
                            brute.bf16_rne_from_fraction(part)))
                out[t, h] = brute.bf16_rne_from_fraction(acc)
        outs.append(out)
    return outs


def test_combine_dense_brute_force_tiny():
    rng = np.random.default_rng(13)
    for trial in range(12):
        W = int(rng.integers(1, 4))
        el = int(rng.integers(1, 4))
        E = W * el
        K = int(rng.integers(1, min(E, 4) + 1))
        T = int(rng.integers(1, 6))
        H = 3
        ids_l, wts_l, pls = [], [], []
        for s in range(W):
            ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
            pad = rng.random(T) < 0.2
            ids[pad] = -1
            ids_l.append(ids)
            wts_l.append(rng.random((T, K)).astype(np.float32))
            pls.append([np.zeros((T, 16), np.uint8)])
        Ys = {}

        def yfn(r, b):
            Y = wl.f32_to_bf16_bits(
                rng.standard_normal((el, b["expert_cap"], H)).astype(np.float32))
            Ys[r] = Y
            return Y

        res = oracle.run_path(ids_l, wts_l, pls, E, W, T, yfn)
        # (source, token, expert) -> row, from the set-based formulations
        rowmap = {}
        packs = [brute.pack_sets(ids_l[s], wts_l[s], E, W) for s in range(W)]
        for r in range(W):
            recv = []
            for s in range(W):
                cnt, slot, picks, _ = packs[s]
                slots = min(K, el)
                rows = [None] * cnt[r]
                for (d, t), sl in slot.items():
                    if d == r:
                        lst = [e for e, _ in picks[(d, t)]]
                        rows[sl] = lst + [-1] * (slots - len(lst))
                recv.append((cnt[r], rows))
            row, _ = brute.batch_sorted(recv, el)
            for s in range(W):
                cnt, slot, picks, _ = packs[s]
                for (d, t), sl in slot.items():
                    if d != r:
                        continue
                    for j, (e, _) in enumerate(picks[(d, t)]):
                        rowmap[(s, t, r * el + e)] = row[(s, sl, j)]
        exp = _dense_combine_reference(ids_l, wts_l, E, W, Ys, rowmap)
        for s in range(W):
            assert np.array_equal(res["outs"][s], exp[s]), (trial, s)


# --------------------------------------------------------------------------
# Special cases with textbook answers
# --------------------------------------------------------------------------

def test_w1_pack_is_stream_compaction_and_batch_is_stable_counting_sort():
    rng = np.random.default_rng(21)
    E, K, T = 6, 3, 40
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    ids[rng.random(T) < 0.25] = -1
    ids[3, 1] = -1                                    # partial padding
    wts = rng.random((T, K)).astype(np.float32)
    pay = rng.integers(0, 255, size=(T, 32)).astype(np.uint8)
    r = oracle.dispatch_pack(ids, wts, E, 1, T, [pay])
    routed = [t for t in range(T) if (ids[t] >= 0).any()]
    assert r["send_cnt"][0] == len(routed)
    assert np.array_equal(r["send"][0][0, :len(routed)], pay[routed])
    # receive side, W = 1: a stable sort by expert of the routed entries in
    # (token, k) order
    b = oracle.expert_batch(r["send_cnt"], r["send_eloc"], 1, E, K, T,
                            [r["send"][0]])
    flat = [(t, k, int(ids[t, k])) for t in range(T) for k in range(K)
            if ids[t, k] >= 0]
    order = np.argsort(np.array([e for _, _, e in flat]), kind="stable")
    by_e = {}
    for i in order:
        t, k, e = flat[i]
        by_e.setdefault(e, []).append(t)
    for e in range(E):
        toks = by_e.get(e, [])
        assert b["expert_num_tokens"][e] == len(toks)
        assert np.array_equal(b["b"][0][e, :len(toks)], pay[toks])


def test_e_local_1_rows_are_rank_major_concatenation():
    """With one expert per rank every valid slot has one pick, and the row
    of (s, slot) is sum_{s' < s} cnt[s'] + slot."""
    w = wl.WORKLOADS[3].scaled(T=300, cap=300, H=64)
    packs = [oracle.dispatch_pack(*wl.routing(w, s), w.E, w.W, w.cap)
             for s in range(w.W)]
    for r in range(w.W):
        cnt = np.array([p["send_cnt"][r] for p in packs], np.int32)
        eloc = np.stack([p["send_eloc"][r] for p in packs])
        b = oracle.expert_batch(cnt, eloc, w.W, 1, w.K, w.cap)
        base = np.concatenate([[0], np.cumsum(cnt)])
        for s in range(w.W):
            exp = base[s] + np.arange(cnt[s])
            assert np.array_equal(b["recv_row"][s, :cnt[s], 0], exp)
        assert b["expert_num_tokens"][0] == cnt.sum()


# --------------------------------------------------------------------------
# Invariants stated by the page, on every workload (metadata at full size)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_invariants_full_size_metadata(wid):
    w = wl.WORKLOADS[wid]
    el = w.e_local
    srcs = [wl.routing(w, s) for s in range(w.W)]
    packs = [oracle.dispatch_pack(i, x, w.E, w.W, w.cap) for i, x in srcs]
    for (ids, wts), p in zip(srcs, packs):
        assert p["err"] == 0
        ts = p["token_slot"]
        # I1/I2: each (d, t) at most once; padding rows never sent
        pad = (ids < 0).all(axis=1)
        assert (ts[pad] == -1).all()
        # I3: counts = unique (token, destination) pairs
        pairs = {(t, int(e) // el) for t, e in zip(*np.nonzero(ids >= 0))
                 for e in [ids[t, e]]}
        assert int(p["send_cnt"].sum()) == len(pairs)
        for d in range(w.W):
            toks = np.nonzero(ts[:, d] >= 0)[0]
            # I4: slots strictly ascending in t, and dense 0..cnt-1
            assert np.array_equal(ts[toks, d], np.arange(len(toks)))
            assert len(toks) == p["send_cnt"][d]
            # I5/I6: picks are the token's ids on d, in router order, with
            # their weights bit for bit
            sl = ts[toks, d]
            eloc = p["send_eloc"][d, sl]
            ww = p["send_w"][d, sl]
            sel = (ids[toks] >= 0) & (ids[toks] // el == d)
            for i, t in enumerate(toks):
                exp_e = ids[t][sel[i]] - d * el
                exp_w = wts[t][sel[i]]
                n = len(exp_e)
                assert eloc[i, :n].tolist() == exp_e.tolist()
                assert (eloc[i, n:] == -1).all()
                assert ww[i, :n].view(np.uint32).tolist() == \
                    exp_w.view(np.uint32).tolist()
                assert (ww[i, n:].view(np.uint32) == 0).all()
    for r in range(w.W):
        cnt = np.array([p["send_cnt"][r] for p in packs], np.int32)
        eloc = np.stack([p["send_eloc"][r] for p in packs])
        b = oracle.expert_batch(cnt, eloc, w.W, el, w.K, w.cap)
        assert b["err"] == 0
        # I8: rows = valid received picks = routed entries aimed at r
        n_pick = sum(int(((i >= 0) & (i // el == r)).sum()) for i, _ in srcs)
        assert int(b["expert_num_tokens"].sum()) == n_pick
        # rows of each expert are 0..n-1 exactly once
        rr = b["recv_row"]
        for e in range(el):
            valid = np.zeros(rr.shape, bool)
            for s in range(w.W):
                valid[s, :cnt[s]] = eloc[s, :cnt[s]] == e
            got = np.sort(rr[valid])
            assert np.array_equal(got, np.arange(b["expert_num_tokens"][e]))


# --------------------------------------------------------------------------
# Combine: closed forms on scaled workloads
# --------------------------------------------------------------------------

def _scaled(wid):
    base = wl.WORKLOADS[wid]
    if wid == 1:
        return base
    return base.scaled(T=97, cap=97, H=128)


def _run_identity(w, scale_fn=None):
    srcs = [wl.routing(w, s) for s in range(w.W)]
    pls = [wl.payloads(w, s, ids=i, wts=x) for s, (i, x) in enumerate(srcs)]

    def yfn(r, b):
        Y = b["b"][0].view(np.uint16).reshape(w.e_local, -1, w.H)
        if scale_fn is None:
            return Y.copy()
        f = wl.bf16_bits_to_f32(Y)
        for e in range(w.e_local):
            f[e] *= np.float32(scale_fn(r * w.e_local + e))
        return wl.f32_to_bf16_bits(f)

    return srcs, pls, oracle.run_path([s[0] for s in srcs], [s[1] for s in srcs],
                                      pls, w.E, w.W, w.cap, yfn)


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_identity_round_trip_returns_a1(wid):
    """I12: Y := b_a1 and softmax weights (sum 1 in fp32) return a1. Error
    bound: each partial rounds once to bf16 and the sum once more, so
    |out - a1*sum(w)| <= 2^-8 (sum_d |p_d| + |out|) + fp32 slack."""
    w = _scaled(wid)
    srcs, pls, res = _run_identity(w)
    for s in range(w.W):
        ids, wts = srcs[s]
        a1 = wl.bf16_bits_to_f32(pls[s][0].view(np.uint16))
        out = wl.bf16_bits_to_f32(res["outs"][s])
        wsum = np.where(ids >= 0, wts, 0).sum(axis=1, dtype=np.float64)
        exp = a1 * wsum[:, None]
        bound = 2.0 ** -8 * (np.abs(a1) * wsum[:, None] + np.abs(out)) * 1.001 \
            + 1e-6 * np.abs(a1)
        assert (np.abs(out - exp) <= bound).all()
        routed = (ids >= 0).any(axis=1)
        # round trip within 1 bf16 ulp of a1 itself
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(a1), 1e-30))) - 7)
        assert (np.abs(out[routed] - a1[routed]) <= ulp[routed] * 1.0001).all()
        # I14: padding rows are +0.0 bit for bit
        assert (res["outs"][s][~routed] == 0).all()


@pytest.mark.parametrize("W", [1, 2, 4])
def test_single_destination_tokens_are_exact(W):
    """I13: a token whose experts all live on one rank gets exactly
    RNE(sum_k fl(w_k * a1)) in router order (one rounding, no partials)."""
    w = wl.WORKLOADS[1].scaled(W=W, E=4 * W, K=3, T=80, cap=80)
    srcs, pls, res = _run_identity(w)
    n_checked = 0
    for s in range(w.W):
        ids, wts = srcs[s]
        a1 = wl.bf16_bits_to_f32(pls[s][0].view(np.uint16))
        for t in range(w.T):
            d = {int(e) // w.e_local for e in ids[t] if e >= 0}
            if len(d) != 1:
                continue
            acc = np.zeros(w.H, np.float32)
            for k in range(w.K):
                if ids[t, k] >= 0:
                    acc = (acc + (a1[t] * wts[t, k]).astype(np.float32)).astype(np.float32)
            assert np.array_equal(res["outs"][s][t], wl.f32_to_bf16_bits(acc))
            n_checked += 1
    assert n_checked > 0


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_power_of_two_experts(wid):
    """I15: experts that scale by 2^m_e (exact in bf16) make the output a
    layout-free closed form: out ~ sum_k w_k 2^m_(e_k) a1, within the
    partial/final rounding bound. A wrong row or expert mapping breaks it."""
    w = _scaled(wid)
    m = lambda e: 2.0 ** ((e * 7) % 5 - 2)
    srcs, pls, res = _run_identity(w, m)
    for s in range(w.W):
        ids, wts = srcs[s]
        a1 = wl.bf16_bits_to_f32(pls[s][0].view(np.uint16)).astype(np.float64)
        out = wl.bf16_bits_to_f32(res["outs"][s]).astype(np.float64)
        coef = np.zeros(w.T)
        absp = np.zeros(w.T)
        for t in range(w.T):
            for k in range(w.K):
                if ids[t, k] >= 0:
                    coef[t] += wts[t, k] * m(int(ids[t, k]))
                    absp[t] += wts[t, k] * m(int(ids[t, k]))
        exp = coef[:, None] * a1
        bound = 2.0 ** -8 * (absp[:, None] * np.abs(a1) + np.abs(out)) * 1.001 \
            + 1e-6 * np.abs(a1) + 1e-30
        assert (np.abs(out - exp) <= bound).all()


def test_fp32_path_round_trip():
    w = _scaled(2)
    srcs = [wl.routing(w, s) for s in range(w.W)]
    a1 = [wl.hidden_f32(w, s) for s in range(w.W)]
    pls = [[a.view(np.uint8).reshape(w.T, -1)] for a in a1]

    def yfn(r, b):
        return b["b"][0].view(np.float32).reshape(w.e_local, -1, w.H).copy()

    res = oracle.run_path([s[0] for s in srcs], [s[1] for s in srcs], pls,
                          w.E, w.W, w.cap, yfn)
    for s in range(w.W):
        ids, wts = srcs[s]
        wsum = np.where(ids >= 0, wts, 0).sum(axis=1, dtype=np.float64)
        exp = a1[s] * wsum[:, None]
        assert np.allclose(res["outs"][s], exp, rtol=1e-6, atol=0)


# --------------------------------------------------------------------------
# Data errors and their defined behaviour
# --------------------------------------------------------------------------

def test_error_bits():
    # id >= E dropped (bit 0); duplicates beyond slots dropped (bit 1)
    ids = np.array([[0, 9], [1, 1]], np.int32)          # E=4, W=4 -> slots 1
    wts = np.ones((2, 2), np.float32)
    r = oracle.dispatch_pack(ids, wts, 4, 4, 2)
    assert r["err"] == oracle.ERR_ID_RANGE | oracle.ERR_PICKS
    assert r["send_cnt"].tolist() == [1, 1, 0, 0]
    # received local id >= e_local dropped (bit 2); count > cap clamped (bit 4)
    cnt = np.array([3, 1], np.int32)
    eloc = np.array([[[0], [5]], [[1], [0]]], np.int32)
    b = oracle.expert_batch(cnt, eloc, 2, 2, 1, 2)
    assert b["err"] == oracle.ERR_ELOC | oracle.ERR_CNT
    assert b["recv_row"][0, :, 0].tolist() == [0, -1]
    assert b["expert_num_tokens"].tolist() == [1, 1]
    # rows past expert_cap (only duplicate ids can get there) dropped (bit 3),
    # and expert_num_tokens clamped to expert_cap: W = 1, e_local = 2, K = 2
    # (slots 2), cap 2, so expert_cap = 2; both slots hold local expert 0
    # twice, which asks for rows 0, 1, 2, 3 of it
    cnt = np.array([2], np.int32)
    eloc = np.array([[[0, 0], [0, 0]]], np.int32)
    b = oracle.expert_batch(cnt, eloc, 1, 2, 2, 2)
    assert b["err"] == oracle.ERR_ROWCAP
    assert b["recv_row"][0].tolist() == [[0, 1], [-1, -1]]
    assert b["expert_num_tokens"].tolist() == [2, 0]


# --------------------------------------------------------------------------
# Generators
# --------------------------------------------------------------------------

def test_generators_are_deterministic_and_shaped():
    import hashlib
    w = wl.WORKLOADS[5].scaled(T=64)
    a = wl.routing(w, 3)
    b = wl.routing(w, 3)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    ids, wts = a
    assert ids.dtype == np.int32 and wts.dtype == np.float32
    assert ((ids >= 0).all(axis=1) | (ids < 0).all(axis=1)).all()
    assert int((ids < 0).all(axis=1).sum()) == w.n_pad
    for t in range(w.T):
        if ids[t, 0] >= 0:
            assert len(set(ids[t].tolist())) == w.K
    pl = wl.payloads(w, 3, ids=ids, wts=wts)
    assert [p.shape[1] for p in pl] == [14336, 7168, 224, 32, 32]
    h1 = hashlib.sha256(pl[0].tobytes()).hexdigest()
    h2 = hashlib.sha256(wl.payloads(w, 3)[0].tobytes()).hexdigest()
    assert h1 == h2
    assert wl.WORKLOADS[3].n_pad == 245 and wl.WORKLOADS[5].n_pad == 819
    assert wl.WORKLOADS[4].n_pad == 12 and wl.WORKLOADS[1].n_pad == 3


# ---------------------------------------------------------------------------
# Send-side ranks (the rows of the receive side, counted by each source)
# ---------------------------------------------------------------------------

def test_golden_pick_ranks():
    G = _gold("worked_example.json")
    g, gp, gb = G["pick_ranks"], G["pack"], G["batch"]
    cnt = np.array(gp["send_cnt"], np.int32)
    eloc = np.full((gp["W"], gp["max_num_tokens"], gp["expect_slots"]), -1, np.int32)
    for d in range(gp["W"]):
        eloc[d, :cnt[d]] = gp["send_eloc"][d]
    r = oracle.pick_ranks(cnt, eloc, gp["E"] // gp["W"])
    for d in range(gp["W"]):
        assert r["send_rank"][d, :cnt[d]].tolist() == g["send_rank"][d]
    assert r["send_ecnt"].tolist() == g["send_ecnt"]
    # the batch example's sources: counts before + rank = the golden rows
    W, el, cap = gb["W"], gb["e_local"], gb["max_num_tokens"]
    bcnt = np.array(gb["recv_cnt"], np.int32)
    beloc = np.array(gb["recv_eloc"], np.int32)
    before = np.zeros(el, np.int64)
    for s in range(W):
        rs = oracle.pick_ranks(bcnt[s:s + 1], beloc[s:s + 1], el)
        c = int(bcnt[s])
        assert rs["send_rank"][0, :c].tolist() == g["batch_source_ranks"][s]
        assert rs["send_ecnt"][0].tolist() == g["batch_source_ecnt"][s]
        rows = [[int(before[e]) + int(k) if e >= 0 else -1
                 for e, k in zip(er, kr)]
                for er, kr in zip(beloc[s, :c].tolist(), rs["send_rank"][0, :c].tolist())]
        assert rows == gb["recv_row_valid"][s]
        before += rs["send_ecnt"][0]
    assert before.tolist() == gb["expert_num_tokens"]


def _ranks_by_pairs(ids, E, W):
    """rank of every kept pick by counting, over all (token, pick) pairs of
    the source, the earlier kept picks with the same expert id (token order,
    then router order); the kept picks come from the set formulation."""
    cnt, slot, picks, _ = brute.pack_sets(ids, np.zeros(ids.shape, np.float32), E, W)
    e_local = E // W
    flat = []                         # (token, column, d, global id)
    for (d, t), lst in picks.items():
        for j, (e, _) in enumerate(lst):
            flat.append((t, j, d, d * e_local + e))
    ranks = {}
    for (t, j, d, g) in flat:
        ranks[(d, t, j)] = sum(1 for (t2, j2, d2, g2) in flat
                               if g2 == g and (t2, j2) < (t, j))
    ecnt = np.zeros((W, e_local), np.int64)
    for (t, j, d, g) in flat:
        ecnt[d, g - d * e_local] += 1
    return cnt, slot, ranks, ecnt


def _check_ranks_against_pairs(ids, E, W):
    T, K = ids.shape
    p = oracle.dispatch_pack(ids, np.ones((T, K), np.float32), E, W, T)
    r = oracle.pick_ranks(p["send_cnt"], p["send_eloc"], E // W)
    cnt, slot, ranks, ecnt = _ranks_by_pairs(ids, E, W)
    assert r["send_ecnt"].tolist() == ecnt.tolist(), ids
    for (d, t), sl in slot.items():
        n = sum(1 for (d2, t2, _j) in ranks if (d2, t2) == (d, t))
        want = [ranks[(d, t, j)] for j in range(n)] + [-1] * (p["slots"] - n)
        assert r["send_rank"][d, sl].tolist() == want, (ids, d, t)


@pytest.mark.parametrize("W,K", [(1, 2), (2, 2), (4, 1)])
def test_pick_ranks_exhaustive_micro(W, K):
    """Every id tuple over T=3 tokens, E=4 (duplicates and padding included):
    the oracle's ranks, from the pack's outputs, equal counts over all
    pairs of the source's kept picks."""
    E, T = 4, 3
    vals = [-1, 0, 1, 2, 3]
    per_tok = list(itertools.product(vals, repeat=K))
    for combo in itertools.product(per_tok, repeat=T):
        _check_ranks_against_pairs(np.array(combo, np.int32).reshape(T, K), E, W)


def test_pick_ranks_random_micro():
    """Random sources with more picks per token, duplicates past the pick
    columns and ids out of range, against the same pair counts."""
    rng = np.random.default_rng(13)
    for _ in range(1500):
        W = int(rng.choice([1, 2, 3, 4]))
        el = int(rng.integers(1, 4))
        K = int(rng.integers(1, 6))
        T = int(rng.integers(0, 8))
        ids = rng.integers(-2, W * el + 2, size=(T, K)).astype(np.int32)
        _check_ranks_against_pairs(ids, W * el, W)


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_pick_ranks_give_the_receive_rows(wid):
    """On every workload (scaled): for each destination, the counts of the
    sources before s plus the rank equal the receive-side rows of the
    oracle's batch (taken in (source, slot, pick) order), and the summed
    counts equal expert_num_tokens."""
    w = wl.WORKLOADS[wid]
    if w.T > 300:
        w = w.scaled(T=300, cap=300)
    packs, ranks = [], []
    for s in range(w.W):
        ids, wts = wl.routing(w, s, 4)
        packs.append(oracle.dispatch_pack(ids, wts, w.E, w.W, w.cap))
        ranks.append(oracle.pick_ranks(packs[-1]["send_cnt"], packs[-1]["send_eloc"],
                                       w.e_local))
    for r in range(w.W):
        cnt = np.ascontiguousarray(np.stack([p["send_cnt"][r] for p in packs]))
        eloc = np.ascontiguousarray(np.stack([p["send_eloc"][r] for p in packs]))
        b = oracle.expert_batch(cnt, eloc, w.W, w.e_local, w.K, w.cap)
        before = np.zeros(w.e_local, np.int64)
        for s in range(w.W):
            c = int(cnt[s])
            e = eloc[s, :c]
            k = ranks[s]["send_rank"][r, :c]
            rows = np.where(e >= 0, before[np.maximum(e, 0)] + k, -1)
            assert np.array_equal(rows, b["recv_row"][s, :c]), (r, s)
            before += ranks[s]["send_ecnt"][r]
        assert np.array_equal(before, b["expert_num_tokens"])
