"""GPU parity: the HIP path (through the C ABI) against the CPU oracle,
element by element, on seeded inputs at sizes the oracle finishes in
seconds. Sizes span several routing tiles (256 tokens), several receive-scan
tiles (1024 picks), ragged vector tails and the degenerate cases."""
import numpy as np
import pytest
import torch

import workloads as wl
from parity import run_full_parity, say

pytestmark = pytest.mark.gpu

W1, W2, W3, W4, W5 = (wl.WORKLOADS[i] for i in range(1, 6))

CASES = {
    # the tiny workload at its real size
    "tiny": W1,
    # DeepSeek-V3 shape, fewer tokens; ragged vs the 256-token tile, rows of
    # 129 vectors (ragged vs 256 lanes), cap > T
    "dsv3_small": W2.scaled(T=300, cap=320, H=1032),
    # Mixtral shape: e_local = 1, Zipf 1.1, 3 % padding, several scan tiles
    "mixtral_small": W3.scaled(T=700, cap=700, H=512),
    # decode at its real size: W = 32, T = 128, H = 7168
    "decode": W4,
    # five payloads (bf16, fp8, scales, ids, weights), Zipf 1.2, 10 % padding
    "multi_small": W5.scaled(T=300, cap=300, H=1024),
    # one rank: pack is a compaction, batch a counting sort
    "w1": W1.scaled(W=1, E=8, K=2, T=200, cap=200, H=64),
    # the largest world, 2 experts per rank, slots = e_local < K
    "w64": W1.scaled(W=64, E=128, K=4, T=90, cap=96, H=128),
    # many local experts (e_local = 512): 9-bit multi-split
    "e_local_512": W1.scaled(W=2, E=1024, K=8, T=260, cap=260, H=64),
    # top-1
    "k1": W1.scaled(W=4, E=16, K=1, T=129, cap=129, H=32),
    # every row padding
    "all_padding": W1.scaled(T=40, cap=40, pad_frac=1.0),
    # no tokens at all
    "empty": W1.scaled(T=0, cap=16),
    # the limits: 64 pick columns per slot (K = e_local = 64) ...
    "max_slots": W1.scaled(W=2, E=128, K=64, T=50, cap=50, H=64),
    # ... 1024 local experts on one rank ...
    "max_e_local": W1.scaled(W=1, E=1024, K=8, T=300, cap=300, H=64),
    # ... and a wide row (32 KiB of bf16) through every pass of every kernel
    "wide_row": W1.scaled(W=4, E=16, K=4, T=40, cap=48, H=16384),
    # enough tokens that the unpack covers whole rows in one block: rows of
    # 288 vectors in bf16, 576 in fp32 (above the 512 that switch the
    # combine kernels to 4 vectors per lane)
    "whole_row_unpack": W1.scaled(W=4, E=16, K=4, T=2100, cap=2100, H=2304),
    # more than 64 routing tiles of 256 tokens (67): the send side takes the
    # column scan for send_cnt and the tile offsets it writes
    "many_route_tiles": W1.scaled(W=4, E=16, K=4, T=17000, cap=17000, H=128),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_parity(name):
    w = CASES[name]
    say(f"[parity] {name}: T={w.T} H={w.H} E={w.E} K={w.K} W={w.W} cap={w.cap}")
    run_full_parity(w, salt=3)


# the per-expert ranks need K <= 16 and E <= 4096 (every case but max_slots)
RANKED_CASES = sorted(n for n, w in CASES.items() if w.K <= 16 and w.E <= 4096)


@pytest.mark.parametrize("name", RANKED_CASES)
def test_parity_ranked(name):
    """Packs with the per-expert ranks (moe_ep_dispatch_pack's send_rank and
    send_ecnt, against the oracle's) and the receive side from them
    (moe_ep_expert_batch_ranked): every output as in test_parity."""
    w = CASES[name]
    say(f"[parity ranked] {name}: T={w.T} H={w.H} E={w.E} K={w.K} W={w.W} cap={w.cap}")
    run_full_parity(w, salt=3, ranked=True)


def test_parity_ranked_bad_ids_duplicates_and_corrupt_count():
    """Dropped ids, duplicates past the pick columns and a corrupted
    received count, through the ranked pack and batch: bit-exact with the
    oracle, flags included."""
    w = W1.scaled(W=4, E=8, K=3, T=300, cap=300, H=64, pad_frac=0.0)
    srcs, pls = [], []
    for s in range(w.W):
        ids, wts = wl.routing(w, s, 7)
        ids = ids.copy()
        ids[3, 1] = 8 + s            # out of range
        ids[5] = [2, 2, 2]           # duplicates: e_local 2 -> slots 2
        ids[260] = [3, 3, 1]         # in the second routing tile
        ids[9, 0] = -5               # any negative id is padding
        srcs.append((ids, wts))
        pls.append(wl.payloads(w, s, 7))
    say("[parity ranked] bad ids")
    run_full_parity(w, srcs=srcs, pls=pls, ranked=True)
    say("[parity ranked] corrupt count")
    run_full_parity(W1.scaled(W=4, E=8, K=2, T=50, cap=50, H=64), salt=9,
                    corrupt_cnt=(1, 2, 77), ranked=True)
    # one tile of tokens (the pack ranks by itself) with duplicates
    w = W1.scaled(W=4, E=8, K=3, T=70, cap=70, H=64, pad_frac=0.0)
    srcs, pls = [], []
    for s in range(w.W):
        ids, wts = wl.routing(w, s, 8)
        ids = ids.copy()
        ids[1] = [5, 5, 4]
        ids[40] = [1, 0, 1]
        srcs.append((ids, wts))
        pls.append(wl.payloads(w, s, 8))
    say("[parity ranked] duplicates, one tile")
    run_full_parity(w, srcs=srcs, pls=pls, ranked=True)


@pytest.mark.parametrize("T", [100, 300])
def test_parity_ranked_many_experts(T):
    """More experts than the token masks of the fast form cover (E = 2048):
    the ranks come from the general forms (counts in the pack for one tile,
    the multi-split in the routing kernel)."""
    w = W1.scaled(W=4, E=2048, K=8, T=T, cap=T, H=64)
    say(f"[parity ranked] E={w.E} T={T}")
    run_full_parity(w, salt=19, ranked=True)


@pytest.mark.parametrize("ranked", [False, True])
@pytest.mark.parametrize("H", [4104, 7000, 8192, 8200, 12000])
def test_parity_rows_around_the_early_pass(H, ranked):
    """Rows of one payload just above 8 KiB (513 vectors, where the batch
    copy starts loading a row's first pass before planning), a ragged 875,
    exactly the 1,024 vectors of that pass, one vector past it, and 1,500:
    with the receiver's scan (guarded loads) and with the senders' ranks
    (buffer loads whose range check stops at the row's end)."""
    w = W1.scaled(W=4, E=16, K=4, T=300, cap=300, H=H)
    say(f"[parity rows] H={H} ranked={ranked}")
    run_full_parity(w, salt=41, ranked=ranked)


@pytest.mark.parametrize("T", [200, 300])
def test_parity_ranked_at_the_form_limits(T):
    """K = 16 picks and E = 4096 experts, the largest the ranked form takes
    (1,024 local experts on each of 4 ranks): the largest LDS tables of the
    routing kernel's general ranks, the pack's own counts and the ranked
    batch copy's count table."""
    w = W1.scaled(W=4, E=4096, K=16, T=T, cap=T, H=64)
    say(f"[parity ranked] limits K=16 E=4096 T={T}")
    run_full_parity(w, salt=37, ranked=True)


@pytest.mark.parametrize("K,E,W,T", [(12, 32, 8, 600), (16, 64, 4, 600), (16, 64, 4, 200),
                                     (9, 16, 8, 300)])
def test_parity_ranked_wide_topk(K, E, W, T):
    """More than 8 picks per token (up to the form's limit of 16), over
    several routing tiles and within one: the code unrolled to 16 picks.
    With e_local < K a token keeps at most e_local picks per rank."""
    w = W1.scaled(W=W, E=E, K=K, T=T, cap=T, H=64)
    say(f"[parity ranked] K={K} E={E} W={W} T={T}")
    run_full_parity(w, salt=31, ranked=True)


@pytest.mark.parametrize("name", ["dsv3_small", "decode", "many_route_tiles"])
@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_parity_ranked_quantised(name, fmt):
    w = CASES[name]
    say(f"[parity ranked {fmt}] {name}")
    if fmt == "fp8":
        run_full_parity(w.scaled(H=1024) if w.H % 128 else w, salt=21, fp8_group=128,
                        ranked=True)
    else:
        run_full_parity(w.scaled(H=1024) if w.H % 32 else w, salt=37, fp4=True, ranked=True)


@pytest.mark.parametrize("name", ["dsv3_small", "decode", "w64"])
def test_parity_ranked_fused_local(name):
    say(f"[parity ranked fused local] {name}")
    run_full_parity(CASES[name], salt=23, fused_local=True, ranked=True)


@pytest.mark.parametrize("name", ["tiny", "dsv3_small", "mixtral_small", "wide_row",
                                  "whole_row_unpack"])
def test_parity_fp32_combine(name):
    w = CASES[name]
    say(f"[parity fp32] {name}")
    run_full_parity(w, salt=5, f32=True)


@pytest.mark.parametrize("name", ["tiny", "decode", "multi_small"])
def test_parity_batch_plan_then_copy(name):
    """moe_ep_expert_batch_plan + moe_ep_expert_batch_copy == the one call."""
    say(f"[parity split batch] {name}")
    run_full_parity(CASES[name], salt=17, split_batch=True)


def test_parity_second_seed():
    say("[parity] dsv3_small seed 2")
    run_full_parity(CASES["dsv3_small"], salt=11)


def test_bad_ids_and_duplicates_follow_defined_behaviour():
    """ids >= E are dropped (bit 0), duplicate ids past the slots are dropped
    (bit 1), both exactly as the oracle does."""
    w = W1.scaled(W=4, E=8, K=3, T=70, cap=70, H=64, pad_frac=0.0)
    srcs, pls = [], []
    for s in range(w.W):
        ids, wts = wl.routing(w, s, 7)
        ids = ids.copy()
        ids[3, 1] = 8 + s            # out of range
        ids[5] = [2, 2, 2]           # duplicates: e_local 2 -> slots 2
        ids[9, 0] = -5               # any negative id is padding
        srcs.append((ids, wts))
        pls.append(wl.payloads(w, s, 7))
    say("[parity] bad ids")
    run_full_parity(w, srcs=srcs, pls=pls)


def test_received_count_out_of_range_is_clamped():
    w = W1.scaled(W=4, E=8, K=2, T=50, cap=50, H=64)
    say("[parity] corrupt count")
    run_full_parity(w, salt=9, corrupt_cnt=(1, 2, 77))


def test_runs_are_bit_identical():
    """Same inputs twice: every output byte equal (no order dependence)."""
    w = CASES["mixtral_small"]
    say("[determinism] mixtral_small x2")
    ep1, _ = run_full_parity(w, salt=13)
    outs1 = [ep1.out.clone(), ep1.ret.clone(), ep1.recv_row.clone(),
             ep1.token_slot.clone()]
    del ep1
    ep2, _ = run_full_parity(w, salt=13)
    outs2 = [ep2.out, ep2.ret, ep2.recv_row, ep2.token_slot]
    for a, b in zip(outs1, outs2):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


FP8_CASES = {
    "tiny": W1,
    "dsv3_small": W2.scaled(T=300, cap=320, H=1024),
    "multi_small": W5.scaled(T=300, cap=300, H=1024),
    "decode": W4,
    "w64": W1.scaled(W=64, E=128, K=4, T=90, cap=96, H=128),
    "empty": W1.scaled(T=0, cap=16),
    "many_route_tiles": CASES["many_route_tiles"],
}


@pytest.mark.parametrize("name", sorted(FP8_CASES))
@pytest.mark.parametrize("group", [128, 32])
def test_parity_fp8_pack(name, group):
    """Quantize-on-pack: codes, scales and every other output bit-exact."""
    w = FP8_CASES[name]
    say(f"[parity fp8] {name} group {group}")
    run_full_parity(w, salt=21, fp8_group=group)


def test_fp8_conversion_sweep_all_bf16_in_range():
    """Every bf16 value in [-448, 448] through the quantiser with scale 1
    (each 128-column group holds a +-448), codes bit-exact with the oracle:
    checks the hardware conversion's rounding on every input value,
    including all ties between neighbouring codes."""
    pos = np.arange(0x0000, 0x43E1, dtype=np.uint32)           # 0 .. 448
    vals = np.concatenate([pos, pos | 0x8000]).astype(np.uint16)
    H, group = 1024, 128
    per_group = group - 1
    n_groups = -(-len(vals) // per_group)
    T = -(-n_groups // (H // group))
    rows = np.zeros((T * (H // group), group), np.uint16)
    rows[:, 0] = 0x43E0                                          # 448
    flat = rows[:, 1:].reshape(-1)
    flat[:len(vals)] = vals
    rows[:, 1:] = flat.reshape(-1, per_group)
    rows[1::2, 0] = 0xC3E0                                       # -448 on odd groups
    hidden = rows.reshape(T, H)
    w = W1.scaled(W=1, E=2, K=1, T=T, cap=T, H=H, pad_frac=0.0)
    ids = np.zeros((T, 1), np.int32)
    wts = np.ones((T, 1), np.float32)
    say(f"[fp8 sweep] {len(vals)} values in {T} rows")
    run_full_parity(w, srcs=[(ids, wts)],
                    pls=[[hidden.view(np.uint8).reshape(T, 2 * H)]], fp8_group=group)


FUSED_CASES = ["tiny", "dsv3_small", "mixtral_small", "decode", "w64", "k1",
               "all_padding", "empty", "e_local_512"]


@pytest.mark.parametrize("name", FUSED_CASES)
def test_parity_fused_local_combine(name):
    """moe_ep_combine_reduce_peers + moe_ep_combine_unpack_fused: every
    output against the oracle's reduce + unpack; the own block of ret is
    never written."""
    say(f"[parity fused local] {name}")
    run_full_parity(CASES[name], salt=23, fused_local=True)


@pytest.mark.parametrize("name,f32", [("dsv3_small", False), ("mixtral_small", False),
                                      ("tiny", True), ("wide_row", True),
                                      ("whole_row_unpack", True)])
def test_fused_local_combine_is_bit_identical_to_unfused(name, f32):
    say(f"[fused == unfused] {name} f32={f32}")
    ep1, _ = run_full_parity(CASES[name], salt=29, f32=f32)
    out1 = ep1.out.clone()
    del ep1
    ep2, _ = run_full_parity(CASES[name], salt=29, f32=f32, fused_local=True)
    assert torch.equal(out1.view(torch.uint8), ep2.out.view(torch.uint8))


FP4_CASES = dict(FP8_CASES, ragged_scales=W1.scaled(T=70, cap=70, H=544))


@pytest.mark.parametrize("name", sorted(FP4_CASES))
def test_parity_fp4_pack(name):
    """4-bit quantize-on-pack: codes, scale codes (with their 0x00 padding)
    and every other output bit-exact."""
    w = FP4_CASES[name]
    say(f"[parity fp4] {name}")
    run_full_parity(w, salt=37, fp4=True)


def test_fp4_every_bf16_bit_pattern():
    """All 65,536 bf16 bit patterns (zeros, subnormals, normals, infinities,
    NaNs) in 16-column blocks through the 4-bit quantiser: the scales cover
    underflow to 0x00, every normal range and saturation at 448; the codes
    cover every midpoint. Bit-exact with the oracle."""
    rng = np.random.default_rng(41)
    vals = rng.permutation(np.arange(0x10000, dtype=np.uint32)).astype(np.uint16)
    H = 1024
    T = len(vals) // H
    hidden = vals.reshape(T, H)
    w = W1.scaled(W=1, E=2, K=1, T=T, cap=T, H=H, pad_frac=0.0)
    ids = np.zeros((T, 1), np.int32)
    wts = np.ones((T, 1), np.float32)
    say(f"[fp4 sweep] all bf16 patterns in {T} rows")
    try:
        run_full_parity(w, srcs=[(ids, wts)],
                        pls=[[hidden.view(np.uint8).reshape(T, 2 * H)]], fp4=True)
    except AssertionError as e:
        # name the inputs of the first differing code byte (row, byte)
        import re
        m = re.search(r"\((\d+), (\d+)\)", str(e))
        if m:
            t, b = int(m.group(1)), int(m.group(2))
            blk = hidden[t, (2 * b) // 16 * 16:(2 * b) // 16 * 16 + 16]
            say(f"[fp4 sweep] row {t} byte {b}: columns {2 * b}, {2 * b + 1} = "
                f"{hidden[t, 2 * b]:#06x}, {hidden[t, 2 * b + 1]:#06x}; block "
                + " ".join(f"{v:04x}" for v in blk))
        raise


def _e4m3_positive_values():
    vals = []
    for c in range(0x7F):
        e, f = c >> 3, c & 7
        vals.append((f / 8) * 2.0 ** -6 if e == 0 else (1 + f / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def _bf16_nearest(v: np.ndarray) -> np.ndarray:
    return wl.f32_to_bf16_bits(np.asarray(v, np.float32))


def test_fp8_quotients_near_midpoints():
    """Groups whose scale is not a power of two and whose entries make x / s
    land on or next to every E4M3 midpoint: for each amax (every bf16
    significand in [1, 2) at three exponents) the group holds amax and, per
    midpoint m between neighbouring codes, the bf16 value nearest to
    m * amax / 448. Here x / s and x * (448 / amax) often round to different
    codes; the kernel's codes must be the oracle's (fp32 quotient, then
    nearest even)."""
    vals = _e4m3_positive_values()
    mids = (vals[:-1] + vals[1:]) / 2                     # 126 midpoints
    group, groups = 128, []
    for ex in (-3, 0, 5):
        for m7 in range(128):
            amax = (1 + m7 / 128) * 2.0 ** ex
            g = np.zeros(group, np.uint16)
            g[0] = _bf16_nearest(np.array([amax]))[0]
            x = _bf16_nearest(mids * amax / 448.0)
            g[1:1 + len(x)] = x
            g[1 + len(x)] = x[len(x) // 2] | 0x8000          # one negative
            groups.append(g)
    H = 1024
    rows = np.stack(groups).reshape(-1, H)
    T = rows.shape[0]
    w = W1.scaled(W=1, E=2, K=1, T=T, cap=T, H=H, pad_frac=0.0)
    ids = np.zeros((T, 1), np.int32)
    wts = np.ones((T, 1), np.float32)
    say(f"[fp8 midpoints] {len(groups)} groups in {T} rows")
    run_full_parity(w, srcs=[(ids, wts)],
                    pls=[[rows.view(np.uint8).reshape(T, 2 * H)]], fp8_group=group)


def test_fp4_quotients_at_midpoints():
    """Blocks of 16 whose scale s = value(e4m3(amax / 6)) runs over every
    E4M3 code reachable from a bf16 amax = 6 s, holding amax and, per E2M1
    midpoint m (0.25 .. 5) and sign, the bf16 value nearest to m * s (exactly
    m * s where that is a bf16 value: a tie that x * fp32(1 / s) would break
    the wrong way where 1 / s is inexact). Codes bit-exact with the oracle."""
    vals = _e4m3_positive_values()
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    blocks = []
    for s in vals[1:]:
        b = np.zeros(16, np.uint16)
        b[0] = _bf16_nearest(np.array([6.0 * s]))[0]
        x = _bf16_nearest(mids * s)
        b[1:8] = x
        b[8:15] = x | 0x8000
        blocks.append(b)
    H = 512
    n = -(-len(blocks) // (H // 16)) * (H // 16)
    blocks += [np.zeros(16, np.uint16)] * (n - len(blocks))
    rows = np.stack(blocks).reshape(-1, H)
    T = rows.shape[0]
    w = W1.scaled(W=1, E=2, K=1, T=T, cap=T, H=H, pad_frac=0.0)
    ids = np.zeros((T, 1), np.int32)
    wts = np.ones((T, 1), np.float32)
    say(f"[fp4 midpoints] {len(vals) - 1} scales in {T} rows")
    run_full_parity(w, srcs=[(ids, wts)],
                    pls=[[rows.view(np.uint8).reshape(T, 2 * H)]], fp4=True)


def test_fp8_every_bf16_bit_pattern():
    """All 65,536 bf16 bit patterns through the fp8 quantiser (groups of
    128): NaN entries never set a group's amax; groups with an infinite
    amax get scale inf (finite entries give zero codes, infinite ones the
    NaN code); codes carry their input's sign. Codes and scales bit-exact
    with the oracle."""
    rng = np.random.default_rng(43)
    vals = rng.permutation(np.arange(0x10000, dtype=np.uint32)).astype(np.uint16)
    H = 1024
    T = len(vals) // H
    hidden = vals.reshape(T, H)
    w = W1.scaled(W=1, E=2, K=1, T=T, cap=T, H=H, pad_frac=0.0)
    ids = np.zeros((T, 1), np.int32)
    wts = np.ones((T, 1), np.float32)
    say(f"[fp8 sweep] all bf16 patterns in {T} rows")
    run_full_parity(w, srcs=[(ids, wts)],
                    pls=[[hidden.view(np.uint8).reshape(T, 2 * H)]], fp8_group=128)


def _batch_outputs(w, split: bool):
    """Per destination: expert_num_tokens, recv_row and the valid expert rows
    of a step's batch half, through the one call or through plan + copy."""
    from combine_topk_ids_dest_amd.emulate import LogicalEP
    srcs = [wl.routing(w, s, 23) for s in range(w.W)]
    pls = [wl.payloads(w, s, 23, ids=srcs[s][0], wts=srcs[s][1]) for s in range(w.W)]
    ep = LogicalEP(w.T, w.H, w.E, w.K, w.W, w.cap, [p.shape[1] for p in pls[0]],
                   torch.bfloat16, "cuda", fill=0xFF)
    for s in range(w.W):
        ep.set_source(s, srcs[s][0], srcs[s][1], pls[s])
        ep.pack(s)
    out = []
    for r in range(w.W):
        if split:
            ep.batch_plan(r)
            ep.batch_copy(r)
        else:
            ep.batch(r)
        ent = ep.expert_num_tokens[r].clone()
        rows = [torch.cat([b[e, :int(ent[e])] for e in range(ep.e_local)]).clone()
                for b in ep.b]
        out.append((ent, ep.recv_row[r].clone(), rows))
    torch.cuda.synchronize()
    assert int(ep.err.item()) == 0
    return out, ep.slots


@pytest.mark.parametrize("cap,tiles", [(64, 2), (2048, 64), (2080, 65)])
def test_combined_batch_is_bit_identical_to_plan_then_copy(cap, tiles):
    """moe_ep_expert_batch skips the column scan for at most 64 pick tiles
    (the copy sums the tile offsets itself); plan + copy always runs it.
    At 2, exactly 64 and 65 tiles both give the same bytes."""
    w = W1.scaled(W=8, E=32, K=4, T=cap, cap=cap, H=64, pad_frac=0.05)
    one, slots = _batch_outputs(w, split=False)
    two, _ = _batch_outputs(w, split=True)
    assert -(-w.W * w.cap * slots // 1024) == tiles
    say(f"[batch one call vs plan + copy] cap={cap}: {tiles} pick tiles")
    for r, ((e1, r1, b1), (e2, r2, b2)) in enumerate(zip(one, two)):
        assert torch.equal(e1, e2), f"expert_num_tokens of destination {r}"
        assert torch.equal(r1, r2), f"recv_row of destination {r}"
        for p, (x, y) in enumerate(zip(b1, b2)):
            assert torch.equal(x, y), f"expert rows of destination {r}, payload {p}"
