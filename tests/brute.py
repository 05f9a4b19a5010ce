"""Independent set- and dictionary-based formulations of the layout transform,
used to pin the oracle by brute force on tiny inputs.

They are written differently from the oracle on purpose: the oracle walks
destinations and tokens with running counters; these build explicit sets,
sort them, and look positions up. Only the statement of the method is shared
(vLLM "alltoall_batched" documentation page, AllToAllBatchedPrepareAndFinalize
prepare() / finalize()), not any code.
"""
from __future__ import annotations

import struct
from typing import Dict, List, Tuple

import numpy as np


def f32(x) -> np.float32:
    return np.float32(x)


def bf16_to_f32(bits: int) -> np.float32:
    return np.frombuffer(struct.pack("<I", (int(bits) & 0xFFFF) << 16),
                         dtype=np.float32)[0]


def f32_bits(x: np.float32) -> int:
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def bf16_rne_from_fraction(x: np.float32) -> int:
    """bf16 rounding by exact rational arithmetic on the value (not on bits):
    pick the nearer of the two bf16 neighbours; on a tie the one with an even
    last significand bit. Used only for finite values."""
    from fractions import Fraction
    v = Fraction(float(x))
    if v == 0:
        return 0x8000 if f32_bits(x) >> 31 else 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    # a in [1,2): significand with 7 fraction bits
    scaled = a * 128
    lo = int(scaled)
    frac = scaled - lo
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    if lo == 256:
        lo = 128
        e += 1
    biased = e + 127
    if biased >= 255:
        return sign | 0x7F80
    if biased <= 0:
        raise ValueError("subnormal bf16 not needed here")
    return sign | (biased << 7) | (lo - 128)


def pack_sets(ids: np.ndarray, wts: np.ndarray, E: int, W: int
              ) -> Tuple[List[int], Dict[Tuple[int, int], int],
                         Dict[Tuple[int, int], List[Tuple[int, float]]], int]:
    """Set-based send side of one source.

    Returns (cnt[d], slot[(d,t)], picks[(d,t)] = [(local id, weight)] in
    router order truncated to the expert slots per token, error bits).
    """
    T, K = ids.shape
    e_local = E // W
    slots = min(K, e_local)
    err = 0
    dests_of = {}
    for t in range(T):
        ds = set()
        for k in range(K):
            i = int(ids[t, k])
            if i >= E:
                err |= 1
            elif i >= 0:
                ds.add(i // e_local)
        dests_of[t] = ds
    cnt, slot, picks = [], {}, {}
    for d in range(W):
        members = sorted(t for t in range(T) if d in dests_of[t])
        cnt.append(len(members))
        for pos, t in enumerate(members):
            slot[(d, t)] = pos
            lst = [(int(ids[t, k]) - d * e_local, float(wts[t, k]))
                   for k in range(K)
                   if 0 <= int(ids[t, k]) < E and int(ids[t, k]) // e_local == d]
            if len(lst) > slots:
                err |= 2
            picks[(d, t)] = lst[:slots]
    return cnt, slot, picks, err


def batch_sorted(recv: List[Tuple[int, List[List[int]]]], e_local: int,
                 expert_cap: int = 1 << 62
                 ) -> Tuple[Dict[Tuple[int, int, int], int], List[int]]:
    """recv[s] = (count, eloc rows [count][slots]). Rows by sorting the valid
    entries lexicographically and numbering each expert's group; numbers at
    or past expert_cap are not kept, and the counts are clamped to it."""
    entries = []
    for s, (c, rows) in enumerate(recv):
        for slot in range(c):
            for j, e in enumerate(rows[slot]):
                if 0 <= e < e_local:
                    entries.append((s, slot, j, e))
    entries.sort()
    row = {}
    per_e = [[x for x in entries if x[3] == e] for e in range(e_local)]
    for e in range(e_local):
        for r, (s, slot, j, _) in enumerate(per_e[e]):
            if r < expert_cap:
                row[(s, slot, j)] = r
    return row, [min(len(g), expert_cap) for g in per_e]
