"""Pins of the oracle's 4-bit quantize-on-pack (CPU): OCP E2M1 codes with
E4M3 scales per 16 columns.

Independent references: the OCP E2M1 magnitudes written out here; exact
rational nearest-even rounding (fractions.Fraction) on every midpoint, its
neighbours and random values; torch's float8_e4m3fn conversion (a library
routine) for the scale codes and their values; and hand-derived rows
(tests/golden/fp4_quant.json).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from test_oracle_fp8 import e4m3_nearest_even, e4m3_value, rn_f32

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def e2m1_value(code: int) -> float:
    return (-1.0 if code & 8 else 1.0) * MAGS[code & 7]


def e2m1_exact(x: float) -> int:
    """Nearest E2M1 code by exact rational distance; ties to the even code;
    above 6 the largest magnitude."""
    a = abs(Fraction(x))
    best = min(range(8), key=lambda c: (abs(a - Fraction(MAGS[c])), c & 1))
    return (8 if np.signbit(x) else 0) | best


def test_e4m3_decoder_matches_definition_and_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in range(256):
        got = oracle.e4m3_to_f32(c)
        want = e4m3_value(c)
        if np.isnan(want):
            assert np.isnan(got) and np.isnan(tv[c])
        else:
            assert got == want == tv[c], (hex(c), got, want, tv[c])


def test_e2m1_every_code_round_trips():
    for c in range(16):
        assert oracle.f32_to_e2m1(e2m1_value(c)) == c, c


def test_e2m1_midpoints_neighbours_and_random_match_exact_rounding():
    vals = []
    for m0, m1 in zip(MAGS, MAGS[1:]):
        mid = np.float32((m0 + m1) / 2)
        vals += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(9))]
    vals += [np.float32(v) for v in (6.0, 6.5, 7.0, 1e30, 2.0 ** -140, 0.0)]
    rng = np.random.default_rng(5)
    vals += list(rng.uniform(-8, 8, 4000).astype(np.float32))
    vals += list((rng.standard_normal(1000) * 0.3).astype(np.float32))
    for v in vals:
        for x in (float(v), -float(v)):
            assert oracle.f32_to_e2m1(x) == e2m1_exact(x), x
    assert oracle.f32_to_e2m1(float("inf")) == 7
    assert oracle.f32_to_e2m1(float("-inf")) == 15


def test_golden_fp4_rows():
    with open(os.path.join(GOLD, "fp4_quant.json")) as fh:
        g = json.load(fh)
    for row in g["rows"]:
        bits = np.array([int(h, 16) for h in row["bf16_hex"]], np.uint16)
        vals = (bits.astype(np.uint32) << 16).view(np.float32)
        want = np.array(row["values"], np.float32)
        assert np.array_equal(vals, want) and np.array_equal(np.signbit(vals), np.signbit(want))
        q, sc = oracle.quantize_fp4(bits[None, :])
        assert q[0].tobytes().hex().upper() == row["codes_hex"]
        assert sc[0].tobytes().hex().upper() == row["scales_hex"]


def e2m1_nearest_even(y: Fraction, negative: bool) -> int:
    """E2M1 code of an exact value: nearest magnitude, ties to the even code,
    saturating at 6; the sign bit as given."""
    a = abs(y)
    best = min(range(8), key=lambda c: (abs(a - Fraction(MAGS[c])), c & 1))
    return (8 if negative else 0) | best


def _codes_hex(codes):
    return bytes(c0 | (c1 << 4) for c0, c1 in zip(codes[0::2], codes[1::2])).hex().upper()


def test_golden_fp4_rows_rederived_in_exact_arithmetic():
    """s = value(e4m3(fp32(amax / 6))) and code = e2m1(fp32(x / s)), every
    rounding done on exact rationals here, give the golden codes and scale
    codes; where a row lists the codes of x * fp32(1 / s), those differ."""
    with open(os.path.join(GOLD, "fp4_quant.json")) as fh:
        g = json.load(fh)
    for row in g["rows"]:
        vals = np.array(row["values"], np.float32)
        codes, recip, scales = [], [], []
        for b0 in range(0, len(vals), 16):
            xs = [Fraction(float(v)) for v in vals[b0:b0 + 16]]
            amax = max(abs(x) for x in xs)
            s8 = e4m3_nearest_even(rn_f32(amax / 6)) if amax > 0 else 0
            s = Fraction(e4m3_value(s8))
            scales.append(s8)
            r = rn_f32(1 / s) if s > 0 else Fraction(0)
            for x, v in zip(xs, vals[b0:b0 + 16]):
                neg = bool(np.signbit(v))
                codes.append(e2m1_nearest_even(rn_f32(x / s) if s > 0 else Fraction(0), neg))
                recip.append(e2m1_nearest_even(rn_f32(x * r), neg))
        assert _codes_hex(codes) == row["codes_hex"]
        assert bytes(scales).hex().upper() == row["scales_hex"]
        if "times_reciprocal_codes_hex" in row:
            assert _codes_hex(recip) == row["times_reciprocal_codes_hex"] != row["codes_hex"]


def _rows(wid=2, T=64):
    w = wl.WORKLOADS[wid].scaled(T=T, cap=T)
    return w, wl.hidden_bf16(w, 0, 9)


def test_fp4_scales_are_e4m3_of_amax_over_6():
    w, x = _rows()
    q, sc = oracle.quantize_fp4(x)
    f = (x.astype(np.uint32) << 16).view(np.float32)
    amax = np.abs(f.reshape(w.T, -1, 16)).max(axis=2)
    s = (amax / np.float32(6)).astype(np.float32)
    want = torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(sc, want)


def test_fp4_dequantisation_error_bound():
    """|x - value(q) * s| <= half the E2M1 spacing at |x / s| (0.25, 0.5, 1
    below 2, 4, 6) times s; above 6 (the scale rounded down) the
    saturation error, at most 6 * 2^-4 / (1 - 2^-4) times s."""
    w, x = _rows(T=128)
    q, sc = oracle.quantize_fp4(x)
    f = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(w.T, -1, 16)
    codes = np.stack([q & 0xF, q >> 4], axis=2).reshape(w.T, -1, 16)
    vals = np.vectorize(lambda c: e2m1_value(int(c)))(codes)
    s = np.vectorize(lambda c: e4m3_value(int(c)))(sc)[:, :, None]
    assert (s > 0).all() and (s < 448).all()
    y = np.abs(f) / np.where(s > 0, s, 1)
    half = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    sat = np.maximum(y - 6, 0)
    assert (sat <= 6 * 2.0 ** -4 / (1 - 2.0 ** -4) + 1e-6).all()
    err = np.abs(f - vals * s)
    assert (err <= (np.maximum(half, sat) + 1e-6) * s + 1e-30).all()


def test_pack_fp4_is_quantize_then_pack_with_zero_scale_padding():
    w, x = _rows(T=40)
    w = w.scaled(H=32 * 16 + 16)                  # H/16 = 33 scale bytes, padded to 48
    x = wl.hidden_bf16(w, 1, 3)
    ids, wts = wl.routing(w, 1, 3)
    extra = np.arange(w.T * 16, dtype=np.uint8).reshape(w.T, 16)
    r = oracle.dispatch_pack_fp4(ids, wts, w.E, w.W, w.cap, x, [extra], fill=0xAB)
    q, sc = oracle.quantize_fp4(x)
    assert oracle.fp4_scale_pitch(w.H) == 48
    ts = r["token_slot"]
    for d in range(w.W):
        for t in range(w.T):
            slot = ts[t, d]
            if slot < 0:
                continue
            assert np.array_equal(r["send"][0][d, slot], q[t])
            assert np.array_equal(r["send"][1][d, slot, :33], sc[t])
            assert (r["send"][1][d, slot, 33:] == 0).all()
            assert np.array_equal(r["send"][2][d, slot], extra[t])
    plain = oracle.dispatch_pack(ids, wts, w.E, w.W, w.cap)
    for k in ("send_cnt", "send_eloc", "token_slot"):
        assert np.array_equal(r[k], plain[k])


def test_fp4_nonfinite_inputs():
    """Hand-derived: NaN never becomes a block's amax, even followed by
    smaller values; an infinite amax saturates the scale at 448; every code
    carries its input's sign bit (a NaN gives a zero of its sign)."""
    row = np.zeros(32, np.uint16)
    # block 0: -sNaN, +inf, 1.0, -2.0: amax = inf, scale 0x7E (s = 448)
    row[0:4] = [0xFFBC, 0x7F80, 0x3F80, 0xC000]
    # block 1: 1.0, +sNaN, 0.5: amax = 1, 1/6 -> e4m3 0.171875 (0x23):
    # 1.0 / s = 5.82 -> 7; 0.5 / s = 2.91 -> 3 (code 5); NaN -> +0
    row[16:19] = [0x3F80, 0x7FA0, 0x3F00]
    q, sc = oracle.quantize_fp4(row[None, :])
    assert sc[0].tolist() == [0x7E, 0x23]
    want = [0x78, 0x80, 0, 0, 0, 0, 0, 0, 0x07, 0x05, 0, 0, 0, 0, 0, 0]
    assert q[0].tolist() == want
