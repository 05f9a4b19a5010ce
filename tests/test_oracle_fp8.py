"""Pins of the oracle's fp8 e4m3 encoding and quantize-on-pack (CPU).

Independent references: the OCP E4M3 definition decoded code by code here
(exponent bias 7, 3 fraction bits, subnormals, 448 the largest finite
value), exact midpoints between neighbouring codes, torch's
float8_e4m3fn conversion (a library routine) on random in-range values,
hand-derived quantised rows (tests/golden/fp8_quant.json), and the rule
(s = fp32(amax / 448), code = e4m3(fp32(x / s))) re-derived in exact
rational arithmetic.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e4m3_value(code: int) -> float:
    """Value of an OCP E4M3 code, from the definition."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    f = code & 0x7
    if e == 0xF and f == 0x7:
        return float("nan")
    if e == 0:
        return sign * (f / 8.0) * 2.0 ** -6
    return sign * (1.0 + f / 8.0) * 2.0 ** (e - 7)


FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_every_finite_code_round_trips():
    for c in FINITE:
        v = e4m3_value(c)
        got = oracle.f32_to_e4m3(v)
        if v == 0.0:
            assert got == (0x80 if c & 0x80 else 0x00)
        else:
            assert got == c, (hex(c), v, hex(got))


def test_midpoints_round_to_even_and_neighbours_to_nearest():
    pos = sorted((e4m3_value(c), c) for c in FINITE if not c & 0x80)
    for (v0, c0), (v1, c1) in zip(pos, pos[1:]):
        mid = np.float32((v0 + v1) / 2)
        assert float(mid) == (v0 + v1) / 2          # exact in fp32
        even = c0 if c0 % 2 == 0 else c1
        assert oracle.f32_to_e4m3(float(mid)) == even
        assert oracle.f32_to_e4m3(-float(mid)) == even | 0x80
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        assert oracle.f32_to_e4m3(float(below)) == c0
        assert oracle.f32_to_e4m3(float(above)) == c1


def test_saturation_and_nan():
    for v in [448.0, 448.0001, 463.9, 464.0, 480.0, 1e6, 3.4e38, float("inf")]:
        assert oracle.f32_to_e4m3(v) == 0x7E
        assert oracle.f32_to_e4m3(-v) == 0xFE
    assert oracle.f32_to_e4m3(float("nan")) & 0x7F == 0x7F


def test_matches_torch_conversion_in_range():
    import torch
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-447.9, 447.9, 20000),
                        rng.standard_normal(20000) * 4,
                        rng.uniform(-2 ** -5, 2 ** -5, 20000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.f32_to_e4m3(float(v)) for v in x], np.uint8)
    assert np.array_equal(got, ref)


def _golden_rows():
    with open(os.path.join(GOLD, "fp8_quant.json")) as fh:
        g = json.load(fh)
    H, group = g["H"], g["group"]
    for r in g["rows"]:
        row = np.zeros(H, np.float32)
        for k, v in r["row_values"].items():
            row[int(k)] = v
        bits = wl.f32_to_bf16_bits(row.reshape(1, H))
        assert np.array_equal(wl.bf16_bits_to_f32(bits)[0], row)   # exact in bf16
        exp = np.zeros(H, np.uint8)
        for k, v in r["codes"].items():
            exp[int(k)] = int(v, 16)
        yield H, group, r, row, bits, exp


def test_golden_quantized_row():
    for H, group, r, row, bits, exp in _golden_rows():
        q, sc = oracle.quantize_fp8(bits, group)
        assert [hex(v) for v in sc[0].view(np.uint32)] == \
            [hex(int(h, 16)) for h in r["scales_f32_hex"]]
        assert q[0].tolist() == exp.tolist()


def rn_f32(q: Fraction) -> Fraction:
    """q rounded to binary32, nearest, ties to even (normal range only)."""
    if q == 0:
        return q
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                   # 2^e <= a < 2^(e+1)
    assert -126 <= e <= 127
    unit = Fraction(2) ** (e - 23)
    n, rem = divmod(a, unit)
    if rem * 2 > unit or (rem * 2 == unit and n % 2 == 1):
        n += 1
    return (n * unit) * (1 if q > 0 else -1)


E4M3_POS = [(Fraction(e4m3_value(c)), c) for c in range(0x7F)]


def e4m3_nearest_even(y: Fraction) -> int:
    """The E4M3 code nearest to y, ties to the even code, magnitudes past
    448 saturating to 448 (the sign taken from y)."""
    a = min(abs(y), Fraction(448))
    _, c = min(E4M3_POS, key=lambda vc: (abs(a - vc[0]), vc[1] & 1))
    return c | (0x80 if y < 0 else 0)


def test_golden_rows_rederived_in_exact_arithmetic():
    """s = fp32(amax / 448) and code = e4m3(fp32(x / s)), both roundings done
    on exact rationals here, give every code and scale of the golden rows;
    the alternative rules listed with the rows give other codes."""
    for H, group, r, row, bits, exp in _golden_rows():
        for g0 in range(0, H, group):
            xs = [Fraction(float(v)) for v in row[g0:g0 + group]]
            amax = max(abs(v) for v in xs)
            s = rn_f32(amax / 448) if amax > 0 else Fraction(1)
            assert float(s) == float(np.uint32(int(r["scales_f32_hex"][g0 // group], 16))
                                      .view(np.float32))
            r448 = rn_f32(Fraction(448) / amax) if amax > 0 else Fraction(1)
            for h, x in enumerate(xs):
                col = g0 + h
                code = e4m3_nearest_even(rn_f32(x / s)) if x != 0 else \
                    (0x80 if np.signbit(row[col]) else 0)
                assert code == exp[col], (col, hex(code), hex(exp[col]))
                if str(col) in r.get("times_448_over_amax_codes", {}):
                    other = e4m3_nearest_even(rn_f32(x * r448))
                    assert other == int(r["times_448_over_amax_codes"][str(col)], 16)
                    assert other != code
                if str(col) in r.get("exact_quotient_codes", {}):
                    other = e4m3_nearest_even(x / s)
                    assert other == int(r["exact_quotient_codes"][str(col)], 16)
                    assert other != code


def test_quantize_dequantize_error_bound():
    """|q*scale - x| <= half an e4m3 step of |x/scale| times scale, i.e.
    2^-4 relative for normal codes, plus the subnormal step."""
    w = wl.WORKLOADS[2].scaled(T=16, H=1024)
    bits = wl.hidden_bf16(w, 0)
    q, sc = oracle.quantize_fp8(bits, 128)
    x = wl.bf16_bits_to_f32(bits).reshape(16, 8, 128)
    deq = np.vectorize(e4m3_value)(q.astype(np.int64)).reshape(16, 8, 128)
    s = sc[:, :, None]
    err = np.abs(deq * s - x)
    bound = np.abs(x) * 2.0 ** -4 + s * 2.0 ** -10
    assert (err <= bound * (1 + 1e-6)).all()
    # the group maximum maps to 448 exactly
    amax_pos = np.abs(x).argmax(axis=2)
    codes_at_max = np.take_along_axis(q.reshape(16, 8, 128), amax_pos[:, :, None], 2)
    assert ((codes_at_max & 0x7F) == 0x7E).all()


def test_pack_fp8_is_quantize_then_pack():
    w = wl.WORKLOADS[1].scaled(H=256, T=40, cap=40)
    ids, wts = wl.routing(w, 0)
    bits = wl.hidden_bf16(w, 0)
    r = oracle.dispatch_pack_fp8(ids, wts, w.E, w.W, w.cap, bits, 128)
    q, sc = oracle.quantize_fp8(bits, 128)
    for d in range(w.W):
        toks = np.nonzero(r["token_slot"][:, d] >= 0)[0]
        c = len(toks)
        assert np.array_equal(r["send"][0][d, :c], q[toks])
        Gp = (sc.shape[1] + 3) // 4 * 4
        got = r["send"][1][d, :c].view(np.float32)
        assert got.shape[1] == Gp
        assert np.array_equal(got[:, :sc.shape[1]], sc[toks])
        assert (got[:, sc.shape[1]:].view(np.uint32) == 0).all()


def test_fp8_nonfinite_inputs():
    """Hand-derived, groups of 32: NaN never becomes a group's amax; an
    infinite amax gives scale inf and r = 0; every code carries its input's
    sign bit (NaN, and inf * 0, give the NaN code with x's sign)."""
    row = np.zeros(64, np.uint16)
    row[0:4] = [0xFFBC, 0x7F80, 0x3F80, 0xC000]     # -sNaN, +inf, 1.0, -2.0
    row[32:35] = [0x3F80, 0x7FA0, 0x3F00]           # 1.0, +sNaN, 0.5
    q, sc = oracle.quantize_fp8(row[None, :], 32)
    assert np.isinf(sc[0, 0]) and sc[0, 1] == np.float32(1.0) / np.float32(448.0)
    assert q[0, :4].tolist() == [0xFF, 0x7F, 0x00, 0x80]
    assert (q[0, 4:32] == 0).all()
    # r = 448: 1.0 -> 448 (0x7E); NaN -> 0x7F; 0.5 -> 224 = 1.75 * 2^7 (0x76)
    assert q[0, 32:35].tolist() == [0x7E, 0x7F, 0x76]
    assert (q[0, 35:] == 0).all()
