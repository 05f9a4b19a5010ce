"""The quantising pack divides by a scale s as fp32(x * fp64(1 / s)): the
fp64 product of x and the correctly rounded fp64 reciprocal, rounded once to
binary32. That equals the correctly rounded binary32 quotient x / s, because
x * fp64(1 / s) is within 2^-52 (relative) of x / s while a quotient of two
binary32 numbers is never a binary32 midpoint and is at least 2^-49
(relative) away from every one. This checks the identity on the CPU (IEEE
arithmetic in numpy) over every finite bf16 value x and scales of the kinds
the pack forms: fp32(amax / 448) for bf16 amax, every positive E4M3 value,
and random fp32 values. Quotients in the binary32 subnormal range are left
out: they encode to a zero code in both formats either way.
"""
import numpy as np


def _scales():
    bits = np.arange(0x0001, 0x7F80, 3, dtype=np.uint32) << 16     # bf16 amax
    amax = bits.view(np.float32)
    s1 = (amax / np.float32(448)).astype(np.float32)
    e4 = []
    for c in range(1, 0x7F):
        e, f = c >> 3, c & 7
        e4.append((f / 8) * 2.0 ** -6 if e == 0 else (1 + f / 8) * 2.0 ** (e - 7))
    s2 = np.array(e4, np.float32)
    rng = np.random.default_rng(7)
    s3 = (rng.random(2000) * 2.0 ** rng.integers(-60, 60, 2000)).astype(np.float32)
    s = np.concatenate([s1, s2, s3])
    return s[(s > 0) & np.isfinite(s)]


def test_fp64_reciprocal_product_is_the_fp32_quotient():
    x = (np.arange(0x10000, dtype=np.uint32) << 16).view(np.float32)
    x = x[np.isfinite(x)]
    S = _scales()
    checked = 0
    with np.errstate(all="ignore"):
        for i in range(0, len(S), 128):
            s = S[i:i + 128][:, None]
            want = x[None, :] / s
            got = (x[None, :].astype(np.float64) * (1.0 / s.astype(np.float64))).astype(np.float32)
            same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
            tiny = np.abs(want) < np.float32(2.0 ** -126)
            bad = ~same & ~tiny
            assert not bad.any(), (s[np.argwhere(bad)[0][0], 0], x[np.argwhere(bad)[0][1]])
            checked += int((~tiny).sum())
    assert checked > 3e8
