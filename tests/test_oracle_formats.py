"""Pins for the oracle's element and scale formats (CPU only).

Each test checks the oracle against something other than itself: a value set
the pages print, a textbook formula, an exact Fraction brute force, a
different rounding construction, or torch's own FP8 decoders.
"""
import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_golden

MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
        Fraction(3), Fraction(4), Fraction(6)]


def test_e2m1_value_set_matches_page(orc):
    printed = read_golden("e2m1_value_set.txt")[0].split()
    want = sorted(float(v) for v in printed)
    got = sorted(orc.e2m1_value(c) for c in range(16))
    assert got == want
    # both zeros exist and differ only in sign: the redundancy RaZeR reclaims
    assert orc.e2m1_value(0) == 0.0 and not math.copysign(1, orc.e2m1_value(0)) < 0
    assert orc.e2m1_value(8) == 0.0 and math.copysign(1, orc.e2m1_value(8)) < 0


def test_e2m1_code_layout_is_textbook_e2m1(orc):
    # 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; E=0 is subnormal M/2
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = m / 2 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        v = orc.e2m1_value(c)
        assert v == (-mag if s else mag)
        assert math.copysign(1, v) == (-1 if s else 1)


def _fraction_nearest(y: Fraction, sign_neg: bool) -> int:
    """Exact brute force: nearest magnitude, ties to the even index."""
    a = abs(y)
    d = [abs(a - m) for m in MAGS]
    best = min(d)
    cands = [k for k in range(8) if d[k] == best]
    idx = [k for k in cands if k % 2 == 0][0] if len(cands) > 1 else cands[0]
    return (8 if sign_neg else 0) | idx


def test_e2m1_nearest_fraction_bruteforce(orc):
    rnd = random.Random(7)
    vals = []
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for m in mids:  # every midpoint and its fp32 neighbours
        f = np.float32(m)
        vals += [float(f), float(np.nextafter(f, np.float32(0))),
                 float(np.nextafter(f, np.float32(100)))]
    vals += [0.0, 6.0, 6.5, 7.0, 1e30, 1e-30]
    vals += [float(np.float32(rnd.uniform(0, 7))) for _ in range(3000)]
    for v in vals:
        for sgn in (1.0, -1.0):
            y = sgn * v
            want = _fraction_nearest(Fraction(abs(y)) * (-1 if sgn < 0 else 1), sgn < 0)
            assert orc.e2m1_nearest(y) == want, y


def _rint_rule(a: np.ndarray) -> np.ndarray:
    """Independent construction: IEEE round-half-even with one mantissa bit.

    In [0,2) the grid step is 0.5, in [2,4) it is 1, in [4,8) it is 2;
    np.rint rounds half to even, and an even multiple of the step is the even
    code. Results above 6 saturate to 6 (index 7).
    """
    idx = np.empty(a.shape, np.int64)
    lo = a < 2
    mid = (a >= 2) & (a < 4)
    hi = a >= 4
    idx[lo] = np.rint(a[lo] * 2).astype(np.int64)
    idx[mid] = np.rint(a[mid]).astype(np.int64) + 2
    with np.errstate(over="ignore", invalid="ignore"):
        k = np.rint(np.minimum(a[hi], 16.0) / 2)
    idx[hi] = np.minimum(k.astype(np.int64) + 4, 7)
    return idx


@pytest.mark.parametrize("e", [-127, -120, -3, 0, 1, 7, 127])
def test_e2m1_nearest_all_bf16_patterns(orc, e):
    pats = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        f = (pats << 16).view(np.float32).astype(np.float64)
    keep = np.isfinite(f)
    f = f[keep]
    y = np.ldexp(f, -e)
    # the oracle is only asked about magnitudes a valid block can produce
    sel = np.abs(y) <= 8.0
    y = y[sel]
    want = (np.signbit(y).astype(np.int64) << 3) | _rint_rule(np.abs(y))
    lib = orc._load()
    got = np.fromiter((lib.orc_e2m1_nearest(float(v)) for v in y), np.int64, count=y.size)
    assert np.array_equal(got, want)


def test_e4m3_decoder_matches_torch(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in range(256):
        v = orc.e4m3_value(c)
        if math.isnan(tv[c]):
            assert math.isnan(v), c
        else:
            assert v == float(tv[c]) and math.copysign(1, v) == math.copysign(1, float(tv[c])), c


def test_e4m3_encoder_midpoints(orc):
    vals = [orc.e4m3_value(c) for c in range(0x7F)]
    assert vals == sorted(vals) and vals[-1] == 448.0
    for c in range(0x7E):
        lo, hi = vals[c], vals[c + 1]
        mid = (lo + hi) / 2  # exact in double
        even = c if c % 2 == 0 else c + 1
        assert orc.e4m3_encode(mid) == even, (c, mid)
        m32 = np.float32(mid)
        if float(m32) == mid:  # fp32 neighbours of the midpoint
            assert orc.e4m3_encode(float(np.nextafter(m32, np.float32(1e9)))) == c + 1
            assert orc.e4m3_encode(float(np.nextafter(m32, np.float32(0)))) == c
        assert orc.e4m3_encode(lo) == c and orc.e4m3_encode(hi) == c + 1
    # saturation above the largest finite value and flush below half the smallest
    for v in (448.0, 460.0, 464.0, 500.0, 1e30):
        assert orc.e4m3_encode(v) == 0x7E
    assert orc.e4m3_encode(2.0 ** -10) == 0
    assert orc.e4m3_encode(float(np.nextafter(np.float32(2.0 ** -10), np.float32(1)))) == 1


def test_e8m0_decoder_matches_torch(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e8m0fnu).to(torch.float32).numpy()
    for b in range(256):
        v = orc.e8m0_value(b)
        if math.isnan(tv[b]):
            assert math.isnan(v) and b == 255
        else:
            assert v == float(tv[b]), b


def test_e8m0_ceiling_rule_minimal_exhaustive(orc):
    """Every non-negative finite bf16 amax: 6*2^e covers it, 6*2^(e-1) does not."""
    for h in range(0x7F80):
        amax = orc.bf16_to_f32(h)
        b = orc.e8m0_scale(amax)
        assert 0 <= b <= 254
        e = b - 127
        assert amax <= 6.0 * 2.0 ** e, h
        assert e == -127 or amax > 6.0 * 2.0 ** (e - 1), h
    assert orc.e8m0_scale(float("inf")) == 0xFF
    assert orc.e8m0_scale(float("nan")) == 0xFF
    assert orc.e8m0_scale(0.0) == 0


def test_e8m0_floor_rule(orc):
    for h in range(1, 0x7F80, 7):
        amax = orc.bf16_to_f32(h)
        b = orc.e8m0_scale(amax, floor_rule=True)
        e = b - 127
        k = math.floor(math.log2(amax))
        assert e == max(-127, min(127, k - 2)), h
    assert orc.e8m0_scale(0.0, floor_rule=True) == 0


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0x00000001, 0x80000001,
                         0x3F808000, 0x3F818000, 0x3F80FFFF, 0x7F7F8000], np.uint32)
    bits = np.concatenate([bits, specials])
    f = bits.view(np.float32)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for i in range(bits.size):
        got = orc.f32_to_bf16(float(f[i]))
        if math.isnan(f[i]):
            assert (got & 0x7F80) == 0x7F80 and (got & 0x7F)
        else:
            assert got == ref[i], hex(int(bits[i]))


def test_e2m1_all_bf16_all_exponents_through_the_block_quantizer(orc):
    """Every finite bf16 pattern at every E8M0 exponent a finite block can
    reach, e in [-127, 126] (about 8 M elements): blocks of 31 test values and
    one pin element, 6 * 2^e (for e = 126, where that overflows fp32, the
    largest finite fp32, which also needs e = 126), so the ceiling rule
    chooses exactly e; the oracle's MXFP4 quantizer must give the
    round-half-even code of x * 2^-e (exact in float64) and the scale byte
    e + 127."""
    pats = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        f32 = (pats << 16).view(np.float32)
    f32 = f32[np.isfinite(f32)]
    total = 0
    for e in range(-127, 127):
        top = np.float32(np.ldexp(6.0, e)) if e < 126 else np.finfo(np.float32).max
        x = f32[np.abs(f32.astype(np.float64)) <= float(top)]
        nb = -(-x.size // 31)
        blocks = np.zeros((nb, 32), np.float32)
        vals = np.zeros(nb * 31, np.float32)
        vals[:x.size] = x
        blocks[:, :31] = vals.reshape(nb, 31)
        blocks[:, 31] = top
        codes, scales = orc.mx_quantize_f32(blocks)
        assert np.all(scales == e + 127), e
        nib = np.empty((nb, 32), np.uint8)
        nib[:, 0::2], nib[:, 1::2] = codes & 15, codes >> 4
        got = nib[:, :31].reshape(-1)[:x.size].astype(np.int64)
        y = np.ldexp(x.astype(np.float64), -e)
        want = (np.signbit(y).astype(np.int64) << 3) | _rint_rule(np.abs(y))
        assert np.array_equal(got, want), e
        total += x.size
    assert total > 8_000_000
