"""Pins for the oracle's MXINT4 quantizer (CPU only).

"TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization" (technical
summary, the generalisation remark of its results) reports the rotation with
an MXINT4 grid too; the pages name the format and nothing more. The oracle
reads it as the 4-bit microscaling integer element: two's complement k in
[-8, 7] with value k / 4 (two fraction bits, the 4-bit analogue of MXINT8's
k / 64), 32-element blocks, an E8M0 scale, nearest with ties to even k,
clamped to |k| <= 7. The pins below come from that definition and from
library routines, not from the oracle's own code.
"""
from fractions import Fraction

import numpy as np
import pytest

from block_scaled_fp4_absmax_amd import inputs


def _unpack(codes):
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


def _signed(nib):
    """Two's complement of 4-bit codes by numpy's arithmetic shift of int8."""
    return (np.asarray(nib, np.uint8) << 4).astype(np.int8) >> 4


def _f64(x):
    return inputs.bf16_bits_to_f32(x).astype(np.float64)


def test_int4_decoder_is_twos_complement(orc):
    codes = np.arange(16, dtype=np.uint8)
    want = _signed(codes).astype(np.float64) / 4
    got = np.array([orc.int4_value(int(c)) for c in codes])
    assert np.array_equal(got, want)
    assert got.min() == -2.0 and got.max() == 1.75


def test_int4_nearest_matches_rint(orc):
    """np.rint rounds half to even: the oracle's brute-force search agrees on
    random values, every midpoint and one double ulp either side."""
    rng = np.random.default_rng(5)
    ys = list(rng.uniform(-2.5, 2.5, 4000))
    for k in range(-8, 8):
        mid = (2 * k + 1) / 8.0
        ys += [mid, np.nextafter(mid, -9), np.nextafter(mid, 9)]
    ys += [1.75, 1.8, 1.875, 1.9, 2.0, 100.0, -1.75, -1.875, -1.99, -2.0, -300.0, 0.0, -0.0]
    for y in ys:
        k = int(np.clip(np.rint(4 * y), -7, 7))
        assert _signed(orc.int4_nearest(y)) == k, y


def test_int4_nearest_fraction_bruteforce(orc):
    """Exact rational nearest search with an explicit tie rule."""
    rng = np.random.default_rng(6)
    for _ in range(600):
        y = Fraction(int(rng.integers(-80, 81)), 32)  # many exact ties at k / 4 + 1/8
        best = min(range(-7, 8), key=lambda k: (abs(y - Fraction(k, 4)), k % 2))
        assert _signed(orc.int4_nearest(float(y))) == best


def test_mxint4_scale_minimal_exhaustive(orc):
    """Every finite non-negative bf16 magnitude: the byte is the smallest e in
    [-127, 127] with amax <= 1.75 * 2^e; above 1.75 * 2^127 (the top of the
    bf16 range) e stays 127 and the block saturates."""
    bits = np.arange(0, 0x7F80, dtype=np.uint16)
    amax = _f64(bits[None, :])[0]
    e = np.array([orc.mxint4_scale(float(a)) for a in amax]) - 127
    top = amax > 1.75 * 2.0 ** 127
    assert top.sum() > 0 and np.all(e[top] == 127)
    assert np.all((amax <= 1.75 * np.ldexp(1.0, e)) | top)
    assert np.all((e == -127) | (amax > 1.75 * np.ldexp(1.0, e - 1)))
    assert orc.mxint4_scale(float("inf")) == 0xFF and orc.mxint4_scale(float("nan")) == 0xFF


def test_mxint4_floor_rule(orc):
    rng = np.random.default_rng(8)
    a = np.ldexp(rng.uniform(1, 2, 500), rng.integers(-120, 120, 500))
    for v in a:
        assert orc.mxint4_scale(float(v), True) - 127 == np.frexp(v)[1] - 1
    assert orc.mxint4_scale(0.0, True) == 0


def test_mxint4_nearest_grid_and_no_clipping(orc):
    """Whole pipeline: every decoded value is a nearest point of its block's
    grid {k 2^(e-2), |k| <= 7}, and within half a step of the input."""
    x = inputs.gen_c3(rows=128, cols=1024)
    codes, scales = orc.mxint4_quantize(x)
    xh = orc.dequantize_f64(codes, scales, 2)
    xf = _f64(x)
    rows, cols = x.shape
    e = scales.astype(np.int64) - 127
    grid = np.arange(-7, 8)[None, None, :] * np.ldexp(1.0, e - 2)[:, :, None]
    xb = xf.reshape(rows, cols // 32, 32)
    dist = np.abs(xb[..., None] - grid[:, :, None, :]).min(-1)
    assert np.array_equal(np.abs(xb - xh.reshape(xb.shape)), dist)
    assert np.all(np.abs(xb - xh.reshape(xb.shape)) <= np.ldexp(1.0, e - 3)[..., None])
    assert np.all(_signed(_unpack(codes)) != -8)


def test_mxint4_scale_invariance_and_sign_symmetry(orc):
    x = inputs.gen_c1(rows=64, cols=512)
    c0, s0 = orc.mxint4_quantize(x)
    for k in (-30, -1, 2, 50):
        xk = inputs.f64_to_bf16_bits(_f64(x) * 2.0 ** k)
        assert np.array_equal(_f64(xk), _f64(x) * 2.0 ** k)
        ck, sk = orc.mxint4_quantize(xk)
        assert np.array_equal(ck, c0)
        assert np.array_equal(sk.astype(int), s0.astype(int) + k)
    cn, sn = orc.mxint4_quantize(x ^ np.uint16(0x8000))
    assert np.array_equal(sn, s0)
    assert np.array_equal(_signed(_unpack(cn)), -_signed(_unpack(c0)))


def test_mxint4_floor_rule_saturates(orc):
    """Under the floor rule a block maximum in [1.875, 2) * 2^e saturates at 1.75."""
    x = np.zeros((1, 32), np.float64)
    x[0, 0] = 1.9375 * 2.0 ** 3
    x[0, 1] = -1.9375 * 2.0 ** 3
    x[0, 2] = 0.5 * 2.0 ** 3
    xb = inputs.f64_to_bf16_bits(x)
    c, s = orc.mxint4_quantize(xb, floor_rule=True)
    assert s[0, 0] == 127 + 3
    k = _signed(_unpack(c))[0]
    assert k[0] == 7 and k[1] == -7 and k[2] == 2
    c, s = orc.mxint4_quantize(xb)  # default rule: the next exponent, nothing clipped
    assert s[0, 0] == 127 + 4 and _signed(_unpack(c))[0, 0] == 4


def test_mxint4_nonfinite_block(orc):
    x = inputs.gen_c1(rows=2, cols=64)
    x[0, 5] = 0x7FC0  # NaN
    x[1, 40] = 0xFF80  # -Inf
    c, s = orc.mxint4_quantize(x)
    assert s[0, 0] == 0xFF and s[1, 1] == 0xFF and s[0, 1] != 0xFF and s[1, 0] != 0xFF
    u = _unpack(c)
    assert np.all(u[0, :32] == 0) and np.all(u[1, 32:] == 0)
    d = orc.dequantize_f64(c, s, 2)
    assert np.all(np.isnan(d[0, :32])) and np.all(np.isnan(d[1, 32:]))


@pytest.mark.parametrize("had", [32])
def test_mxint4_rotation_helps_heavy_tails(orc, had):
    """On the heavy-tailed activations with outlier channels an integer grid
    gains from the block Hadamard (the rotation spreads an outlier over its
    block, which a uniform grid needs more than a floating-point one)."""
    x = inputs.gen_c3(rows=256, cols=2048)
    xf = _f64(x)
    c0, s0 = orc.mxint4_quantize(x)
    plain = orc.sqnr_db(xf, orc.dequantize_f64(c0, s0, 2))
    c1, s1, y = orc.rotate_quantize_mxint4(x, None, had)
    back = orc.unrotate_f64(orc.dequantize_f64(c1, s1, 2), None, had)
    rot = orc.sqnr_db(xf, back)
    assert rot > plain + 1.0, (plain, rot)
