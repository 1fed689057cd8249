"""Pins for the oracle's GEMM of quantized operands (CPU only).

The RaZeR page (technical summary sec. 2.3) describes GEMM kernels that take
the quantized weights and activations. The oracle decodes both operands
exactly and multiplies in float64; these pins check it against an exact
rational evaluation written from the format definitions, not from the oracle.
"""
from fractions import Fraction

import numpy as np
import pytest

from conftest import read_golden

E2M1 = [Fraction(v) for v in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]


def _val(code):
    m = E2M1[code & 7]
    return -m if code & 8 else m


def _rand_operand(rng, rows, k, emin=120, emax=134):
    codes = rng.integers(0, 256, (rows, k // 2), dtype=np.uint8)
    scales = rng.integers(emin, emax, (rows, k // 32), dtype=np.uint8)
    return codes, scales


def _exact(codes, scales):
    rows, half = codes.shape
    out = [[None] * (2 * half) for _ in range(rows)]
    for r in range(rows):
        for j in range(2 * half):
            c = int(codes[r, j // 2]) >> (4 * (j % 2)) & 15
            out[r][j] = _val(c) * Fraction(2) ** (int(scales[r, j // 32]) - 127)
    return out


def test_e2m1_values_are_the_page_set():
    want = sorted({Fraction(v) for v in read_golden("e2m1_value_set.txt")[0].split()} | {0})
    assert sorted(set(E2M1) | {-v for v in E2M1}) == sorted(set(want) | {-v for v in want})


@pytest.mark.parametrize("m,n,k", [(3, 4, 32), (5, 2, 96)])
def test_gemm_matches_exact_rational(orc, m, n, k):
    rng = np.random.default_rng(m * 100 + n)
    ac, as_ = _rand_operand(rng, m, k)
    bc, bs = _rand_operand(rng, n, k)
    c = orc.gemm_f64(ac, as_, bc, bs)
    A, B = _exact(ac, as_), _exact(bc, bs)
    for i in range(m):
        for j in range(n):
            assert Fraction(c[i, j]) == sum(A[i][t] * B[j][t] for t in range(k))


def test_gemm_one_hot(orc):
    k = 64
    ac = np.zeros((1, k // 2), np.uint8)
    ac[0, 5] = 0x30  # element 11: code 3 = 1.5
    as_ = np.full((1, 2), 127, np.uint8)
    as_[0, 0] = 129  # block 0 scaled by 4: element 11 is 6
    rng = np.random.default_rng(3)
    bc, bs = _rand_operand(rng, 7, k)
    c = orc.gemm_f64(ac, as_, bc, bs)
    B = _exact(bc, bs)
    assert all(Fraction(c[0, j]) == 6 * B[j][11] for j in range(7))


def test_gemm_block_scale_bilinear(orc):
    rng = np.random.default_rng(4)
    ac, as_ = _rand_operand(rng, 6, 256)
    bc, bs = _rand_operand(rng, 5, 256)
    c0 = orc.gemm_f64(ac, as_, bc, bs)
    as2 = as_.copy()
    as2[2] += 1  # every block of row 2 doubles
    c1 = orc.gemm_f64(ac, as2, bc, bs)
    assert np.array_equal(c1[2], 2 * c0[2])
    assert np.array_equal(np.delete(c1, 2, 0), np.delete(c0, 2, 0))
    bs2 = bs.copy()
    bs2[:, 3] -= 2  # block 3 of every B row quartered: only that block's terms change
    c2 = orc.gemm_f64(ac, as_, bc, bs2)
    a = orc.dequantize_f64(ac, as_, 0)
    b = orc.dequantize_f64(bc, bs, 0)
    part = a[:, 96:128] @ b[:, 96:128].T
    assert np.allclose(c2, c0 - 0.75 * part, rtol=0, atol=1e-9 * np.abs(c0).max())


def _e4m3_exact(b):
    """OCP E4M3 (fn): bias 7, subnormals m 2^-9, from the definition."""
    e, m = (b >> 3) & 15, b & 7
    if e == 0:
        return Fraction(m, 512)
    return (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


@pytest.mark.parametrize("razer_a,razer_b", [(False, False), (True, True), (True, False)])
def test_nv_gemm_matches_exact_rational(orc, razer_a, razer_b):
    """NVFP4 operands (E4M3 block scales, fp32 tensor scales, RaZeR code 0x8 =
    +-5 by the scale's top bit) against exact rationals."""
    rng = np.random.default_rng(21 + razer_a + 2 * razer_b)
    m, n, k = 3, 4, 48
    ac = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    as_ = rng.integers(0, 256 if razer_a else 127, (m, k // 16), dtype=np.uint8) & \
        np.uint8(0xFF if razer_a else 0x7F)
    bs = rng.integers(0, 256 if razer_b else 127, (n, k // 16), dtype=np.uint8) & \
        np.uint8(0xFF if razer_b else 0x7F)
    as_[as_ & 0x7F == 0x7F] -= 1  # no NaN scale
    bs[bs & 0x7F == 0x7F] -= 1
    ta, tb = float(np.float32(0.0123)), float(np.float32(3.75e-3))
    c = orc.gemm_f64(ac, as_, bc, bs, 1, razer_a, ta, tb, razer_b=razer_b)

    def val(codes, scales, r, j, rz, ts):
        code = int(codes[r, j // 2]) >> (4 * (j % 2)) & 15
        sbyte = int(scales[r, j // 16])
        if rz and code == 8:
            v = Fraction(-5 if sbyte & 0x80 else 5)
        else:
            v = _val(code)
        return v * _e4m3_exact(sbyte & 0x7F if rz else sbyte) * Fraction(ts)

    # the decoded values are exact in float64; their products need up to 62
    # bits, so the float64 matmul rounds: k roundings of 2^-53 at most
    for i in range(m):
        for j in range(n):
            terms = [val(ac, as_, i, t, razer_a, ta) * val(bc, bs, j, t, razer_b, tb)
                     for t in range(k)]
            want = sum(terms)
            bound = k * Fraction(1, 2 ** 52) * sum(abs(x) for x in terms)
            assert abs(Fraction(c[i, j]) - want) <= bound
