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
