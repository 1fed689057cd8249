"""Pins for NVFP4 of fp32 values and the 16-point block rotation (CPU only).

"TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization" (technical
summary, the generalisation remark of its results) reports the rotation with
NVFP4 as well; NVFP4 blocks hold 16 elements, so the intra-block rotation is
the 16-point Hadamard there and the quantizer sees fp32 rotated values.
"""
import numpy as np
import pytest
import scipy.linalg

from block_scaled_fp4_absmax_amd import inputs


def _rotated(orc, rows=64, cols=1024, seed=3):
    x = inputs.gen_c3(rows=rows, cols=cols)
    perm = np.random.default_rng(seed).permutation(cols).astype(np.int32)
    return orc.rotate(x, perm, 16), x, perm


def test_rotate16_matches_dense_product(orc):
    x = inputs.gen_c3(rows=8, cols=256)
    perm = np.random.default_rng(0).permutation(256).astype(np.int32)
    y = orc.rotate(x, perm, 16)
    xf = inputs.bf16_bits_to_f32(x).astype(np.float64)[:, perm]
    h = scipy.linalg.hadamard(16) / 4.0
    ref = (xf.reshape(8, 16, 16) @ h.T).reshape(8, 256)
    assert np.array_equal(y, ref.astype(np.float32))


@pytest.mark.parametrize("name,rows", [("c2", 64), ("c5_4", 16)])
def test_rotation16_preserves_norm(orc, name, rows):
    x = inputs.generate(name, rows=rows)
    cols = x.shape[1]
    perm = np.random.default_rng(2).permutation(cols).astype(np.int32)
    xf = inputs.bf16_bits_to_f32(x).astype(np.float64)
    for p in (None, perm):
        y = orc.rotate(x, p, 16).astype(np.float64)
        nx, ny = np.linalg.norm(xf, axis=1), np.linalg.norm(y, axis=1)
        assert np.all(np.abs(ny - nx) <= 1e-6 * nx)
        assert np.abs(orc.unrotate_f64(y, p, 16) - xf).max() <= 1e-6 * np.abs(xf).max()


@pytest.mark.parametrize("razer", [False, True])
def test_nv_f32_reduces_to_bf16_quantizer(orc, razer):
    """On fp32 inputs that are bf16 values the fp32 entry point gives the bf16
    entry point's bytes. Both run the same block function, so this checks the
    entry points' marshalling only; the block arithmetic itself is pinned in
    test_oracle_nv_steps.py."""
    x = inputs.gen_c2(rows=128, cols=1024)
    a = orc.nv_quantize(x, razer)
    b = orc.nv_quantize_f32(inputs.bf16_bits_to_f32(x), razer)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


def test_nv_f32_tensor_scale(orc):
    y, _, _ = _rotated(orc)
    amax = orc.nv_tensor_amax_f32(y)
    assert amax == np.abs(y).max()
    st = orc.nv_tensor_scale(amax)
    assert abs(6 * 448 * st - amax) <= amax * 2 ** -23


@pytest.mark.parametrize("razer", [False, True])
def test_nv_f32_error_bound(orc, razer):
    """Per element |y - y_hat| <= half a grid step * s_eff (+ fp32 rounding)."""
    y, _, _ = _rotated(orc)
    c, s, st = orc.nv_quantize_f32(y, razer)
    yh = orc.dequantize_f64(c, s, 1, razer, st)
    yf = y.astype(np.float64)
    sb = (s & 0x7F).astype(int)
    seff = np.array([orc.e4m3_value(b) for b in range(128)])[sb] * st
    seff = np.repeat(seff, 16, axis=1)
    a = np.abs(yf) / np.where(seff > 0, seff, 1)
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    err = np.abs(yf - yh)
    bound = half * seff + np.abs(yf) * 2 ** -21 + seff * 6 * 2 ** -21
    sat = a > 6
    assert np.all(err[~sat] <= bound[~sat])
    assert np.all(a[sat] < 6 * (1 + 2 ** -4) * (1 + 2 ** -20))


def test_nv_f32_scale_invariance_and_symmetry(orc):
    y, _, _ = _rotated(orc, rows=32, cols=512)
    c0, s0, st0 = orc.nv_quantize_f32(y, True)
    for k in (-5, 3):
        ck, sk, stk = orc.nv_quantize_f32(y * np.float32(2.0 ** k), True)
        assert stk == st0 * 2.0 ** k
        assert np.array_equal(ck, c0) and np.array_equal(sk, s0)
    cp, sp, _ = orc.nv_quantize_f32(y, False)
    cn, sn, _ = orc.nv_quantize_f32(-y, False)
    assert np.array_equal(sn, sp) and np.array_equal(cn, cp ^ np.uint8(0x88))


def test_nv_f32_razer_never_worse_per_block(orc):
    y, _, _ = _rotated(orc, rows=64, cols=1024)
    cr, sr, st = orc.nv_quantize_f32(y, True)
    cp, sp, _ = orc.nv_quantize_f32(y, False, st)
    er = (orc.dequantize_f64(cr, sr, 1, True, st) - y) ** 2
    ep = (orc.dequantize_f64(cp, sp, 1, False, st) - y) ** 2
    rows, cols = y.shape
    br = er.reshape(rows, cols // 16, 16).sum(-1)
    bp = ep.reshape(rows, cols // 16, 16).sum(-1)
    # same block scales; the RaZeR code book contains the plain one
    assert np.array_equal(sr & 0x7F, sp)
    assert np.all(br <= bp * (1 + 1e-12) + 1e-30)


def test_rotation16_nvfp4_round_trip(orc):
    """The rotated NVFP4 path decodes back (inverse rotation) to within NVFP4
    accuracy. On these synthetic heavy-tailed activations the fixed 16-point
    Hadamard does not beat plain NVFP4, whose fine E4M3 block scales already
    isolate outliers; the round trip stays well inside the 4-bit regime."""
    x = inputs.gen_c3(rows=256, cols=2048)
    xf = inputs.bf16_bits_to_f32(x).astype(np.float64)
    for razer in (False, True):
        c, s, st, y = orc.rotate_quantize_nv(x, None, 16, razer)
        back = orc.unrotate_f64(orc.dequantize_f64(c, s, 1, razer, st), None, 16)
        assert orc.sqnr_db(xf, back) > 20.0
        # the rotated values themselves quantize as well as any fp32 tensor
        assert orc.sqnr_db(y, orc.dequantize_f64(c, s, 1, razer, st)) > 20.0
