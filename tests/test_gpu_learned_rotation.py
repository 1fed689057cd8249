"""GPU parity of the two-level rotation with a learned block matrix.

"TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization", technical
summary sec. 2(b): the rotation inside each 32-block is a learned orthogonal
matrix. The kernel applies R (fp32, split into three exact bf16 terms) on
the matrix cores after the permutation, then quantizes to MXFP4: rotated
values meet the rotated-path tolerance against the oracle's fp64 product, the
quantizer is bit-exact on the kernel's own rotated values, and at most 1e-4
of codes differ end to end. The inverse (decode, R^T, un-permute, bf16) meets
one bf16 rounding plus the fp32 sum bound.
"""
import numpy as np
import pytest
import scipy.stats

torch = pytest.importorskip("torch")

import block_scaled_fp4_absmax_amd as fp4
from block_scaled_fp4_absmax_amd import inputs
from parity_util import bf16_bits, check_rotated, note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp4.lib()


def sync():
    torch.cuda.synchronize()


def np_u8(t):
    return t.cpu().numpy()


def _random_rotation(seed):
    return scipy.stats.ortho_group.rvs(32, random_state=seed).astype(np.float32)


@pytest.fixture(scope="module")
def learned():
    """R calibrated on a Student-t activation sample with its permutation."""
    x = inputs.gen_c3(rows=256, cols=2048)
    e = fp4.channel_energy(to_dev(x))
    perm = fp4.build_permutation(e)
    R, loss = fp4.calibrate_block_rotation(to_dev(x), perm, iters=60, angles=32)
    assert loss[1] <= loss[0]
    assert not np.array_equal(R.numpy(), R.numpy().T)  # a general (non-Hadamard) matrix
    return R.numpy()


def _case(orc, x, perm, R):
    xt = to_dev(x)
    pt = torch.from_numpy(np.ascontiguousarray(perm, np.int32)).cuda()
    rt = torch.from_numpy(np.ascontiguousarray(R, np.float32)).cuda()
    c, s, y = fp4.rotate_quantize_r(xt, pt, rt, want_rotated=True)
    sync()
    yg = y.cpu().numpy()
    # the quantizer is exact on the kernel's own rotated values
    qc, qs = orc.mx_quantize_f32(yg)
    assert np.array_equal(np_u8(c), qc) and np.array_equal(np_u8(s), qs)
    oc, os_, oy = orc.rotate_quantize_r(x, perm, R.astype(np.float64))
    return check_rotated(yg, oy, np_u8(c), np_u8(s), oc, os_), (c, s, pt, rt)


def _unrotate_check(orc, c, s, perm, R, pt, rt):
    d = fp4.dequantize_r(c, s, pt, rt)
    sync()
    yh = orc.dequantize_f64(np_u8(c), np_u8(s), 0)
    want = orc.unrotate_r_f64(yh, perm, R.astype(np.float64))
    got = inputs.bf16_bits_to_f32(bf16_bits(d)).astype(np.float64)
    # fp32 sums of 96 exact products (3 bf16 terms of R), one bf16 rounding
    rows, cols = want.shape
    absy = np.abs(yh).reshape(rows, cols // 32, 32)
    bound = (absy @ np.abs(R.astype(np.float64))).reshape(rows, cols)  # sum_i |R_ij| |y_i|
    inv = np.empty(cols, np.int64)
    inv[perm] = np.arange(cols)
    bound = bound[:, inv]
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 2.0 ** -20 * bound)
    return got


# cols 96 .. 16384: one to four MFMA tiles per wave per row, partial tiles at
# 96, 2080 and 8224; 1537 and 2500 rows: work-groups with unequal row counts
@pytest.mark.parametrize("rows,cols", [(3, 96), (37, 2080), (5, 16384), (6, 8224), (4, 12288),
                                       (1537, 8192), (2500, 1024)])
def test_learned_rotation_shapes(orc, rows, cols):
    note(f"case: learned block matrix, random orthogonal R, {rows}x{cols}")
    x = inputs.gen_c3(rows=rows, cols=cols)
    perm = np.random.default_rng(cols + rows).permutation(cols).astype(np.int32)
    R = _random_rotation(cols)
    r, (c, s, pt, rt) = _case(orc, x, perm, R)
    note(f"  {r}")
    _unrotate_check(orc, c, s, perm, R, pt, rt)


@pytest.mark.parametrize("rows,cols", [(5, 28672), (300, 24576)])
def test_learned_rotation_wide_rows(orc, rows, cols):
    """Rows wider than 16384 (forward only: the inverse permutation is
    limited to 16384 columns)."""
    note(f"case: learned block matrix, wide rows {rows}x{cols}")
    x = inputs.gen_c3(rows=rows, cols=cols)
    perm = np.random.default_rng(cols + rows).permutation(cols).astype(np.int32)
    r, _ = _case(orc, x, perm, _random_rotation(cols))
    note(f"  {r}")


@pytest.mark.parametrize("kind", [2, 8])
def test_learned_rotation_channel_runs(orc, learned, kind):
    note(f"case: learned R with a permutation of {kind}-channel runs, 300x8192")
    x = inputs.gen_c4(rows=300)
    runs = np.random.default_rng(kind).permutation(8192 // kind).astype(np.int32)
    perm = (kind * runs[:, None] + np.arange(kind)[None, :]).reshape(-1).astype(np.int32)
    r, (c, s, pt, rt) = _case(orc, x, perm, learned)
    note(f"  {r}")
    _unrotate_check(orc, c, s, perm, learned, pt, rt)


def test_learned_rotation_strided_and_untouched_padding(orc, learned):
    note("case: learned R, strided input and padded outputs, 33x2048")
    rows, cols = 33, 2048
    x = inputs.gen_c3(rows=rows, cols=cols)
    perm = np.random.default_rng(1).permutation(cols).astype(np.int32)
    big = torch.zeros((rows, cols + 40), dtype=torch.bfloat16, device="cuda")
    big[:, :cols] = to_dev(x)
    cbuf = torch.full((rows, cols // 2 + 12), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((rows, cols // 32 + 8), 0xCD, dtype=torch.uint8, device="cuda")
    pt = torch.from_numpy(perm).cuda()
    rt = torch.from_numpy(learned).cuda()
    c, s, _ = fp4.rotate_quantize_r(big[:, :cols], pt, rt, codes=cbuf[:, :cols // 2],
                                    scales=sbuf[:, :cols // 32])
    ref_c, ref_s, _ = fp4.rotate_quantize_r(to_dev(x), pt, rt)
    sync()
    assert torch.equal(c, ref_c) and torch.equal(s, ref_s)
    assert np.all(np_u8(cbuf)[:, cols // 2:] == 0xAB) and np.all(np_u8(sbuf)[:, cols // 32:] == 0xCD)
    obuf = torch.full((rows, cols + 16), 7.0, dtype=torch.bfloat16, device="cuda")
    d = fp4.dequantize_r(c, s, pt, rt, out=obuf[:, :cols])
    d2 = fp4.dequantize_r(ref_c, ref_s, pt, rt)
    sync()
    assert torch.equal(d, d2) and bool((obuf[:, cols:] == 7.0).all())


def test_hadamard_matrix_agrees_with_the_hadamard_path(orc):
    """R = H / sqrt(32) in fp32 through the learned path against the
    dedicated Hadamard kernel: rotated values within the rotated-path
    tolerance of each other, codes nearly all equal."""
    note("case: learned path with R = H / sqrt(32) vs the Hadamard path, 512x8192")
    x = inputs.gen_c3(rows=512)
    perm = np.random.default_rng(3).permutation(8192).astype(np.int32)
    H = (orc.hadamard_matrix(32)).astype(np.float32)
    pt = torch.from_numpy(perm).cuda()
    c1, s1, y1 = fp4.rotate_quantize_r(to_dev(x), pt, torch.from_numpy(H).cuda(),
                                       want_rotated=True)
    c2, s2, y2 = fp4.rotate_quantize(to_dev(x), pt, 32, want_rotated=True)
    sync()
    r = check_rotated(y1.cpu().numpy(), y2.cpu().numpy(), np_u8(c1), np_u8(s1), np_u8(c2),
                      np_u8(s2))
    note(f"  {r}")


def test_learned_rotation_c4_full_size_sampled(orc, learned):
    note("case: C4 full 16384x8192, permutation + learned R, sampled rows vs oracle")
    x = inputs.gen_c4()
    xt = to_dev(x)
    perm = fp4.build_permutation(fp4.channel_energy(xt)).numpy()
    pt = torch.from_numpy(perm).cuda()
    rt = torch.from_numpy(learned).cuda()
    c, s, y = fp4.rotate_quantize_r(xt, pt, rt, want_rotated=True)
    sync()
    rows = np.sort(np.random.default_rng(9).choice(x.shape[0], 48, replace=False))
    oc, os_, oy = orc.rotate_quantize_r(np.ascontiguousarray(x[rows]), perm,
                                        learned.astype(np.float64))
    ri = torch.from_numpy(rows).cuda()
    r = check_rotated(y[ri].cpu().numpy(), oy, np_u8(c[ri]), np_u8(s[ri]), oc, os_)
    note(f"  {r}")
    d = fp4.dequantize_r(c, s, pt, rt)
    sync()
    sq = orc.sqnr_db(inputs.bf16_bits_to_f32(x[rows]),
                     inputs.bf16_bits_to_f32(bf16_bits(d[ri])))
    note(f"  round-trip SQNR on the sampled rows {sq:.2f} dB")
    assert sq > 15


def test_learned_rotation_empty(orc, learned):
    note("case: learned R, zero rows")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    pt = torch.arange(64, dtype=torch.int32, device="cuda")
    rt = torch.from_numpy(learned).cuda()
    c, s, _ = fp4.rotate_quantize_r(x, pt, rt)
    d = fp4.dequantize_r(c, s, pt, rt)
    sync()
    assert c.shape == (0, 32) and d.shape == (0, 64)
