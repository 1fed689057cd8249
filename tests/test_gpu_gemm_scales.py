"""GPU checks of MXFP4 scale bytes in the GEMM order (FP4_FLAG_SCALES_GEMM).

With the flag, the quantizers must write the same codes as without it, and
the scale byte of row r, block b at (r / 32) * ld + (b / 8) * 256 +
(r % 32) * 8 + b % 8 -- the byte that the row-major call writes at (r, b) --
and nothing else (the buffer is filled with a sentinel first). The GEMM
reading either operand's scales in that order must return exactly what it
returns from row-major scales (the same kernels and arithmetic), with every
byte the quantizer leaves unwritten set to 0xFF (a NaN scale) to show that
none reaches an output; one case per tile kernel is also held to the
oracle's float64 product by the GEMM bar of test_gpu_gemm.py.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_scaled_fp4_absmax_amd as fp4
from block_scaled_fp4_absmax_amd import inputs
from parity_util import note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp4.lib()


def to_gemm_order(sc, ld, fill):
    """Row-major scale bytes [rows, nb] placed in the GEMM order."""
    rows, nb = sc.shape
    out = np.full(((rows + 31) // 32, ld), fill, np.uint8)
    r = np.arange(rows)[:, None]
    b = np.arange(nb)[None, :]
    out[r // 32, (b // 8) * 256 + (r % 32) * 8 + b % 8] = sc
    return out


def test_gemm_order_positions():
    # a worked position: row 33, block 9 -> group 1, step 1, row 1, byte 1
    sc = np.zeros((34, 10), np.uint8)
    sc[33, 9] = 7
    g = to_gemm_order(sc, 512, 0)
    assert g.shape == (2, 512) and g[1, 256 + 8 + 1] == 7 and g.sum() == 7


def _x(rows, cols, seed, ld=None):
    x = inputs.gen_c4(rows=rows, cols=cols, seed=seed)
    if ld is None:
        return to_dev(x)
    buf = np.zeros((rows, ld), np.uint16)
    buf[:, :cols] = x
    return to_dev(buf)[:, :cols]


def _gemm_scales(rows, cols, fill=0xA5, extra_steps=0):
    g, ld = fp4.gemm_scale_shape(rows, cols)
    return torch.full((g, ld + 256 * extra_steps), fill, dtype=torch.uint8, device="cuda")


# shapes: whole 256-column steps, ragged rows, a partial last step (96, 544),
# one block, one row; (100, 8192) has 32 steps and a partial last group
QUANT_SHAPES = [(64, 256), (100, 8192), (33, 96), (3, 544), (1, 32), (257, 1024)]


@pytest.mark.parametrize("rows,cols", QUANT_SHAPES)
@pytest.mark.parametrize("floor_rule", [False, True])
def test_quantize_gemm_order(rows, cols, floor_rule):
    note(f"quantize gemm order {rows}x{cols} floor={floor_rule}")
    x = _x(rows, cols, seed=rows + cols)
    c0, s0, _ = fp4.quantize(x, floor_rule=floor_rule)
    S = _gemm_scales(rows, cols, extra_steps=1)  # a group stride past the minimum
    c1, s1, _ = fp4.quantize(x, floor_rule=floor_rule, gemm_scales=True, scales=S)
    torch.cuda.synchronize()
    assert s1.data_ptr() == S.data_ptr()
    assert torch.equal(c0, c1)
    want = to_gemm_order(s0.cpu().numpy(), S.shape[1], 0xA5)
    assert np.array_equal(S.cpu().numpy(), want)


def test_quantize_gemm_order_strided():
    note("quantize gemm order strided input and codes")
    rows, cols = 70, 1088
    x = _x(rows, cols, seed=5, ld=cols + 64)
    c0, s0, _ = fp4.quantize(x)
    cbuf = torch.full((rows, cols // 2 + 32), 0x33, dtype=torch.uint8, device="cuda")
    S = _gemm_scales(rows, cols)
    c1, _, _ = fp4.quantize(x, gemm_scales=True, codes=cbuf[:, :cols // 2], scales=S)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1)
    assert torch.all(cbuf[:, cols // 2:] == 0x33)
    assert np.array_equal(S.cpu().numpy(), to_gemm_order(s0.cpu().numpy(), S.shape[1], 0xA5))


# the rotation kernels: permutation + H32 (rows staged in LDS), H32 alone
# (streaming), no transform, a grouped permutation (wide gathers), rows wider
# than 16384 (staged straight into LDS), and the fp32 y written alongside
ROT_CASES = [
    ("perm_h32", 100, 4096, True, 32, 1),
    ("h32", 70, 8192, False, 32, 1),
    ("none", 40, 2048, False, 0, 1),
    ("perm_group4", 66, 4096, True, 32, 4),
    ("perm_wide", 20, 20480, True, 32, 1),
    ("perm_only", 35, 1024, True, 0, 1),
]


@pytest.mark.parametrize("name,rows,cols,use_perm,had,group", ROT_CASES)
def test_rotate_quantize_gemm_order(name, rows, cols, use_perm, had, group):
    note(f"rotate_quantize gemm order {name} {rows}x{cols}")
    x = _x(rows, cols, seed=cols + 7)
    perm = None
    if use_perm:
        perm = fp4.build_permutation(fp4.channel_energy(x), 32, group).cuda()
    c0, s0, y0 = fp4.rotate_quantize(x, perm, had, want_rotated=True)
    S = _gemm_scales(rows, cols)
    c1, s1, y1 = fp4.rotate_quantize(x, perm, had, want_rotated=True, gemm_scales=True, scales=S)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1) and torch.equal(y0, y1)
    assert np.array_equal(S.cpu().numpy(), to_gemm_order(s0.cpu().numpy(), S.shape[1], 0xA5))


def _operand(rows, k, seed, gemm_order):
    x = _x(rows, k, seed=seed)
    nb = k // 32  # row-major scale rows padded to the GEMM's 4-byte multiple
    pad = torch.full((rows, -(-nb // 4) * 4), 0xFF, dtype=torch.uint8, device="cuda")
    codes, scales, _ = fp4.quantize(x, scales=pad[:, :nb])
    if not gemm_order:
        return codes, scales
    S = _gemm_scales(rows, k, fill=0xFF)  # unwritten bytes: NaN scales
    c2, _, _ = fp4.quantize(x, gemm_scales=True, scales=S)
    assert torch.equal(codes, c2)
    return codes, S


# split-K kernels (m <= 256 with few tiles), 128 x 128 tiles, 256 x 256 tiles
# (m, n >= 2048); ragged m, n and a k that is not a whole 256-element step
GEMM_SHAPES = [(16, 512, 1024), (64, 2048, 2048), (200, 96, 544), (512, 768, 2048),
               (300, 200, 544), (2048, 2304, 1024), (2100, 2050, 800)]


@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
@pytest.mark.parametrize("order", ["a", "b", "ab"])
def test_gemm_gemm_order_matches_row_major(m, n, k, order):
    note(f"gemm gemm-order {order} {m}x{n}x{k}")
    A, SA = _operand(m, k, 11, False)
    B, SB = _operand(n, k, 12, False)
    want = fp4.gemm(A, SA, B, SB, out_dtype=torch.bfloat16)
    A2, SA2 = _operand(m, k, 11, "a" in order)
    B2, SB2 = _operand(n, k, 12, "b" in order)
    got = fp4.gemm(A2, SA2, B2, SB2, out_dtype=torch.bfloat16, a_gemm_scales="a" in order,
                   b_gemm_scales="b" in order)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


@pytest.mark.parametrize("m,n,k", [(16, 512, 1024), (512, 768, 2048), (2048, 2304, 544)])
def test_gemm_gemm_order_oracle(orc, m, n, k):
    note(f"gemm gemm-order vs oracle {m}x{n}x{k}")
    A, SA = _operand(m, k, 21, True)
    B, SB = _operand(n, k, 22, True)
    got = fp4.gemm(A, SA, B, SB, a_gemm_scales=True, b_gemm_scales=True)
    torch.cuda.synchronize()
    ac, bc = A.cpu().numpy(), B.cpu().numpy()
    # the row-major scales, read back from the GEMM order
    def rows_of(S, rows):
        s = S.cpu().numpy()
        r = np.arange(rows)[:, None]
        b = np.arange(k // 32)[None, :]
        return np.ascontiguousarray(s[r // 32, (b // 8) * 256 + (r % 32) * 8 + b % 8])
    as_, bs = rows_of(SA, m), rows_of(SB, n)
    want = orc.gemm_f64(ac, as_, bc, bs)
    a = np.abs(orc.dequantize_f64(ac, as_, 0))
    b = np.abs(orc.dequantize_f64(bc, bs, 0))
    tol = 2.0 ** -22 * (k / 64 + 1) * (a @ b.T)
    err = np.abs(got.cpu().numpy().astype(np.float64) - want)
    assert np.all(err <= tol), f"max err {err.max()}"
