"""GPU parity of MXINT4 (plain, rotated, and the inverse rotation on decode).

"TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization" (technical
summary, the generalisation remark of its results) names an MXINT4 grid; the
format read here is the 4-bit microscaling integer element (two's complement
k / 4, 32-element blocks, E8M0 scale), as the oracle defines it.

Plain quantization and decoding are bit-exact. The rotated path is held to
two bars: the rotated fp32 values within 1e-5 of the block amax of the
oracle's dense product, codes and scales bit-exact with the oracle's MXINT4
quantizer applied to the kernels' own rotated values, and at most 1e-4 of
codes differing from the oracle run end to end (a differing scale byte counts
as its whole block).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_scaled_fp4_absmax_amd as fp4
from block_scaled_fp4_absmax_amd import inputs
from parity_util import ROT_CODE_FRAC, ROT_REL, bf16_bits, note, same_bf16, to_dev, unpack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp4.lib()


def np_u8(t):
    return t.cpu().numpy()


def _signed(nib):
    return (np.asarray(nib, np.uint8) << 4).astype(np.int8) >> 4


def test_mxint4_c1_bitexact(orc):
    note("case: MXINT4 256x4096 quantize + dequantize (seed 0)")
    x = inputs.gen_c1()
    c, s, _ = fp4.quantize(to_dev(x), fp4.MXINT4)
    d = fp4.dequantize(c, s, fp4.MXINT4)
    torch.cuda.synchronize()
    oc, os_ = orc.mxint4_quantize(x)
    assert np.array_equal(np_u8(s), os_)
    assert np.array_equal(np_u8(c), oc)
    assert np.array_equal(bf16_bits(d), orc.dequantize(oc, os_, 2))


def exhaustive_int_tensor():
    """Blocks pairing every finite bf16 pattern with an anchor for every
    reachable exponent (anchor 1.75 * 2^e, or the largest bf16)."""
    pats = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        f = (pats << 16).view(np.float32)
    mag = np.abs(f.astype(np.float64))
    finite = np.isfinite(f)
    blocks = []
    for e in range(-127, 128):
        anchor_f = np.float32(min(1.75 * 2.0 ** e, 3.3895313892515355e38))
        anchor = np.uint16(anchor_f.view(np.uint32) >> 16)
        a = float((np.uint32(anchor) << 16).view(np.float32))
        members = pats[finite & (mag <= a)].astype(np.uint16)
        nblk = -(-members.size // 31)
        body = np.zeros(nblk * 31, np.uint16)
        body[:members.size] = members
        body = body.reshape(nblk, 31)
        sign = np.where(np.arange(nblk) % 2 == 0, 0, 0x8000).astype(np.uint16)[:, None]
        blocks.append(np.concatenate([anchor | sign, body], axis=1))
    allb = np.concatenate(blocks)
    pad = (-allb.shape[0]) % 32
    allb = np.concatenate([allb, np.zeros((pad, 32), np.uint16)])
    return allb.reshape(-1, 1024)


@pytest.mark.parametrize("floor_rule", [False, True])
def test_mxint4_exhaustive_bf16_patterns(orc, floor_rule):
    x = exhaustive_int_tensor()
    x[0, 3] = 0x7F80   # +Inf block
    x[1, 40] = 0xFFC1  # NaN block
    note(f"case: MXINT4 exhaustive bf16 x exponent sweep {x.shape} floor={floor_rule}")
    c, s, _ = fp4.quantize(to_dev(x), fp4.MXINT4, floor_rule=floor_rule)
    d = fp4.dequantize(c, s, fp4.MXINT4)
    torch.cuda.synchronize()
    oc, os_ = orc.mxint4_quantize(x, floor_rule)
    assert np.array_equal(np_u8(s), os_)
    assert np.array_equal(np_u8(c), oc)
    assert same_bf16(bf16_bits(d), orc.dequantize(oc, os_, 2))


def test_mxint4_edge_cases(orc):
    note("case: MXINT4 zeros, subnormals, saturation at the top exponent, empty")
    f = np.zeros((6, 64), np.float64)
    f[1, :32] = 2.0 ** -130                       # subnormal block maximum
    f[2, :32] = np.linspace(-1, 1, 32) * 2.0 ** -127
    f[3, :32] = 3.0e38                            # above 1.75 * 2^127: saturates
    f[3, 32:] = -3.0e38
    f[4, :] = np.linspace(-1.9, 1.9, 64)
    f[5, 5] = -0.0
    x = inputs.f64_to_bf16_bits(f)
    for floor_rule in (False, True):
        c, s, _ = fp4.quantize(to_dev(x), fp4.MXINT4, floor_rule=floor_rule)
        torch.cuda.synchronize()
        oc, os_ = orc.mxint4_quantize(x, floor_rule)
        assert np.array_equal(np_u8(s), os_) and np.array_equal(np_u8(c), oc)
    st = fp4.lib().fp4_quantize(None, 0, 64, 64, 2, 32, 0, 0, None, 32, None, 2, None, None)
    assert st == 0


# ---------------------------------------------------------------- rotation --
def _check_int(orc, x, perm, had, floor_rule=False):
    pt = None if perm is None else torch.from_numpy(perm).cuda()
    c, s, y = fp4.rotate_quantize(to_dev(x), pt, had, floor_rule=floor_rule, want_rotated=True,
                                  fmt=fp4.MXINT4)
    c2, s2, _ = fp4.rotate_quantize(to_dev(x), pt, had, floor_rule=floor_rule, fmt=fp4.MXINT4)
    torch.cuda.synchronize()
    c, s, y = np_u8(c), np_u8(s), y.cpu().numpy()
    assert np.array_equal(np_u8(c2), c) and np.array_equal(np_u8(s2), s)
    oc, os_, oy = orc.rotate_quantize_mxint4(x, perm, had, floor_rule)
    rows, cols = x.shape
    yo = oy.astype(np.float64).reshape(rows, cols // 32, 32)
    yg = y.astype(np.float64).reshape(rows, cols // 32, 32)
    amax = np.abs(yo).max(-1)
    assert np.all(np.abs(yg - yo) <= ROT_REL * np.maximum(amax, 1e-30)[..., None])
    sc, ss = orc.mxint4_quantize_f32(y, floor_rule)
    assert np.array_equal(s, ss) and np.array_equal(c, sc)
    bad_blk = s != os_
    ug = unpack(c).reshape(rows, cols // 32, 32)
    uo = unpack(oc).reshape(rows, cols // 32, 32)
    n_codes = int(((ug != uo) & ~bad_blk[..., None]).sum())
    n_bad = n_codes + 32 * int(bad_blk.sum())
    if had == 0:
        assert n_bad == 0 and np.array_equal(y, oy)
    assert n_bad <= ROT_CODE_FRAC * rows * cols, f"{n_bad} of {rows * cols} codes differ"
    return {"codes_differ": n_codes, "blocks_differ": int(bad_blk.sum())}


def test_mxint4_hadamard_c3_small(orc):
    note("case: MXINT4 + H32, 512x8192 Student-t(3) with outlier channels")
    note(f"  {_check_int(orc, inputs.gen_c3(rows=512), None, 32)}")


@pytest.mark.parametrize("had,floor_rule", [(32, False), (32, True), (0, False)])
def test_mxint4_two_level_c4_small(orc, had, floor_rule):
    note(f"case: MXINT4 permutation + H{had} floor={floor_rule}, 1024x8192")
    x = inputs.gen_c4(rows=1024)
    perm = orc.build_perm(orc.channel_energy(x).astype(np.float32), 32)
    note(f"  {_check_int(orc, x, perm, had, floor_rule)}")


@pytest.mark.parametrize("group", [2, 8])
def test_mxint4_grouped_permutation(orc, group):
    note(f"case: MXINT4 permutation of {group}-channel runs + H32, 512x8192")
    x = inputs.gen_c4(rows=512)
    perm = orc.build_perm(orc.channel_energy(x).astype(np.float32), 32, group)
    _check_int(orc, x, perm, 32)


@pytest.mark.parametrize("rows,cols,use_perm", [
    (3, 96, True), (37, 2080, True), (5, 16384, True), (6, 8224, True), (1537, 8192, True),
    (2500, 1024, True), (37, 2080, False), (1, 32, False), (9, 28672, True)])
def test_mxint4_rotation_ragged(orc, rows, cols, use_perm):
    note(f"case: MXINT4 rotate ragged {rows}x{cols} perm={use_perm} H32")
    x = inputs.gen_c3(rows=rows, cols=cols)
    perm = np.random.default_rng(cols).permutation(cols).astype(np.int32) if use_perm else None
    _check_int(orc, x, perm, 32)


@pytest.mark.parametrize("rows,cols,kind,had", [
    (256, 4096, 1, 32), (3, 96, 1, 32), (37, 2080, 1, 32), (5, 16384, 1, 32), (1537, 8192, 1, 32),
    (300, 8192, 4, 32), (300, 8192, 1, 0), (1537, 8192, None, 32), (7, 5152, 1, 32),
    (7, 5152, None, 32)])
def test_mxint4_dequant_unrotate(orc, rows, cols, kind, had):
    note(f"case: MXINT4 dequantize + inverse rotation {rows}x{cols} perm runs={kind} H{had}")
    x = inputs.gen_c3(rows=rows, cols=cols)
    rng = np.random.default_rng(cols + rows)
    if kind is None:
        perm = None
    else:
        runs = rng.permutation(cols // kind).astype(np.int32)
        perm = (kind * runs[:, None] + np.arange(kind)[None, :]).reshape(-1).astype(np.int32)
    pt = None if perm is None else torch.from_numpy(perm).cuda()
    c, s, _ = fp4.rotate_quantize(to_dev(x), pt, had, fmt=fp4.MXINT4)
    d = fp4.dequantize(c, s, fp4.MXINT4, perm=pt, hadamard=had)
    torch.cuda.synchronize()
    want = orc.unrotate_f64(orc.dequantize_f64(np_u8(c), np_u8(s), 2), perm, had)
    got = inputs.bf16_bits_to_f32(bf16_bits(d)).astype(np.float64)
    rowmax = np.abs(want).max(1, keepdims=True)
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-6 * rowmax)
    if had == 0:
        plain = orc.dequantize(np_u8(c), np_u8(s), 2)
        inv = np.empty_like(plain)
        inv[:, perm] = plain
        assert np.array_equal(bf16_bits(d), inv)
    if rows == 256:
        sq = orc.sqnr_db(inputs.bf16_bits_to_f32(x), got)
        note(f"  round-trip SQNR {sq:.2f} dB")
        assert sq > 15


def test_mxint4_dequant_hadamard_all_scale_bytes(orc):
    # Every scale byte 0..255 on its own blocks, with every code -8..7 (the
    # quantizer writes -7..7; -8 is a valid code): the bytes 6..254 take the
    # scale after the Hadamard, 0..5 before it, 255 is NaN. Compared with the
    # oracle's exact result rounded to bf16 (fp32, then bf16, nearest-even):
    # where that overflows the GPU value must be the same infinity, elsewhere
    # finite and within one bf16 rounding (plus fp32 rounding of tiny sums).
    note("case: MXINT4 dequantize + H32, scale bytes 0..255, codes -8..7")
    rng = np.random.default_rng(241)
    nbytes = 256
    rows, cols = 6, 32 * nbytes
    k = rng.integers(-8, 8, size=(rows, cols))
    k[0, :] = np.where(np.arange(cols) % 32 == 0, -8, 0)  # a lone -8 per block
    k[1, :] = 7      # constant blocks: the largest sums
    nib = (k & 0xF).astype(np.uint8)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = np.tile(np.arange(nbytes, dtype=np.uint8), (rows, 1))
    d = fp4.dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                       fp4.MXINT4, perm=None, hadamard=32)
    torch.cuda.synchronize()
    fin = np.arange(cols) < 32 * 255
    vals = np.ldexp(k.astype(np.float64), np.repeat(np.arange(nbytes), 32)[None, :] - 129)
    want = orc.unrotate_f64(np.where(fin, vals, 0.0), None, 32)
    gb = bf16_bits(d)
    got = inputs.bf16_bits_to_f32(gb).astype(np.float64)
    assert np.all(np.isnan(got[:, ~fin])), "scale byte 0xFF decodes to NaN"
    with np.errstate(over="ignore"):
        want_b = inputs.bf16_bits_to_f32(inputs.f64_to_bf16_bits(want)).astype(np.float64)
    g, w, wb = got[:, fin], want[:, fin], want_b[:, fin]
    inf = np.isinf(wb)
    assert inf.sum() > 0 and (~inf).sum() > 0
    assert np.array_equal(g[inf], wb[inf]), "an overflowing result is not the same infinity"
    assert np.all(np.isfinite(g[~inf])), "a finite result came out infinite"
    blockmax = np.repeat(np.abs(w).reshape(rows, 255, 32).max(2), 32, axis=1)
    tol = 2.0 ** -8 * np.abs(w) + 2.0 ** -20 * np.where(np.isinf(blockmax), 0, blockmax) \
        + 2.0 ** -133
    err = np.abs(g - w)
    ok = err[~inf] <= tol[~inf]
    assert np.all(ok), f"{(~ok).sum()} results off by more than one bf16 rounding"
