"""GPU parity of NVFP4 with the two-level rotation (16-point Hadamard).

"TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization" (technical
summary, the generalisation remark of its results) applies the rotation with
NVFP4 too; the quantizer then sees fp32 rotated values, every amax (tensor
scale, block scales, RaZeR choice) taken over them.

Two checks per case:
  * the rotated fp32 values agree with the oracle's dense fp64 product to the
    rotated-path tolerance (1e-5 of the block amax), and the codes, scale
    bytes and tensor scale the kernels produced are bit-exact with the
    oracle's NVFP4 quantizer applied to the kernels' own rotated values;
  * against the oracle run end to end from the bf16 input, at most 1e-4 of
    codes differ (a scale byte or RaZeR choice that differs counts as its
    whole block), and s_t agrees to 1e-5 relative.
Without the Hadamard the rotated values are exact, so everything is
bit-exact with the oracle.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_scaled_fp4_absmax_amd as fp4
from block_scaled_fp4_absmax_amd import inputs
from parity_util import ROT_CODE_FRAC, ROT_REL, bf16_bits, note, to_dev, unpack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp4.lib()


def np_u8(t):
    return t.cpu().numpy()


def _f32_bits(v):
    return np.float32(v).view(np.uint32)


def _run(x, perm, had, razer, st=None, want_rotated=True):
    pt = None if perm is None else torch.from_numpy(perm).cuda()
    tst = None if st is None else torch.tensor([st], dtype=torch.float32, device="cuda")
    mode = fp4.RAZER if razer else fp4.PLAIN
    c, s, y, ts = fp4.rotate_quantize(to_dev(x), pt, had, want_rotated=want_rotated,
                                      fmt=fp4.NVFP4, mode=mode, tensor_scale=tst)
    torch.cuda.synchronize()
    return (np_u8(c), np_u8(s), None if y is None else y.cpu().numpy(),
            float(ts.cpu().numpy()[0]))


def _check_nv(orc, x, perm, had, razer, st=None):
    """Both checks of the module docstring; returns a dict of counts."""
    c, s, y, ts = _run(x, perm, had, razer, st)
    oc, os_, ots, oy = orc.rotate_quantize_nv(x, perm, had, razer, st)
    rows, cols = x.shape
    # rotated values
    yo = oy.astype(np.float64).reshape(rows, cols // 16, 16)
    yg = y.astype(np.float64).reshape(rows, cols // 16, 16)
    amax = np.abs(yo).max(-1)
    assert np.all(np.abs(yg - yo) <= ROT_REL * np.maximum(amax, 1e-30)[..., None]), \
        "rotated values: element error above tolerance"
    if had == 0:
        assert np.array_equal(y, oy)
    # the kernels' quantizer on their own rotated values: bit-exact
    if st is None:
        assert _f32_bits(ts) == _f32_bits(orc.nv_tensor_scale(orc.nv_tensor_amax_f32(y)))
    else:
        assert ts == np.float32(st)
    sc, ss, _ = orc.nv_quantize_f32(y, razer, ts)
    assert np.array_equal(s, ss), "scale bytes differ from the oracle on the same rotated values"
    assert np.array_equal(c, sc), "codes differ from the oracle on the same rotated values"
    # the oracle end to end from x
    assert abs(ts - ots) <= ROT_REL * ots
    bad_blk = s != os_
    ug = unpack(c).reshape(rows, cols // 16, 16)
    uo = unpack(oc).reshape(rows, cols // 16, 16)
    vg = np.where((ug & 7) == 0, 0, ug)  # +0 and -0 are one value
    vo = np.where((uo & 7) == 0, 0, uo)
    n_codes = int(((vg != vo) & ~bad_blk[..., None]).sum())
    n_bad = n_codes + 16 * int(bad_blk.sum())
    if had == 0:
        assert n_bad == 0 and _f32_bits(ts) == _f32_bits(ots)
    assert n_bad <= ROT_CODE_FRAC * rows * cols, f"{n_bad} of {rows * cols} codes differ"
    # the variant that does not write the rotated values gives the same result
    c2, s2, _, ts2 = _run(x, perm, had, razer, st, want_rotated=False)
    assert np.array_equal(c2, c) and np.array_equal(s2, s) and ts2 == ts
    return {"codes_differ": n_codes, "blocks_differ": int(bad_blk.sum()), "s_t": ts}


@pytest.mark.parametrize("razer", [False, True])
def test_nv_hadamard16_c3_small(orc, razer):
    note(f"case: NVFP4 + H16 razer={razer}, 512x8192 Student-t(3) with outlier channels")
    x = inputs.gen_c3(rows=512)
    note(f"  {_check_nv(orc, x, None, 16, razer)}")


@pytest.mark.parametrize("had,razer", [(16, True), (16, False), (0, True)])
def test_nv_two_level_c4_small(orc, had, razer):
    note(f"case: NVFP4 permutation + H{had} razer={razer}, 1024x8192 log-normal block variances")
    x = inputs.gen_c4(rows=1024)
    perm = orc.build_perm(orc.channel_energy(x).astype(np.float32), 16)
    note(f"  {_check_nv(orc, x, perm, had, razer)}")


@pytest.mark.parametrize("shrink", [1.0, 1e-3])
def test_nv_rotation_given_tensor_scale(orc, shrink):
    """A given s_t is used as is (and saturates block scales when small)."""
    note(f"case: NVFP4 + permutation + H16 RaZeR, given tensor scale x{shrink}, 256x4096")
    x = inputs.gen_c4(rows=256, cols=4096)
    perm = np.random.default_rng(11).permutation(4096).astype(np.int32)
    y = orc.rotate(x, perm, 16)
    st = float(np.float32(orc.nv_tensor_scale(orc.nv_tensor_amax_f32(y)) * shrink))
    note(f"  {_check_nv(orc, x, perm, 16, True, st)}")


def test_nv_rotation_identity_is_plain_nvfp4(orc):
    """No permutation and no Hadamard: the fused path is plain NVFP4."""
    note("case: NVFP4 rotate_quantize(identity) vs oracle plain NVFP4, 128x2048")
    x = inputs.gen_c2(rows=128, cols=2048)
    for razer in (False, True):
        c, s, y, ts = _run(x, None, 0, razer)
        oc, os_, ots = orc.nv_quantize(x, razer)
        assert _f32_bits(ts) == _f32_bits(ots)
        assert np.array_equal(s, os_) and np.array_equal(c, oc)
        assert np.array_equal(y, inputs.bf16_bits_to_f32(x))


@pytest.mark.parametrize("group", [2, 4, 8])
def test_nv_rotation_grouped_permutation(orc, group):
    note(f"case: NVFP4 permutation of {group}-channel runs + H16 RaZeR, 512x8192")
    x = inputs.gen_c4(rows=512)
    perm = orc.build_perm(orc.channel_energy(x).astype(np.float32), 16, group)
    note(f"  {_check_nv(orc, x, perm, 16, True)}")


# one to four MFMA tiles per wave per row (partial tiles at 96, 2080, 8224),
# unequal row counts per work-group (1537, 2500), both kernels (perm / none)
@pytest.mark.parametrize("rows,cols,use_perm", [
    (3, 96, True), (37, 2080, True), (5, 16384, True), (6, 8224, True), (4, 12288, True),
    (1537, 8192, True), (2500, 1024, True), (37, 2080, False), (1, 32, False), (3, 96, False),
    (7, 28672, True), (300, 20480, True), (2, 32768, True)])
def test_nv_rotation_ragged(orc, rows, cols, use_perm):
    note(f"case: NVFP4 rotate ragged {rows}x{cols} perm={use_perm} H16 RaZeR")
    x = inputs.gen_c3(rows=rows, cols=cols)
    perm = np.random.default_rng(cols).permutation(cols).astype(np.int32) if use_perm else None
    _check_nv(orc, x, perm, 16, True)


def test_nv_rotation_strided(orc):
    """Row strides beyond the row length (non-flat layout) in every array."""
    note("case: NVFP4 + H16 RaZeR with padded row strides, 40x1024 (no permutation)")
    rows, cols = 40, 1024
    x = inputs.gen_c3(rows=rows, cols=cols)
    xp = np.zeros((rows, cols + 64), np.uint16)
    xp[:, :cols] = x
    xt = to_dev(xp)[:, :cols]
    codes = torch.zeros((rows, cols // 2 + 16), dtype=torch.uint8, device="cuda")[:, :cols // 2]
    scales = torch.zeros((rows, cols // 16 + 8), dtype=torch.uint8, device="cuda")[:, :cols // 16]
    rot = torch.zeros((rows, cols + 32), dtype=torch.float32, device="cuda")[:, :cols]
    fp4.rotate_quantize(xt, None, 16, codes=codes, scales=scales, rotated=rot, fmt=fp4.NVFP4,
                        mode=fp4.RAZER)
    torch.cuda.synchronize()
    c, s, y, ts = _run(x, None, 16, True)
    assert np.array_equal(np_u8(codes), c) and np.array_equal(np_u8(scales), s)
    assert np.array_equal(rot.cpu().numpy(), y)


def test_nv_rotation_empty_gives_unit_scale():
    note("case: NVFP4 rotate_quantize of a 0x64 tensor")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    c, s, _, ts = fp4.rotate_quantize(x, None, 16, fmt=fp4.NVFP4, mode=fp4.RAZER)
    torch.cuda.synchronize()
    assert float(ts.cpu()[0]) == 1.0


# ------------------------------------------------------- inverse rotation --
def _nv_unrotate_case(orc, x, perm, had, razer):
    pt = None if perm is None else torch.from_numpy(perm).cuda()
    mode = fp4.RAZER if razer else fp4.PLAIN
    c, s, _, ts = fp4.rotate_quantize(to_dev(x), pt, had, fmt=fp4.NVFP4, mode=mode)
    d = fp4.dequantize(c, s, fp4.NVFP4, mode, ts, perm=pt, hadamard=had)
    torch.cuda.synchronize()
    st = float(ts.cpu().numpy()[0])
    want = orc.unrotate_f64(orc.dequantize_f64(np_u8(c), np_u8(s), 1, razer, st), perm, had)
    got = inputs.bf16_bits_to_f32(bf16_bits(d)).astype(np.float64)
    rowmax = np.abs(want).max(1, keepdims=True)
    # exact transform of the grid values, one fp32 scaling, one bf16 rounding
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-6 * rowmax)
    if had == 0:  # a pure permutation of plain NVFP4 decoding: bit-exact
        plain = orc.dequantize(np_u8(c), np_u8(s), 1, razer, st)
        inv = np.empty_like(plain)
        inv[:, perm] = plain
        assert np.array_equal(bf16_bits(d), inv)
    return got


@pytest.mark.parametrize("razer", [False, True])
def test_nv_dequant_unrotate_round_trip(orc, razer):
    note(f"case: NVFP4 dequantize with inverse rotation razer={razer}, 256x4096")
    x = inputs.gen_c4(rows=256, cols=4096)
    perm = np.random.default_rng(5).permutation(4096).astype(np.int32)
    got = _nv_unrotate_case(orc, x, perm, 16, razer)
    sq = orc.sqnr_db(inputs.bf16_bits_to_f32(x), got)
    note(f"  round-trip SQNR {sq:.2f} dB")
    assert sq > 15


@pytest.mark.parametrize("rows,cols,kind,had", [
    (3, 96, 1, 16), (37, 2080, 1, 16), (6, 8224, 1, 16), (5, 16384, 1, 16),
    (1537, 8192, 1, 16), (2500, 1024, 1, 16), (300, 8192, 8, 16), (300, 8192, 2, 16),
    (300, 8192, 1, 0), (1537, 8192, None, 16), (37, 2080, None, 16), (7, 5152, 1, 16),
    (7, 5152, None, 16), (3, 4128, 1, 16)])
def test_nv_dequant_unrotate_shapes(orc, rows, cols, kind, had):
    note(f"case: NVFP4 dequantize + inverse rotation {rows}x{cols} perm runs={kind} H{had}")
    x = inputs.gen_c3(rows=rows, cols=cols)
    rng = np.random.default_rng(cols + rows)
    if kind is None:
        perm = None
    else:
        runs = rng.permutation(cols // kind).astype(np.int32)
        perm = (kind * runs[:, None] + np.arange(kind)[None, :]).reshape(-1).astype(np.int32)
    _nv_unrotate_case(orc, x, perm, had, True)
