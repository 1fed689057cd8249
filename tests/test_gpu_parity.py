"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Without rotation codes, scales, tensor scales and dequantized bf16 must match
bit for bit. With rotation the tolerances in parity_util apply.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_scaled_fp4_absmax_amd as fp4
from block_scaled_fp4_absmax_amd import inputs
from parity_util import (bf16_bits, check_rotated, check_rotated_rows, note, same_bf16,
                         to_dev, unpack)

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


# -------------------------------------------------------------------- MXFP4 --
def test_mx_c1_bitexact(orc):
    note("case: MXFP4 256x4096 quantize + dequantize (seed 0)")
    x = inputs.gen_c1()
    c, s, _ = fp4.quantize(to_dev(x), fp4.MXFP4)
    d = fp4.dequantize(c, s, fp4.MXFP4)
    sync()
    oc, os_ = orc.mx_quantize(x)
    assert np.array_equal(np_u8(s), os_)
    assert np.array_equal(np_u8(c), oc)
    assert np.array_equal(bf16_bits(d), orc.dequantize(oc, os_, 0))


def exhaustive_mx_tensor():
    """Blocks pairing every finite bf16 pattern with an anchor for every
    reachable E8M0 exponent (anchor 6*2^e, or the largest bf16)."""
    pats = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        f = (pats << 16).view(np.float32)
    mag = np.abs(f.astype(np.float64))
    finite = np.isfinite(f)
    blocks = []
    for e in range(-127, 127):
        top = 6.0 * 2.0 ** e
        anchor_f = np.float32(min(top, 3.3895313892515355e38))
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
def test_mx_exhaustive_bf16_patterns(orc, floor_rule):
    x = exhaustive_mx_tensor()
    # add blocks holding Inf / NaN
    x[0, 3] = 0x7F80
    x[1, 40] = 0xFFC1
    note(f"case: MXFP4 exhaustive bf16 x exponent sweep {x.shape} floor={floor_rule}")
    c, s, _ = fp4.quantize(to_dev(x), fp4.MXFP4, floor_rule=floor_rule)
    sync()
    oc, os_ = orc.mx_quantize(x, floor_rule)
    assert np.array_equal(np_u8(s), os_)
    assert np.array_equal(np_u8(c), oc)


@pytest.mark.parametrize("fmt,razer", [(0, False), (1, False), (1, True), (2, False)])
def test_dequant_every_code_and_scale(orc, fmt, razer):
    note(f"case: dequantize every code x scale byte fmt={fmt} razer={razer}")
    blk = 16 if fmt == 1 else 32
    rows, cols = 256, 512
    codes = np.tile(np.arange(256, dtype=np.uint8), (rows, 1))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], cols // blk, axis=1)
    ts = np.float32(0.37109375) if fmt == 1 else np.float32(1.0)
    tst = torch.tensor([ts], device="cuda")
    d = fp4.dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), fmt,
                       fp4.RAZER if razer else fp4.PLAIN, tst if fmt == 1 else None)
    sync()
    want = orc.dequantize(codes, scales, fmt, razer, float(ts))
    assert same_bf16(bf16_bits(d), want)


# -------------------------------------------------------------------- NVFP4 --
@pytest.mark.parametrize("razer", [True, False])
def test_nv_c2_bitexact(orc, razer):
    note(f"case: NVFP4 4096x4096 razer={razer} (seed 1)")
    x = inputs.gen_c2()
    mode = fp4.RAZER if razer else fp4.PLAIN
    c, s, ts = fp4.quantize(to_dev(x), fp4.NVFP4, mode)
    d = fp4.dequantize(c, s, fp4.NVFP4, mode, ts)
    sync()
    oc, os_, ots = orc.nv_quantize(x, razer)
    assert np.float32(ts.cpu().numpy()[0]).view(np.uint32) == np.float32(ots).view(np.uint32)
    assert np.array_equal(np_u8(s), os_)
    assert np.array_equal(np_u8(c), oc)
    assert np.array_equal(bf16_bits(d), orc.dequantize(oc, os_, 1, razer, ots))
    if razer:
        u = unpack(oc)
        assert (u == 8).sum() > 1000 and (os_ >> 7).sum() > 100


@pytest.mark.parametrize("shrink", [1.0, 0.25, 1e-3])
def test_nv_given_tensor_scale_saturates(orc, shrink):
    """A caller-given s_t smaller than amax/2688 saturates block scales at 448
    and elements at 6, including scaled values far above 16."""
    note(f"case: NVFP4 RaZeR with given tensor scale x{shrink}")
    x = inputs.gen_c2(rows=256, cols=2048)
    st = np.float32(orc.nv_tensor_scale(orc.nv_tensor_amax(x)) * shrink)
    tst = torch.tensor([st], device="cuda")
    c, s, _ = fp4.quantize(to_dev(x), fp4.NVFP4, fp4.RAZER, tensor_scale=tst)
    sync()
    oc, os_, _ = orc.nv_quantize(x, True, float(st))
    assert np.array_equal(np_u8(s), os_)
    assert np.array_equal(np_u8(c), oc)
    assert float(tst.cpu()[0]) == float(st)  # the given scale is left untouched


def test_nv_edge_cases(orc):
    rows, cols = 8, 64
    x = np.zeros((rows, cols), np.uint16)  # all-zero tensor: s_t = 1, codes 0
    note("case: NVFP4 all-zero tensor")
    c, s, ts = fp4.quantize(to_dev(x), fp4.NVFP4, fp4.RAZER)
    sync()
    assert float(ts.cpu()[0]) == 1.0 and not np_u8(c).any() and not np_u8(s).any()
    # blocks whose E4M3 scale rounds to zero, negative zeros, tiny values
    f = np.zeros((rows, cols), np.float32)
    f[0, 0] = 3.0e4
    f[1, :16] = 1e-3
    f[2, :16] = -1e-9
    f[3, 16:32] = -0.0
    f[4, :] = np.linspace(-5.4, 5.4, cols) * 1e2
    x = inputs.f64_to_bf16_bits(f.astype(np.float64))
    for razer in (False, True):
        note(f"case: NVFP4 edge blocks razer={razer}")
        c, s, ts = fp4.quantize(to_dev(x), fp4.NVFP4, fp4.RAZER if razer else fp4.PLAIN)
        sync()
        oc, os_, ots = orc.nv_quantize(x, razer)
        assert float(ts.cpu()[0]) == ots
        assert np.array_equal(np_u8(s), os_) and np.array_equal(np_u8(c), oc)
    # empty tensor with a computed scale still writes s_t = 1
    note("case: NVFP4 empty tensor")
    ts = torch.full((1,), 7.0, device="cuda")
    st = fp4.lib().fp4_quantize(None, 0, 64, 64, 1, 16, 1, 0, None, 32, None, 4,
                                ts.data_ptr(), None)
    sync()
    assert st == 0 and float(ts.cpu()[0]) == 1.0


# ------------------------------------------------------ layouts and shapes ---
@pytest.mark.parametrize("fmt,razer", [(0, False), (1, False), (1, True), (2, False)])
@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 96), (33, 160), (129, 4128)])
def test_strided_ragged(orc, fmt, razer, rows, cols):
    """Row strides larger than the row, odd row counts, rows that are not a
    multiple of the work-group footprint."""
    blk = 16 if fmt == 1 else 32
    if cols % blk:
        pytest.skip("cols not a multiple of the block")
    note(f"case: strided fmt={fmt} razer={razer} {rows}x{cols}")
    x_full = inputs.gen_c2(rows=rows, cols=cols + 24, seed=rows)
    xt = to_dev(x_full)[:, :cols]
    x = np.ascontiguousarray(x_full[:, :cols])
    cbuf = torch.full((rows, cols // 2 + 12), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((rows, cols // blk + 5), 0xCD, dtype=torch.uint8, device="cuda")
    c, s = cbuf[:, :cols // 2], sbuf[:, :cols // blk]
    mode = fp4.RAZER if razer else fp4.PLAIN
    _, _, ts = fp4.quantize(xt, fmt, mode, codes=c, scales=s)
    obuf = torch.zeros((rows, cols + 8), dtype=torch.bfloat16, device="cuda")
    fp4.dequantize(c, s, fmt, mode, ts, out=obuf[:, :cols])
    sync()
    if fmt == 0:
        oc, os_ = orc.mx_quantize(x)
        od = orc.dequantize(oc, os_, 0)
    elif fmt == 2:
        oc, os_ = orc.mxint4_quantize(x)
        od = orc.dequantize(oc, os_, 2)
    else:
        oc, os_, ots = orc.nv_quantize(x, razer)
        assert float(ts.cpu()[0]) == ots
        od = orc.dequantize(oc, os_, 1, razer, ots)
    assert np.array_equal(np_u8(c), oc) and np.array_equal(np_u8(s), os_)
    assert np.all(np_u8(cbuf)[:, cols // 2:] == 0xAB) and np.all(np_u8(sbuf)[:, cols // blk:] == 0xCD)
    assert np.array_equal(bf16_bits(obuf[:, :cols]), od)
    assert not bf16_bits(obuf[:, cols:]).any()


def test_deterministic():
    x = to_dev(inputs.gen_c2(rows=512, cols=4096))
    note("case: determinism, two identical calls")
    a = fp4.quantize(x, fp4.NVFP4, fp4.RAZER)
    b = fp4.quantize(x, fp4.NVFP4, fp4.RAZER)
    r1 = fp4.rotate_quantize(x, None, 32, want_rotated=True)
    r2 = fp4.rotate_quantize(x, None, 32, want_rotated=True)
    sync()
    for p, q in zip(a, b):
        assert torch.equal(p, q)
    for p, q in zip(r1, r2):
        assert torch.equal(p, q)


# ---------------------------------------------------------------- rotation --
def _rot_case(orc, x, perm, had):
    pt = None if perm is None else torch.from_numpy(perm).cuda()
    c, s, y = fp4.rotate_quantize(to_dev(x), pt, had, want_rotated=True)
    sync()
    oc, os_, oy = orc.rotate_quantize(x, perm, had)
    return check_rotated(y.cpu().numpy(), oy, np_u8(c), np_u8(s), oc, os_)


def test_rotate_hadamard_c3_small(orc):
    note("case: MXFP4 + H32, 512x8192 Student-t(3) with outlier channels")
    x = inputs.gen_c3(rows=512)
    r = _rot_case(orc, x, None, 32)
    note(f"  {r}")


def test_rotate_identity_matches_plain(orc):
    """With no permutation and no Hadamard the fused kernel is plain MXFP4."""
    x = inputs.gen_c1(rows=64, cols=1024)
    note("case: rotate_quantize(identity) vs oracle plain MXFP4")
    c, s, y = fp4.rotate_quantize(to_dev(x), None, 0, want_rotated=True)
    sync()
    oc, os_ = orc.mx_quantize(x)
    assert np.array_equal(np_u8(c), oc) and np.array_equal(np_u8(s), os_)
    assert np.array_equal(y.cpu().numpy(), inputs.bf16_bits_to_f32(x))


@pytest.mark.parametrize("had", [32, 0])
def test_rotate_two_level_c4_small(orc, had):
    note(f"case: permutation + H{had}, 1024x8192 log-normal block variances")
    x = inputs.gen_c4(rows=1024)
    e_gpu = fp4.channel_energy(to_dev(x))
    sync()
    e_orc = orc.channel_energy(x)
    assert np.allclose(e_gpu.cpu().numpy(), e_orc, rtol=1e-6, atol=0)
    perm = orc.build_perm(e_orc.astype(np.float32), 32)
    assert np.array_equal(fp4.build_permutation(e_gpu).numpy(),
                          orc.build_perm(e_gpu.cpu().numpy(), 32))
    r = _rot_case(orc, x, perm, had)
    note(f"  {r}")


@pytest.mark.parametrize("group", [2, 4, 8])
def test_rotate_grouped_permutation(orc, group):
    """Permutations of aligned channel runs take the wide-gather path."""
    note(f"case: permutation of {group}-channel runs + H32, 512x8192")
    x = inputs.gen_c4(rows=512)
    e = orc.channel_energy(x).astype(np.float32)
    perm = orc.build_perm(e, 32, group)
    host = fp4.build_permutation(torch.from_numpy(e), 32, group).numpy()
    assert np.array_equal(host, perm)
    r = _rot_case(orc, x, perm, 32)
    note(f"  {r}")
    # one swap breaks the 8/4-alignment: the kernel must fall back, not misread
    bad = perm.copy()
    bad[[0, 2]] = bad[[2, 0]]
    _rot_case(orc, x, bad, 32)


# cols 96 .. 16384 cover one to four MFMA tiles per wave per row (partial
# tiles at 2080 and 8224; 4128 and 5152 leave waves of the eight-wave
# work-group without a block); 1537 and 2500 rows give work-groups unequal row
# counts, odd and even, in the row-at-a-time permuting kernel
@pytest.mark.parametrize("rows,cols", [(3, 96), (37, 2080), (5, 16384), (6, 8224), (4, 12288),
                                       (1537, 8192), (2500, 1024), (7, 5152), (3, 4128)])
def test_rotate_ragged(orc, rows, cols):
    note(f"case: rotate ragged {rows}x{cols}")
    x = inputs.gen_c3(rows=rows, cols=cols)
    perm = np.random.default_rng(cols).permutation(cols).astype(np.int32)
    _rot_case(orc, x, perm, 32)
    _rot_case(orc, x, None, 32)
    runs = np.random.default_rng(cols + 1).permutation(cols // 8).astype(np.int32)
    perm8 = (8 * runs[:, None] + np.arange(8)[None, :]).reshape(-1).astype(np.int32)
    _rot_case(orc, x, perm8, 32)


# the Hadamard without a permutation streams tiles of 16 blocks, four lanes per
# block: strided rows (the non-flat block geometry), block counts that are not
# a multiple of 16, padded outputs whose guard bytes must stay untouched, both
# scale rules and both MX element grids
@pytest.mark.parametrize("fmt", [fp4.MXFP4, fp4.MXINT4])
@pytest.mark.parametrize("rows,cols,floor_rule", [(7, 96, False), (33, 160, True),
                                                  (129, 4128, False), (5, 8224, True)])
def test_rotate_hadamard_strided(orc, fmt, rows, cols, floor_rule):
    note(f"case: H32 streaming fmt={fmt} strided {rows}x{cols} floor={floor_rule}")
    x_full = inputs.gen_c3(rows=rows, cols=cols + 40, seed=cols)
    xt = to_dev(x_full)[:, :cols]
    x = np.ascontiguousarray(x_full[:, :cols])
    cbuf = torch.full((rows, cols // 2 + 16), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((rows, cols // 32 + 7), 0xCD, dtype=torch.uint8, device="cuda")
    rbuf = torch.full((rows, cols + 8), 7.0, dtype=torch.float32, device="cuda")
    c, s, y = fp4.rotate_quantize(xt, None, 32, floor_rule=floor_rule, fmt=fmt,
                                  codes=cbuf[:, :cols // 2], scales=sbuf[:, :cols // 32],
                                  rotated=rbuf[:, :cols])[:3]
    sync()
    if fmt == fp4.MXFP4:
        oc, os_, oy = orc.rotate_quantize(x, None, 32, floor_rule)
    else:
        oc, os_, oy = orc.rotate_quantize_mxint4(x, None, 32, floor_rule)
    r = check_rotated(y.cpu().numpy(), oy, np_u8(c), np_u8(s), oc, os_)
    note(f"  {r}")
    assert np.all(np_u8(cbuf)[:, cols // 2:] == 0xAB)
    assert np.all(np_u8(sbuf)[:, cols // 32:] == 0xCD)
    assert torch.all(rbuf[:, cols:] == 7.0)
    # the launch without the rotated output gives the same bytes
    c2, s2 = fp4.rotate_quantize(xt, None, 32, floor_rule=floor_rule, fmt=fmt)[:2]
    sync()
    assert torch.equal(c2, c.contiguous()) and torch.equal(s2, s.contiguous())


# rows wider than 16384 take the kernel that stages rows straight into LDS:
# sixteen waves of two MFMA tiles (16416 and 20480 leave waves and tiles
# without a block), one work-group per CU, row counts below, at and above the
# grid
@pytest.mark.parametrize("rows,cols", [(3, 16416), (37, 20480), (5, 24576), (6, 28672),
                                       (2, 32768), (300, 28672), (1100, 28704)])
def test_rotate_wide_rows(orc, rows, cols):
    note(f"case: rotate wide rows {rows}x{cols}")
    x = inputs.gen_c4(rows=rows, cols=cols)
    perm = np.random.default_rng(cols + rows).permutation(cols).astype(np.int32)
    r = _rot_case(orc, x, perm, 32)
    note(f"  {r}")
    runs = np.random.default_rng(cols + 1).permutation(cols // 8).astype(np.int32)
    perm8 = (8 * runs[:, None] + np.arange(8)[None, :]).reshape(-1).astype(np.int32)
    _rot_case(orc, x, perm8, 32)
    _rot_case(orc, x, perm, 0)


@pytest.mark.timeout(900)
def test_rotate_down_projection_input_full(orc):
    """The two-level rotation on activations entering the 28672-wide down
    projection: 8192 tokens x 28672 channels with log-normal block variances,
    permutation from the tensor's own channel energies, whole tensor."""
    note("case: permutation + H32 + MXFP4, 8192x28672 activations, whole tensor vs oracle")
    x = inputs.gen_c4(rows=8192, cols=28672)
    xt = to_dev(x)
    perm = fp4.build_permutation(fp4.channel_energy(xt)).numpy()
    pt = torch.from_numpy(perm).cuda()
    c, s, y = fp4.rotate_quantize(xt, pt, 32, want_rotated=True)
    c0, s0, _ = fp4.rotate_quantize(xt, pt, 32)
    sync()
    assert torch.equal(c, c0) and torch.equal(s, s0)
    del xt, c0, s0
    oc, os_, oy = orc.rotate_quantize(x, perm, 32)
    r = check_rotated_rows(y, oy, np_u8(c), np_u8(s), oc, os_)
    note(f"  {r}")


def _unrotate_case(orc, x, perm, had):
    pt = None if perm is None else torch.from_numpy(perm).cuda()
    c, s, _ = fp4.rotate_quantize(to_dev(x), pt, had)
    d = fp4.dequantize(c, s, fp4.MXFP4, perm=pt, hadamard=had)
    sync()
    yh = orc.dequantize_f64(np_u8(c), np_u8(s), 0)
    want = orc.unrotate_f64(yh, perm, had)
    got = inputs.bf16_bits_to_f32(bf16_bits(d)).astype(np.float64)
    rowmax = np.abs(want).max(1, keepdims=True)
    # one bf16 rounding of the fp32 result (exact sums, one fp32 scaling)
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-6 * rowmax)
    return got


def _perm_of(kind, cols, seed):
    rng = np.random.default_rng(seed)
    if kind is None:
        return None
    if kind == 1:
        return rng.permutation(cols).astype(np.int32)
    runs = rng.permutation(cols // kind).astype(np.int32)
    return (kind * runs[:, None] + np.arange(kind)[None, :]).reshape(-1).astype(np.int32)


@pytest.mark.parametrize("perm_on", [False, True])
def test_dequant_unrotate(orc, perm_on):
    note(f"case: dequantize with inverse rotation perm={perm_on}")
    x = inputs.gen_c4(rows=256, cols=4096)
    perm = np.random.default_rng(5).permutation(4096).astype(np.int32) if perm_on else None
    got = _unrotate_case(orc, x, perm, 32)
    # and the round trip is close to the input (SQNR of the two-level path)
    sq = orc.sqnr_db(inputs.bf16_bits_to_f32(x), got)
    note(f"  round-trip SQNR {sq:.2f} dB")
    assert sq > 15


# one to four MFMA tiles per wave per row (partial tiles at 96, 2080, 8224),
# many rows per work-group (1537), aligned channel runs (wider LDS scatters),
# the permutation alone, and the Hadamard alone
@pytest.mark.parametrize("rows,cols,kind,had", [
    (3, 96, 1, 32), (37, 2080, 1, 32), (6, 8224, 1, 32), (5, 16384, 1, 32), (4, 12288, 1, 32),
    (1537, 8192, 1, 32), (2500, 1024, 1, 32), (300, 8192, 2, 32), (300, 8192, 4, 32),
    (300, 8192, 8, 32), (300, 8192, 1, 0), (1537, 8192, None, 32), (37, 2080, None, 32),
    (7, 5152, 1, 32), (7, 5152, None, 32), (3, 4128, None, 32)])
def test_dequant_unrotate_shapes(orc, rows, cols, kind, had):
    note(f"case: dequantize + inverse rotation {rows}x{cols} perm runs={kind} H{had}")
    x = inputs.gen_c3(rows=rows, cols=cols)
    _unrotate_case(orc, x, _perm_of(kind, cols, cols + rows), had)


# ------------------------------------------------------- full-size configs --
# Whole tensors against the oracle. The rotated configurations are launched
# twice: with the rotated values written out (for the value tolerance) and in
# the configuration that bench.py times (codes and scales only); the two must
# agree bit for bit, and their codes meet the rotated-path tolerance.


@pytest.mark.timeout(900)
def test_c3_full_size(orc):
    note("case: C3 full 8192x8192 MXFP4 + H32, whole tensor vs oracle")
    x = inputs.gen_c3()
    xt = to_dev(x)
    c, s, y = fp4.rotate_quantize(xt, None, 32, want_rotated=True)
    c0, s0, _ = fp4.rotate_quantize(xt, None, 32)
    sync()
    assert torch.equal(c, c0) and torch.equal(s, s0)
    del xt, c0, s0
    oc, os_, oy = orc.rotate_quantize(x, None, 32)
    r = check_rotated_rows(y, oy, np_u8(c), np_u8(s), oc, os_)
    note(f"  {r}")


@pytest.mark.timeout(900)
def test_c4_full_size(orc):
    note("case: C4 full 16384x8192 energy + permutation + H32, whole tensor vs oracle")
    x = inputs.gen_c4()
    xt = to_dev(x)
    e_gpu = fp4.channel_energy(xt)
    sync()
    e_orc = orc.channel_energy(x)
    assert np.allclose(e_gpu.cpu().numpy(), e_orc, rtol=1e-6, atol=0)
    perm = fp4.build_permutation(e_gpu).numpy()
    pt = torch.from_numpy(perm).cuda()
    c, s, y = fp4.rotate_quantize(xt, pt, 32, want_rotated=True)
    c0, s0, _ = fp4.rotate_quantize(xt, pt, 32)
    sync()
    assert torch.equal(c, c0) and torch.equal(s, s0)
    del xt, c0, s0
    oc, os_, oy = orc.rotate_quantize(x, perm, 32)
    r = check_rotated_rows(y, oy, np_u8(c), np_u8(s), oc, os_)
    note(f"  {r}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("t", range(7))
def test_c5_layer_sweep_full(orc, t):
    """Every tensor of the layer bit for bit: codes, scale bytes, s_t and the
    decoded bf16, with s_t computed (amax pass) and with s_t given."""
    name, R, C = inputs.C5_SHAPES[t]
    note(f"case: C5 {name} {R}x{C} NVFP4+RaZeR round trip, whole tensor vs oracle")
    x = inputs.gen_c5(t)
    xt = to_dev(x)
    c, s, ts = fp4.quantize(xt, fp4.NVFP4, fp4.RAZER)
    d = fp4.dequantize(c, s, fp4.NVFP4, fp4.RAZER, ts)
    c2, s2, _ = fp4.quantize(xt, fp4.NVFP4, fp4.RAZER, tensor_scale=ts.clone())
    sync()
    del xt
    ots = orc.nv_tensor_scale(orc.nv_tensor_amax(x))
    assert float(ts.cpu()[0]) == ots
    oc, os_, _ = orc.nv_quantize(x, True, ots)
    assert np.array_equal(np_u8(s), os_) and np.array_equal(np_u8(c), oc)
    assert np.array_equal(np_u8(s2), os_) and np.array_equal(np_u8(c2), oc)
    del c2, s2
    assert np.array_equal(bf16_bits(d), orc.dequantize(oc, os_, 1, True, ots))
