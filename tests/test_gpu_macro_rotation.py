"""GPU parity of the inter-block Givens transform and the full two-level path.

"TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization", technical
summary sec. 2(a) (an orthogonal transform from Givens rotations that makes
the block variances equal) and 2(b) (the learned rotation inside each block).
The kernel's rows match the oracle's fp64 rotations to one bf16 rounding plus
the fp32 error of the rotations; channels no rotation touches are moved
exactly.
"""
import numpy as np
import pytest

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


def _random_layers(cols, n_layers, per_layer, seed):
    """Layers of disjoint random pairs with random angles (fp32 cos, sin)."""
    rng = np.random.default_rng(seed)
    pairs, cs, starts = [], [], [0]
    for _ in range(n_layers):
        ch = rng.permutation(cols)[:2 * per_layer].reshape(-1, 2)
        th = rng.uniform(-np.pi, np.pi, len(ch))
        pairs.append(ch)
        cs.append(np.stack([np.cos(th), np.sin(th)], 1))
        starts.append(starts[-1] + len(ch))
    return fp4.MacroRotation(torch.from_numpy(np.concatenate(pairs).astype(np.int32)),
                             torch.from_numpy(np.concatenate(cs).astype(np.float32)),
                             torch.tensor(starts, dtype=torch.int32), (0.0, 0.0))


def _check(orc, x, macro, perm, got):
    """got: bf16 bits [rows, cols] from the kernel."""
    pairs = macro.pairs.cpu().numpy()
    cs = macro.cs.cpu().numpy().astype(np.float64)
    want = orc.apply_givens(x, perm, pairs, cs)
    g = inputs.bf16_bits_to_f32(got).astype(np.float64)
    rowmax = np.abs(want).max(1, keepdims=True)
    assert np.all(np.abs(g - want) <= 2.0 ** -8 * np.abs(want) + 1e-6 * rowmax)
    # channels that no rotation touches are the permuted input, bit for bit
    cols = x.shape[1]
    free = np.setdiff1d(np.arange(cols), pairs.reshape(-1))
    src = np.arange(cols) if perm is None else perm
    assert np.array_equal(got[:, free], x[:, src[free]])


@pytest.mark.parametrize("rows,cols,use_perm", [(3, 96, True), (37, 2080, True),
                                                (1537, 8192, True), (5, 16384, False),
                                                (7, 16384, True), (2500, 1024, False),
                                                (2500, 1024, True)])
def test_random_layers(orc, rows, cols, use_perm):
    note(f"case: Givens layers, random disjoint pairs, {rows}x{cols} perm={use_perm}")
    x = inputs.gen_c3(rows=rows, cols=cols)
    perm = np.random.default_rng(cols).permutation(cols).astype(np.int32) if use_perm else None
    macro = _random_layers(cols, 3, min(cols // 4, 300), cols + rows)
    md = macro.to("cuda")
    pt = None if perm is None else torch.from_numpy(perm).cuda()
    z = fp4.apply_channel_rotation(to_dev(x), md, pt)
    sync()
    _check(orc, x, macro, perm, bf16_bits(z))


def test_gather_with_repeats(orc):
    """An index vector that is not a permutation (repeated and missing
    channels) is a gather: every output channel reads its own source."""
    note("case: Givens layers after a gather with repeats, 37x2080")
    rows, cols = 37, 2080
    x = inputs.gen_c3(rows=rows, cols=cols)
    idx = np.random.default_rng(11).integers(0, cols, cols).astype(np.int32)
    macro = _random_layers(cols, 4, 200, 12)
    z = fp4.apply_channel_rotation(to_dev(x), macro.to("cuda"), torch.from_numpy(idx).cuda())
    sync()
    _check(orc, x, macro, idx, bf16_bits(z))


@pytest.mark.parametrize("n_layers,per_layer,cols", [(1, 0, 16384), (8, 500, 16384),
                                                     (2, 100, 8192), (16, 12, 8192),
                                                     (17, 10, 8192)])
def test_rotation_table_sizes(orc, n_layers, per_layer, cols):
    """Table sizes around the compact kernel's limits: no rotation at all (a
    pure permutation); 4000 rotations over 16384 columns, whose tables leave
    no room for it (the row-wide kernel runs them); layers of 100 rotations
    (two register rounds each); 16 rounds, the most wave 0 holds in
    registers, and 17 (its LDS loop)."""
    rows = 9
    note(f"case: Givens layers, {n_layers} x {per_layer} rotations, {rows}x{cols} with perm")
    x = inputs.gen_c4(rows=rows, cols=cols)
    perm = np.random.default_rng(5).permutation(cols).astype(np.int32)
    macro = _random_layers(cols, n_layers, per_layer, 13)
    z = fp4.apply_channel_rotation(to_dev(x), macro.to("cuda"), torch.from_numpy(perm).cuda())
    sync()
    _check(orc, x, macro, perm, bf16_bits(z))


def test_in_place_and_strided(orc):
    note("case: Givens layers in place and on strided rows, 33x2048")
    rows, cols = 33, 2048
    x = inputs.gen_c3(rows=rows, cols=cols)
    md = _random_layers(cols, 2, 200, 5).to("cuda")
    ref = fp4.apply_channel_rotation(to_dev(x), md)
    big = torch.full((rows, cols + 24), 3.0, dtype=torch.bfloat16, device="cuda")
    big[:, :cols] = to_dev(x)
    fp4.apply_channel_rotation(big[:, :cols], md, out=big[:, :cols])
    sync()
    assert torch.equal(big[:, :cols], ref) and bool((big[:, cols:] == 3.0).all())


@pytest.fixture(scope="module")
def c4_case(orc):
    """Log-normal block variances (1024 x 8192): permutation and Givens
    transform calibrated on the first 256 rows."""
    x = inputs.gen_c4(rows=1024)
    xt = to_dev(x)
    perm = fp4.build_permutation(fp4.channel_energy(xt))
    macro = fp4.calibrate_macro_rotation(xt[:256], perm)
    return x, xt, perm, macro


def test_calibrated_transform_equalises_blocks(orc, c4_case):
    x, xt, perm, macro = c4_case
    note(f"case: calibrated Givens transform on C4 rows, {macro.n_rot} rotations in "
         f"{macro.n_layers} layers, spread {macro.spread[0]:.3g} -> {macro.spread[1]:.3g}")
    assert macro.spread[1] <= 1e-5 < macro.spread[0]
    pt = perm.cuda()
    z = fp4.apply_channel_rotation(xt, macro.to("cuda"), pt)
    sync()
    zb = bf16_bits(z)
    rows = np.sort(np.random.default_rng(4).choice(1024, 64, replace=False))
    _check(orc, np.ascontiguousarray(x[rows]), macro, perm.numpy(), zb[rows])
    # block variances of the kernel's (bf16) output on the calibration rows:
    # each element is within 2^-9 |z| of the exact z, so each block's energy
    # is within 2^-8 (plus 2^-18) of the exact, equal, energies
    zf = inputs.bf16_bits_to_f32(zb[:256]).astype(np.float64)
    v = (zf ** 2).sum(0).reshape(-1, 32).sum(1)
    exact = orc.apply_givens(np.ascontiguousarray(x[:256]), perm.numpy(), macro.pairs.numpy(),
                             macro.cs.numpy().astype(np.float64))
    ve = (exact ** 2).sum(0).reshape(-1, 32).sum(1)
    assert (ve.max() - ve.min()) / ve.mean() <= 1e-5
    assert np.all(np.abs(v - ve) <= (2.0 ** -8 + 2.0 ** -18) * ve)
    note(f"  spread of the bf16 output {(v.max() - v.min()) / v.mean():.3g}")


def test_folding_into_weights(orc, c4_case):
    """The same call on the rows of a consumer's weights: W' z = W x up to
    the bf16 rounding of W' and z."""
    x, xt, perm, macro = c4_case
    note("case: Givens transform folded into weight rows, 256 x 8192")
    md = macro.to("cuda")
    pt = perm.cuda()
    w = inputs.gen_c5(0, rows=256, cols=8192)
    wt = fp4.apply_channel_rotation(to_dev(w), md, pt)
    z = fp4.apply_channel_rotation(xt[:64], md, pt)
    sync()
    W = inputs.bf16_bits_to_f32(w).astype(np.float64)
    X = inputs.bf16_bits_to_f32(x[:64]).astype(np.float64)
    Wt = inputs.bf16_bits_to_f32(bf16_bits(wt)).astype(np.float64)
    Z = inputs.bf16_bits_to_f32(bf16_bits(z)).astype(np.float64)
    want = X @ W.T
    got = Z @ Wt.T
    bound = np.abs(X) @ np.abs(W).T
    assert np.all(np.abs(got - want) <= 2.0 ** -7 * bound)


def test_full_two_level_path(orc, c4_case):
    """Permutation + Givens transform (macro), then the learned block matrix
    (micro) fused with MXFP4: rotated values and codes against the oracle on
    the kernel's own macro output, and the round-trip SQNR of each variant."""
    x, xt, perm, macro = c4_case
    pt = perm.cuda()
    z = fp4.apply_channel_rotation(xt, macro.to("cuda"), pt)
    R, _ = fp4.calibrate_block_rotation(z[:256], None, iters=30, angles=32)
    ident = torch.arange(8192, dtype=torch.int32, device="cuda")
    rt = R.cuda()
    c, s, y = fp4.rotate_quantize_r(z, ident, rt, want_rotated=True)
    sync()
    zb = bf16_bits(z)
    rows = np.sort(np.random.default_rng(6).choice(1024, 64, replace=False))
    oc, os_, oy = orc.rotate_quantize_r(np.ascontiguousarray(zb[rows]), None,
                                        R.numpy().astype(np.float64))
    ri = torch.from_numpy(rows).cuda()
    r = check_rotated(y[ri].cpu().numpy(), oy, c[ri].cpu().numpy(), s[ri].cpu().numpy(), oc, os_)
    note(f"case: full two-level path, sampled rows {r}")
    zf = inputs.bf16_bits_to_f32(zb)
    d = fp4.dequantize_r(c, s, ident, rt)
    sq_full = orc.sqnr_db(zf, inputs.bf16_bits_to_f32(bf16_bits(d)))
    ch, sh, _ = fp4.rotate_quantize(z, None, 32)
    dh = fp4.dequantize(ch, sh, perm=None, hadamard=32)
    cp, sp, _ = fp4.rotate_quantize(xt, pt, 32)
    dp = fp4.dequantize(cp, sp, perm=pt, hadamard=32)
    sync()
    sq_gh = orc.sqnr_db(zf, inputs.bf16_bits_to_f32(bf16_bits(dh)))
    sq_ph = orc.sqnr_db(inputs.bf16_bits_to_f32(x), inputs.bf16_bits_to_f32(bf16_bits(dp)))
    note(f"  SQNR dB: perm+H {sq_ph:.2f}, perm+Givens+H {sq_gh:.2f}, perm+Givens+R {sq_full:.2f}")
    assert min(sq_ph, sq_gh, sq_full) > 15
