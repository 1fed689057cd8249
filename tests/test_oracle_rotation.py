"""Pins for the oracle's two-level rotation (CPU only)."""
import numpy as np
import pytest
import scipy.linalg

from block_scaled_fp4_absmax_amd import inputs


def test_hadamard_is_sylvester_orthonormal(orc):
    for n in (16, 32):
        h = orc.hadamard_matrix(n)
        ref = scipy.linalg.hadamard(n) / np.sqrt(n)  # Sylvester construction
        assert np.array_equal(h, ref)
        assert np.abs(h @ h.T - np.eye(n)).max() < 1e-15


def test_rotate_matches_dense_product(orc):
    x = inputs.gen_c3(rows=8, cols=256)
    perm = np.random.default_rng(0).permutation(256).astype(np.int32)
    y = orc.rotate(x, perm, 32)
    xf = inputs.bf16_bits_to_f32(x).astype(np.float64)[:, perm]
    h = scipy.linalg.hadamard(32) / np.sqrt(32)
    ref = (xf.reshape(8, 8, 32) @ h.T).reshape(8, 256)
    assert np.array_equal(y, ref.astype(np.float32))
    assert np.array_equal(orc.rotate(x, None, 0), inputs.bf16_bits_to_f32(x))


@pytest.mark.parametrize("name,rows", [("c1", 64), ("c2", 64), ("c3", 64), ("c4", 64), ("c5_4", 16)])
def test_rotation_preserves_norm(orc, name, rows):
    """||R x|| = ||x|| to 1e-6 relative on every row (R = H after a permutation)."""
    x = inputs.generate(name, rows=rows)
    cols = x.shape[1]
    perm = np.random.default_rng(1).permutation(cols).astype(np.int32)
    for p in (None, perm):
        y = orc.rotate(x, p, 32).astype(np.float64)
        xf = inputs.bf16_bits_to_f32(x).astype(np.float64)
        nx = np.linalg.norm(xf, axis=1)
        ny = np.linalg.norm(y, axis=1)
        assert np.all(np.abs(ny - nx) <= 1e-6 * nx)
        back = orc.unrotate_f64(y, p, 32)
        assert np.abs(back - xf).max() <= 1e-6 * np.abs(xf).max()


def test_permutation_bijective_and_balancing(orc):
    """The snake-dealt permutation is a bijection and evens out block energy."""
    x = inputs.gen_c4(rows=512)
    e = orc.channel_energy(x)
    xf = inputs.bf16_bits_to_f32(x).astype(np.float64)
    assert np.allclose(e, (xf * xf).sum(0), rtol=1e-12)
    perm = orc.build_perm(e.astype(np.float32), 32)
    assert np.array_equal(np.sort(perm), np.arange(x.shape[1]))
    blk0 = e.reshape(-1, 32).sum(1)
    blk1 = e[perm].reshape(-1, 32).sum(1)
    cv0 = blk0.std() / blk0.mean()
    cv1 = blk1.std() / blk1.mean()
    assert cv1 * 20 <= cv0, (cv0, cv1)
    # greedy invariant: each channel went to a least-loaded open block, so
    # replaying the assignment in energy order reproduces it
    order = np.argsort(-e.astype(np.float32), kind="stable")
    pos = np.empty_like(perm)
    pos[perm] = np.arange(perm.size)
    load = np.zeros(perm.size // 32)
    fill = np.zeros(perm.size // 32, int)
    for c in order:
        b = pos[c] // 32
        open_ = fill < 32
        assert open_[b] and load[b] == load[open_].min()
        assert pos[c] % 32 == fill[b]
        fill[b] += 1
        load[b] += float(np.float32(e[c]))


def test_build_perm_ties_by_index(orc):
    e = np.ones(64, np.float32)
    perm = orc.build_perm(e, 32)
    # all equal: channels 0..63 in order, each to the lower-index least-loaded
    # open block, so they alternate between the two blocks
    want = np.empty(64, np.int32)
    for c in range(64):
        want[32 * (c % 2) + c // 2] = c
    assert np.array_equal(perm, want)


def _mx_sqnr(orc, x, perm, had):
    codes, scales, _ = orc.rotate_quantize(x, perm, had)
    yh = orc.dequantize_f64(codes, scales, 0)
    xh = orc.unrotate_f64(yh, perm, had) if (had or perm is not None) else yh
    return orc.sqnr_db(inputs.bf16_bits_to_f32(x), xh), codes


def test_hadamard_helps_heavy_tails(orc):
    """Student-t(3) with outlier channels: the block Hadamard lowers MSE."""
    x = inputs.gen_c3(rows=256)
    s_plain, c_plain = _mx_sqnr(orc, x, None, 0)
    s_had, _ = _mx_sqnr(orc, x, None, 32)
    assert s_had > s_plain + 1.0, (s_plain, s_had)


def test_outlier_blocks_mostly_zeroed(orc):
    """A block holding an outlier channel has its exponent pushed up, so most of
    its other elements round to zero (the TORQ page's problem statement reports
    more than 90% on real activations; the synthetic heavy-tailed tensor gives a
    smaller but still dominant fraction). The Hadamard spreads the outlier and
    brings the fraction down."""
    rows = 256
    x = inputs.gen_c3(rows=rows)
    ch = inputs.c3_outlier_channels(rows=rows)
    codes, _ = orc.mx_quantize(x)
    u = np.empty((rows, x.shape[1]), np.uint8)
    u[:, 0::2], u[:, 1::2] = codes & 15, codes >> 4
    blocks = np.unique(ch // 32)
    inb = np.zeros(x.shape[1], bool)
    for b in blocks:
        inb[32 * b:32 * b + 32] = True
    others = inb.copy()
    others[ch] = False
    zero_out = ((u[:, others] & 7) == 0).mean()
    zero_norm = ((u[:, ~inb] & 7) == 0).mean()
    assert zero_out > 0.7 and zero_out > 3 * zero_norm, (zero_out, zero_norm)
    ch_, _, _ = orc.rotate_quantize(x, None, 32)
    uh = np.empty_like(u)
    uh[:, 0::2], uh[:, 1::2] = ch_ & 15, ch_ >> 4
    assert ((uh[:, inb] & 7) == 0).mean() < 0.5 * zero_out


def test_two_level_rotation_on_imbalanced_blocks(orc):
    """Block-variance imbalance: pi + H beats plain MXFP4 and pi alone."""
    x = inputs.gen_c4(rows=256)
    e = orc.channel_energy(x).astype(np.float32)
    perm = orc.build_perm(e, 32)
    s_plain, _ = _mx_sqnr(orc, x, None, 0)
    s_two, _ = _mx_sqnr(orc, x, perm, 32)
    assert s_two > s_plain + 0.2, (s_plain, s_two)


@pytest.mark.parametrize("group", [2, 4, 8])
def test_grouped_permutation(orc, group):
    """Units of `group` aligned channels move together; the greedy invariant
    holds on the unit energies; group 1 is the single-channel permutation."""
    x = inputs.gen_c4(rows=256)
    e = orc.channel_energy(x).astype(np.float32)
    perm = orc.build_perm(e, 32, group)
    assert np.array_equal(np.sort(perm), np.arange(perm.size))
    runs = perm.reshape(-1, group)
    assert np.all(runs[:, 0] % group == 0)
    assert np.all(runs - runs[:, :1] == np.arange(group)[None, :])
    ue = e.astype(np.float64).reshape(-1, group).sum(1)
    order = np.argsort(-ue, kind="stable")
    unit_pos = np.empty(ue.size, int)
    unit_pos[runs[:, 0] // group] = np.arange(runs.shape[0])
    load = np.zeros(perm.size // 32)
    fill = np.zeros(perm.size // 32, int)
    for u in order:
        b = unit_pos[u] // (32 // group)
        open_ = fill < 32 // group
        assert open_[b] and load[b] == load[open_].min()
        assert unit_pos[u] % (32 // group) == fill[b]
        fill[b] += 1
        load[b] += ue[u]
    blk = e.astype(np.float64)[perm].reshape(-1, 32).sum(1)
    blk0 = e.astype(np.float64).reshape(-1, 32).sum(1)
    assert blk.std() / blk.mean() < blk0.std() / blk0.mean()
    assert np.array_equal(orc.build_perm(e, 32, 1), orc.build_perm(e, 32))
