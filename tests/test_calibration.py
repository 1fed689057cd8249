"""Host-side calibration of the learned block rotation, checked on the CPU
against the oracle's occupancy loss.

"TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization", technical
summary sec. 2(b): alternating coordinate descent (S-step: block scales; R-
step: a Givens rotation of a badly balanced, complementary coordinate pair at
the best of a finite set of angles) on the code-book occupancy equilibrium
loss, started from the Hadamard.
"""
import ctypes

import numpy as np
import pytest

import block_scaled_fp4_absmax_amd as fp4
from block_scaled_fp4_absmax_amd import build as hip_build
from block_scaled_fp4_absmax_amd import inputs


@pytest.fixture(scope="module")
def L():
    if hip_build.is_stale():
        hip_build.build()
    return fp4.lib()


def _h0():
    i = np.arange(32)
    sign = np.vectorize(lambda a: -1.0 if bin(a).count("1") % 2 else 1.0)(i[:, None] & i[None, :])
    return (sign / np.sqrt(32)).astype(np.float32)


def _calib(L, x, perm, iters, angles):
    rows, cols = x.shape
    R = np.zeros((32, 32), np.float32)
    loss = np.zeros(2, np.float64)
    p = None if perm is None else np.ascontiguousarray(perm, np.int32).ctypes.data
    st = L.fp4_calibrate_block_rotation(x.ctypes.data, rows, cols, cols, p, iters, angles,
                                        R.ctypes.data, loss.ctypes.data)
    assert st == 0
    return R, loss


def _oracle_loss(orc, x, perm, R):
    return orc.occupancy(orc.rotate_r(x, perm, R.astype(np.float64)))[1]


@pytest.fixture(scope="module")
def sample(orc):
    x = inputs.gen_c3(rows=256, cols=2048)
    perm = orc.build_perm(orc.channel_energy(x).astype(np.float32), 32)
    return x, perm


def test_no_steps_returns_the_hadamard(L, orc, sample):
    x, perm = sample
    R, loss = _calib(L, x, perm, 0, 16)
    assert np.array_equal(R, _h0())
    assert loss[0] == loss[1]
    n = x.size
    assert abs(loss[0] - _oracle_loss(orc, x, perm, R)) <= 8 / n


def test_descent_is_orthogonal_lowers_the_loss_and_reports_it(L, orc, sample):
    x, perm = sample
    R, loss = _calib(L, x, perm, 40, 32)
    Rd = R.astype(np.float64)
    assert np.abs(Rd @ Rd.T - np.eye(32)).max() < 1e-6
    assert loss[1] < loss[0]
    n = x.size
    assert abs(loss[0] - _oracle_loss(orc, x, perm, _h0())) <= 8 / n
    assert abs(loss[1] - _oracle_loss(orc, x, perm, R)) <= 8 / n
    # deterministic
    R2, loss2 = _calib(L, x, perm, 40, 32)
    assert np.array_equal(R, R2) and np.array_equal(loss, loss2)


def _per_coordinate_occupancy(orc, y):
    """[32, 8] fractions: E2M1 magnitude index of each element (the oracle's
    MXFP4 quantizer) counted per coordinate inside the block."""
    codes, _ = orc.mx_quantize_f32(y)
    mag = np.empty((y.shape[0], y.shape[1]), np.uint8)
    mag[:, 0::2], mag[:, 1::2] = codes & 7, (codes >> 4) & 7
    mag = mag.reshape(-1, 32)
    return np.stack([np.bincount(mag[:, k], minlength=8) for k in range(32)]) / mag.shape[0]


def test_one_step_pair_and_best_angle(L, orc, sample):
    """One R-step: the pair is (most imbalanced coordinate, most
    complementary partner) of the oracle's per-coordinate occupancy, the
    angle is on the grid k pi / (2A), and no other grid angle for that pair
    has a lower oracle loss."""
    x, perm = sample
    A = 24
    H = _h0().astype(np.float64)
    R, loss = _calib(L, x, perm, 1, A)
    changed = np.where(np.abs(R.astype(np.float64) - H).max(1) > 0)[0]
    assert len(changed) == 2, "the first step on this sample is accepted"
    dev = _per_coordinate_occupancy(orc, orc.rotate_r(x, perm, H)) - 0.125
    imb = (dev * dev).sum(1)
    i = int(np.argmax(imb))
    dots = dev @ dev[i]
    dots[i] = np.inf
    j = int(np.argmin(dots))
    assert set(changed) == {i, j}
    c = float(R[i].astype(np.float64) @ H[i])
    s = -float(R[i].astype(np.float64) @ H[j])
    k = np.arctan2(s, c) / (np.pi / 2 / A)
    assert abs(k - round(k)) < 1e-4 and 1 <= round(k) < A

    def rotated(kk):
        th = kk * np.pi / 2 / A
        G = H.copy()
        G[i] = np.cos(th) * H[i] - np.sin(th) * H[j]
        G[j] = np.sin(th) * H[i] + np.cos(th) * H[j]
        return G.astype(np.float32)

    grid = [_oracle_loss(orc, x, perm, rotated(kk)) for kk in range(1, A)]
    n = x.size
    assert loss[1] <= min(grid) + 8 / n
    assert abs(loss[1] - grid[round(k) - 1]) <= 8 / n


def test_calibration_validation(L):
    x = np.zeros((4, 64), np.uint16)
    R = np.zeros((32, 32), np.float32)
    C = L.fp4_calibrate_block_rotation
    assert C(None, 4, 64, 64, None, 1, 8, R.ctypes.data, None) == -1
    assert C(x.ctypes.data, 4, 64, 64, None, 1, 8, None, None) == -1
    assert C(x.ctypes.data, 4, 48, 48, None, 1, 8, R.ctypes.data, None) == -2
    assert C(x.ctypes.data, 4, 64, 32, None, 1, 8, R.ctypes.data, None) == -2
    assert C(x.ctypes.data, 4, 64, 64, None, 1, 1, R.ctypes.data, None) == -4
    assert C(x.ctypes.data, 4, 64, 64, None, -1, 8, R.ctypes.data, None) == -4
    bad = np.full(64, 64, np.int32)
    assert C(x.ctypes.data, 4, 64, 64, bad.ctypes.data, 1, 8, R.ctypes.data, None) == -2
    # an all-zero sample has nothing to balance: the start is returned
    loss = np.zeros(2)
    assert C(x.ctypes.data, 4, 64, 64, None, 5, 8, R.ctypes.data, loss.ctypes.data) == 0
    assert np.array_equal(R, _h0()) and loss[0] == loss[1] == 0.875


# ------------------------------------------------- inter-block transform --
def _macro(L, x, perm, block=32, tol=1e-6, max_rot=None):
    rows, cols = x.shape
    if max_rot is None:
        max_rot = 4 * (cols // block)
    pairs = np.zeros((max_rot, 2), np.int32)
    cs = np.zeros((max_rot, 2), np.float32)
    starts = np.zeros(max_rot + 1, np.int32)
    n, nl = ctypes.c_int(0), ctypes.c_int(0)
    spread = np.zeros(2)
    p = None if perm is None else np.ascontiguousarray(perm, np.int32).ctypes.data
    st = L.fp4_calibrate_macro_rotation(x.ctypes.data, rows, cols, cols, p, block, tol, max_rot,
                                        pairs.ctypes.data, cs.ctypes.data, starts.ctypes.data,
                                        ctypes.byref(n), ctypes.byref(nl), spread.ctypes.data)
    assert st == 0
    return pairs[:n.value], cs[:n.value], starts[:nl.value + 1], spread


def _block_spread(z, block):
    v = (z.astype(np.float64) ** 2).sum(0).reshape(-1, block).sum(1)
    return (v.max() - v.min()) / v.mean(), v


@pytest.mark.parametrize("block,use_perm", [(32, True), (32, False), (16, True)])
def test_macro_rotation_equalises_block_variances(L, orc, block, use_perm):
    x = inputs.gen_c4(rows=256, cols=2048)
    perm = orc.build_perm(orc.channel_energy(x).astype(np.float32), block) if use_perm else None
    pairs, cs, starts, spread = _macro(L, x, perm, block)
    nb = 2048 // block
    s0, _ = _block_spread(orc.apply_givens(x, perm, pairs[:0], cs[:0]), block)
    z = orc.apply_givens(x, perm, pairs, cs.astype(np.float64))
    s1, _ = _block_spread(z, block)
    assert abs(spread[0] - s0) <= 1e-12 * s0 and abs(spread[1] - s1) <= 1e-9
    assert s1 <= 1e-5 < s0
    # after the permutation every step here is a full one: one per block but
    # the last; from the identity some pairs are too weak and steps are split
    assert len(pairs) <= (nb - 1 if use_perm else 4 * nb)
    # layers: consecutive, and the channels of a layer are disjoint
    assert starts[0] == 0 and starts[-1] == len(pairs) and np.all(np.diff(starts) > 0)
    for a, b in zip(starts[:-1], starts[1:]):
        ch = pairs[a:b].reshape(-1)
        assert len(np.unique(ch)) == len(ch)
    assert np.allclose(cs[:, 0] ** 2 + cs[:, 1] ** 2, 1.0, atol=1e-6)
    # every pair joins two different blocks
    assert np.all(pairs[:, 0] // block != pairs[:, 1] // block)


def test_macro_rotation_first_step(L, orc):
    """The first rotation pairs the strongest channel of the heaviest block
    with the weakest channel of the lightest, and brings one of the two
    blocks to the mean."""
    x = inputs.gen_c4(rows=256, cols=2048)
    perm = orc.build_perm(orc.channel_energy(x).astype(np.float32), 32)
    pairs, cs, _, _ = _macro(L, x, perm)
    xp = inputs.bf16_bits_to_f32(x).astype(np.float64)[:, perm]
    e = (xp ** 2).sum(0)
    v = e.reshape(-1, 32).sum(1)
    p, q = int(np.argmax(v)), int(np.argmin(v))
    i = 32 * p + int(np.argmax(e[32 * p:32 * p + 32]))
    j = 32 * q + int(np.argmin(e[32 * q:32 * q + 32]))
    assert tuple(pairs[0]) == (i, j)
    _, v1 = _block_spread(orc.apply_givens(x, perm, pairs[:1], cs[:1].astype(np.float64)), 32)
    mean = v.mean()
    assert min(abs(v1[p] - mean), abs(v1[q] - mean)) <= 1e-6 * mean
    assert abs(v1.sum() - v.sum()) <= 1e-9 * v.sum()


def test_macro_rotation_validation(L):
    x = np.zeros((4, 64), np.uint16)
    out = np.zeros(16, np.int32)
    cs = np.zeros(16, np.float32)
    n = ctypes.c_int(0)
    C = L.fp4_calibrate_macro_rotation
    args = [x.ctypes.data, 4, 64, 64, None, 32, 1e-6, 8, out.ctypes.data, cs.ctypes.data,
            out.ctypes.data, ctypes.byref(n), ctypes.byref(n), None]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return C(*a)

    assert call(a0=None) == -1
    assert call(a5=24) == -4          # block
    assert call(a2=48, a3=48) == -2   # cols % block
    assert call(a6=-1.0) == -4        # tol
    assert call(a7=-1) == -4          # max_rot
    assert call(a8=None) == -1
    bad = np.full(64, 99, np.int32)
    assert call(a4=bad.ctypes.data) == -2
    # an all-zero sample: nothing to move
    assert call() == 0 and n.value == 0
