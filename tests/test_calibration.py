"""Host-side calibration of the learned block rotation, checked on the CPU
against the oracle's occupancy loss.

"TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization", technical
summary sec. 2(b): alternating coordinate descent (S-step: block scales; R-
step: a Givens rotation of a badly balanced, complementary coordinate pair at
the best of a finite set of angles) on the code-book occupancy equilibrium
loss, started from the Hadamard.
"""
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
