"""Pins for the oracle's RaZeR weight variant (CPU only).

"RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
Remapping", technical summary sec. 2.1-2.2: weights take an E3M3 block scale
(6 bits), and the two freed bits select one of four special values, two
pairs, for the redundant zero code; the block takes the candidate of least
squared error. Readings (the pages give neither): E3M3 with bias 3,
subnormals m 2^-5, largest 30; the second pair, +-2.5, comes from the
offline search in tests/golden/make_razer_w_pair.py.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from block_scaled_fp4_absmax_amd import inputs
from conftest import read_golden

E2M1 = [Fraction(v) for v in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]


def _pair():
    for ln in read_golden("razer_w_pair.txt"):
        if ln.startswith("pair"):
            return float(ln.split()[1])
    raise AssertionError("no pair in razer_w_pair.txt")


PAIR = _pair()


def _e3m3(c):
    e, m = c >> 3, c & 7
    return Fraction(m, 32) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 3)


def _std(code):
    return -E2M1[code & 7] if code & 8 else E2M1[code & 7]


def test_pair_is_a_half_multiple_off_the_grid():
    assert PAIR == 2.5  # the stored result of the offline search
    assert (2 * PAIR).is_integer() and Fraction(PAIR) not in E2M1 and PAIR != 5


def test_e3m3_decoder_closed_form(orc):
    vals = [orc.e3m3_value(c) for c in range(64)]
    assert all(Fraction(v) == _e3m3(c) for c, v in enumerate(vals))
    assert vals[63] == 30.0 and vals[1] == 1 / 32 and vals[8] == 0.25
    assert all(a < b for a, b in zip(vals, vals[1:]))  # strictly increasing


def test_e3m3_encoder_nearest_even(orc):
    """Every midpoint and one double ulp either side, and random values,
    against an exact nearest search with ties to the even code."""
    grid = [_e3m3(c) for c in range(64)]
    ys = list(np.random.default_rng(1).uniform(0, 35, 3000))
    for c in range(63):
        mid = float((grid[c] + grid[c + 1]) / 2)
        ys += [mid, np.nextafter(mid, 0), np.nextafter(mid, 99)]
    for y in ys:
        fy = Fraction(y)
        want = min(range(64), key=lambda c: (abs(fy - grid[c]), c % 2))
        if fy > 30:
            want = 63
        assert orc.e3m3_encode(y) == want, y


def _exact_choice(y, specials):
    """Exact least-SSE candidate (ties: lowest index) and its codes."""
    best = None
    for i, s in enumerate(specials):
        sf = Fraction(s)
        codes, sse = [], Fraction(0)
        for v in y:
            fv = Fraction(float(v))
            std = min(range(16), key=lambda c: (abs(fv - _std(c)), c & 1, c >> 3 if fv >= 0 else
                                                 1 - (c >> 3)))
            # zero is code 0 in RaZeR; the special only when strictly closer
            if _std(std) == 0:
                std = 0
            if abs(fv - sf) < abs(fv - _std(std)):
                codes.append(8)
                sse += (fv - sf) ** 2
            else:
                codes.append(std)
                sse += (fv - _std(std)) ** 2
        if best is None or sse < best[0]:
            best = (sse, i, codes)
    return best[1], best[2]


def test_block_choice_matches_exact_argmin(orc):
    specials = [5.0, -5.0, PAIR, -PAIR]
    rng = np.random.default_rng(7)
    blocks = [rng.uniform(-6.5, 6.5, 16).astype(np.float32) for _ in range(150)]
    for sp in (5.0, PAIR):  # adversarial: near the specials and their midpoints
        for _ in range(40):
            v = rng.choice([sp, sp + 0.25, sp - 0.25, sp + 0.5, -sp, -sp - 0.25], 16)
            blocks.append((v + rng.normal(0, 0.02, 16)).astype(np.float32))
    blocks.append(np.float32([2.5, -2.5, 5, -5] * 4))  # exact ties: lowest selector
    for y in blocks:
        codes, sel = orc.razer_block_set(y, specials)
        wsel, wcodes = _exact_choice(y, specials)
        assert sel == wsel and list(codes) == wcodes


@pytest.mark.parametrize("n", [2, 3])
def test_tiny_block_enumeration(orc, n):
    """Every selector x every code of every element on tiny blocks: the
    squared error separates over elements once the selector is fixed, so the
    best code vector for a selector is the best code per element (all 16,
    with code 0x8 worth that selector's special); the oracle's choice must
    reach the least error over all four selectors."""
    specials = [5.0, -5.0, PAIR, -PAIR]
    alphabet = np.float32([0, 2.3, -2.6, 2.75, 4.6, -5.2, 5.5, 6.1, -1.1])

    def err(v, c, s):
        val = Fraction(specials[s]) if c == 8 else _std(c)
        return (Fraction(float(v)) - val) ** 2

    for y in itertools.product(alphabet, repeat=n):
        y = np.float32(y)
        codes, sel = orc.razer_block_set(y, specials)
        got = sum(err(v, c, sel) for v, c in zip(y, codes))
        best = min(sum(min(err(v, c, s) for c in range(16)) for v in y) for s in range(4))
        assert got == best


def test_weight_quantizer_properties(orc):
    x = inputs.gen_c5(0, rows=64, cols=1024)
    c, s, st = orc.nvw_quantize(x, PAIR)
    amax = float(np.abs(inputs.bf16_bits_to_f32(x)).max())
    assert st == orc.nvw_tensor_scale(amax) and abs(180 * st - amax) <= amax * 2 ** -23
    assert (s & 63).max() == 63  # the largest block reaches the top scale, 30
    # each block is razer_block_set on its scaled values y = x RN(1 / s_eff),
    # and (in that domain, where the choice is made) never worse than the
    # single +-5 pair on the same scale
    sel = s >> 6
    assert set(np.unique(sel)) <= {0, 1, 2, 3} and (sel >= 2).any()
    e3 = np.array([orc.e3m3_value(b) for b in range(64)])
    s_eff = (e3[s & 63] * st).astype(np.float32)
    xs = inputs.bf16_bits_to_f32(x).reshape(64, -1, 16)
    nib = np.empty((64, 1024), np.uint8)
    nib[:, 0::2], nib[:, 1::2] = c & 15, c >> 4
    nib = nib.reshape(64, -1, 16)
    specials = [5.0, -5.0, PAIR, -PAIR]

    def sse(yb, codes, sp, sel_):
        v = np.array([sp[sel_] if q == 8 else float(_std(q)) for q in codes])
        return float(((yb.astype(np.float64) - v) ** 2).sum())

    for r in range(0, 64, 3):
        for b in range(xs.shape[1]):
            if s_eff[r, b] == 0:
                continue
            yb = xs[r, b] * np.float32(np.float32(1) / s_eff[r, b])
            c4, s4 = orc.razer_block_set(yb, specials)
            assert s4 == sel[r, b] and np.array_equal(c4, nib[r, b])
            c2, s2 = orc.razer_block_set(yb, specials[:2])
            assert sse(yb, c4, specials, s4) <= sse(yb, c2, specials, s2)
    # sign symmetry: negated weights flip every selector within its pair
    cn, sn, _ = orc.nvw_quantize(x ^ np.uint16(0x8000), PAIR)
    assert np.array_equal(sn & 63, s & 63)
    # a block whose special is used flips its selector within the pair; one
    # with no gain from any special keeps selector 0 (ties: the lowest)
    used = (nib == 8).any(-1)
    assert used.mean() > 0.5
    # (unless the pair's two signs gain exactly the same, when both keep the
    # lower, even selector)
    same = (sn >> 6) == (s >> 6)
    assert np.all(((sn >> 6) == ((s >> 6) ^ 1))[used] | (same & ((s >> 6) % 2 == 0))[used])
    assert (same & used).mean() < 0.01
    assert not (s >> 6)[~used].any() and not (sn >> 6)[~used].any()
    nibn = np.empty((64, 1024), np.uint8)
    nibn[:, 0::2], nibn[:, 1::2] = cn & 15, cn >> 4
    flip = np.where((nib.reshape(64, -1) & 7) == 0, nib.reshape(64, -1),
                    np.where(nib.reshape(64, -1) == 8, 8, nib.reshape(64, -1) ^ 8))
    flipped = np.repeat(((sn >> 6) == ((s >> 6) ^ 1)) | ~used, 16, axis=1)
    assert np.array_equal(nibn[flipped], flip[flipped])
