"""Pins of the oracle's NVFP4 per-block arithmetic (CPU only).

The NVFP4 quantizers of the oracle (``nv_quantize`` on bf16 input,
``nv_quantize_f32`` on fp32 input, ``nvw_quantize`` for the weight variant)
take, per 16-element block, a fixed sequence of fp32 operations, each rounded
to nearest with ties to even:

    d      = RN(6 s_t)            s_t = RN(amax_tensor / 2688) unless given
    s_raw  = RN(amax_b / d)
    s_b    = nearest E4M3 code to s_raw (ties to the even code, at most 448)
    s_eff  = RN(e4m3(s_b) s_t)
    r      = RN(1 / s_eff)
    y_i    = RN(x_i r)
    code_i = nearest E2M1 value to y_i (ties to the even code); RaZeR: the
             special value of least squared error over the block

The NVFP4 format with its E4M3 block scale and fp32 tensor scale is the one of
the RaZeR page ("RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant
Zero Remapping", technical summary sec. 1); the special value that takes the
redundant zero code, chosen per block by least squared error, is its sec. 2.2;
the weight variant (a narrower block scale freeing two selector bits) its sec.
2.1-2.2. The order of the fp32 operations is a reading: the page does not fix
it.

This file restates the steps with exact rational arithmetic
(``fractions.Fraction``) and a round-to-fp32 helper of its own. E4M3 values
come from ``torch.float8_e4m3fn``, E3M3 values from the format's closed form,
E2M1 values from the set printed on the page (``tests/golden/
e2m1_value_set.txt``). Every scale byte and every code of the oracle is
compared with the restatement on random blocks and on blocks built so that a
plausible slip in the sequence changes a byte:

  * ``div``:  y = RN(x / s_eff) in place of RN(x RN(1 / s_eff));
  * ``div6``: s_raw = RN(RN(amax / 6) / s_t) in place of RN(amax / RN(6 s_t));
  * ``eff``:  s_eff left unrounded, r = RN(1 / (e4m3(s_b) s_t)).

The adversarial sets are checked to separate each slip from the reading, and
the last tests plant each slip in a copy of the oracle's C source, build it and
check that the comparison rejects it.
"""
import ctypes
import functools
import math
import os
import re
import subprocess
from fractions import Fraction as F

import numpy as np
import pytest
import torch

from block_scaled_fp4_absmax_amd import inputs
from conftest import ROOT, read_golden

# ----------------------------------------------------------- value tables ----


def _e2m1_magnitudes():
    """The eight E2M1 magnitudes in code order, from the printed value set
    (codes 0..7 are the non-negative values; each appears with both signs)."""
    vals = read_golden("e2m1_value_set.txt")[0].split()
    pos = [F(v) for v in vals if v.startswith("+")]
    assert len(pos) == 8 and pos == sorted(pos)
    return pos


MAG = _e2m1_magnitudes()
# E4M3 ("fn") values of the non-negative finite codes 0x00..0x7E, from torch
E4M3 = [F(float(v)) for v in
        torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)]
# E3M3: bias 3, subnormals m 2^-5 (e = 0), normals (1 + m/8) 2^(e-3); 64 codes
E3M3 = [F(m, 32) if e == 0 else F(8 + m, 8) * F(2) ** (e - 3)
        for e in range(8) for m in range(8)]
PAIR = F(read_golden("razer_w_pair.txt")[0].split()[1])
SPECIALS = {"razer": [F(5), F(-5)], "razer_w": [F(5), F(-5), PAIR, -PAIR]}


def rn32(q):
    """The fp32 value nearest to the rational q (ties: even significand),
    subnormals included; overflow raises."""
    if q == 0:
        return F(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1  # now 2^e <= a < 2^(e+1)
    ulp = F(2) ** (max(e, -126) - 23)
    n = a / ulp
    k = n.numerator // n.denominator
    rem = n - k
    if rem > F(1, 2) or (rem == F(1, 2) and k % 2 == 1):
        k += 1
    r = k * ulp
    if r >= F(2) ** 128:
        raise OverflowError(q)
    return r if q > 0 else -r


def nearest(v, table):
    """Index of the entry of an increasing table nearest to v; of two equally
    near entries, the even index."""
    dist = [abs(v - t) for t in table]
    m = min(dist)
    ties = [c for c, d in enumerate(dist) if d == m]
    return ties[0] if len(ties) == 1 else [c for c in ties if c % 2 == 0][0]


# ------------------------------------------------------------ the steps ----


def model_block(xs, s_t, kind, slip=None):
    """Scale byte and the 16 codes of one block of fp32 values xs (Python
    floats) with tensor scale s_t. kind: 'plain', 'razer' or 'razer_w'."""
    return _model_block(tuple(xs), s_t, kind, slip)


@functools.lru_cache(maxsize=None)
def _model_block(xs, s_t, kind, slip):
    assert fp32(s_t) == s_t, "the tensor scale is an fp32 value"
    X = [F(x) for x in xs]
    neg = [math.copysign(1.0, x) < 0 for x in xs]
    st = F(s_t)
    table = E3M3 if kind == "razer_w" else E4M3
    amax = max(abs(v) for v in X)
    if slip == "div6":
        s_raw = rn32(rn32(amax / 6) / st)
    else:
        s_raw = rn32(amax / rn32(6 * st))
    sb = nearest(s_raw, table)
    if sb == 0:
        return 0, (0,) * len(xs)
    prod = table[sb] * st
    s_eff = prod if slip == "eff" else rn32(prod)
    if slip == "div":
        ys = [rn32(x / s_eff) for x in X]
    else:
        r = rn32(1 / s_eff)
        ys = [rn32(x * r) for x in X]
    if kind == "plain":  # the sign bit is the input's, also for zeros
        return sb, tuple((8 if n else 0) | nearest(abs(y), MAG) for y, n in zip(ys, neg))
    best = None
    for sel, sp in enumerate(SPECIALS[kind]):
        codes, sse = [], F(0)
        for y, n in zip(ys, neg):
            idx = nearest(abs(y), MAG)
            std = -MAG[idx] if n else MAG[idx]
            if abs(y - sp) < abs(y - std):  # the special only when strictly closer
                codes.append(8)
                v = sp
            else:  # zero is always code 0x0 here
                codes.append((8 if n and idx else 0) | idx)
                v = std
            sse += (y - v) ** 2
        if best is None or sse < best[0]:  # equal error: the lower selector
            best = (sse, sel, codes)
    _, sel, codes = best
    return sb | sel << (7 if kind == "razer" else 6), tuple(codes)


def model_tensor_scale(xs_flat, kind):
    amax = max(abs(F(float(x))) for x in xs_flat)
    if amax == 0:
        return 1.0
    return float(rn32(amax / (180 if kind == "razer_w" else 2688)))


# --------------------------------------------------------------- helpers ----


def _unpack(codes):
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


def _bf16_floats(x):
    return inputs.bf16_bits_to_f32(x).astype(np.float64)


def _to_bf16(v):
    """fp32 values -> bf16 bits, values already bf16-exact."""
    b = np.asarray(v, np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0)
    return (b >> 16).astype(np.uint16)


def _oracle_run(fn, blocks, s_t, kind, f32):
    """Scale bytes [n] and codes [n, 16] of the oracle (or a planted copy's
    entry points ``fn``) on n single-block rows."""
    n = len(blocks)
    if f32:
        x = np.ascontiguousarray(np.array(blocks, np.float32).reshape(n, 16))
        codes = np.zeros((n, 8), np.uint8)
        scales = np.zeros((n, 1), np.uint8)
        fn["nv_f32"](x.ctypes.data, n, 16, 16, int(kind == "razer"), float(s_t),
                     codes.ctypes.data, 8, scales.ctypes.data, 1)
    else:
        x = np.ascontiguousarray(_to_bf16(np.array(blocks, np.float32)).reshape(n, 16))
        codes = np.zeros((n, 8), np.uint8)
        scales = np.zeros((n, 1), np.uint8)
        if kind == "razer_w":
            fn["nvw"](x.ctypes.data, n, 16, 16, float(s_t), float(PAIR), codes.ctypes.data, 8,
                      scales.ctypes.data, 1)
        else:
            fn["nv_bf16"](x.ctypes.data, n, 16, 16, int(kind == "razer"), float(s_t),
                          codes.ctypes.data, 8, scales.ctypes.data, 1)
    return scales[:, 0], _unpack(codes)


def _entry_points(lib):
    i64, i32, f32, f64, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double, \
        ctypes.c_void_p
    fns = {"nv_bf16": lib.orc_nv_quantize_bf16, "nv_f32": lib.orc_nv_quantize_f32,
           "nvw": lib.orc_nvw_quantize_bf16}
    fns["nv_bf16"].argtypes = [vp, i64, i64, i64, i32, f32, vp, i64, vp, i64]
    fns["nv_f32"].argtypes = [vp, i64, i64, i64, i32, f32, vp, i64, vp, i64]
    fns["nvw"].argtypes = [vp, i64, i64, i64, f32, f64, vp, i64, vp, i64]
    for f in fns.values():
        f.restype = None
    return fns


def _mismatches(fn, cases, slip=None):
    """Blocks (of the cases) on which fn's bytes or codes differ from the
    steps restated with the given slip (None: the reading)."""
    bad = 0
    for blocks, s_t, kind, f32 in cases:
        sc, cd = _oracle_run(fn, blocks, s_t, kind, f32)
        for i, xs in enumerate(blocks):
            b, c = model_block(xs, s_t, kind, slip)
            if sc[i] != b or tuple(cd[i]) != c:
                bad += 1
    return bad


def _separating(cases, slip):
    """Blocks of the cases on which the slip changes a byte."""
    n = 0
    for blocks, s_t, kind, _ in cases:
        for xs in blocks:
            if model_block(xs, s_t, kind) != model_block(xs, s_t, kind, slip):
                n += 1
    return n


# --------------------------------------------------------- input builders ----
F32 = np.float32


def _f32_neighbours(v, k):
    """fp32 values v stepped 0, +-1 .. +-k ulps."""
    out = [F32(v)]
    lo = hi = F32(v)
    for _ in range(k):
        lo = np.nextafter(lo, F32(-np.inf))
        hi = np.nextafter(hi, F32(np.inf))
        out += [lo, hi]
    return out


def fp32(v):
    """The fp32 value nearest to v, as a Python float."""
    return float(F32(v))


# tensor scales: powers of two, one ulp either side, and arbitrary values
S_T_LIST = [1.0, 2.0 ** -10, float(np.nextafter(F32(2.0 ** -10), F32(1))),
            float(np.nextafter(F32(2.0 ** -10), F32(0))), fp32(0.0123), fp32(3.1e-5), fp32(7.7e-3)]


def scale_midpoint_cases(kind):
    """fp32 blocks whose maximum puts s_raw at a midpoint of two adjacent
    block-scale values, and 1 or 2 ulps of amax to either side (the NVFP4
    quantizer on fp32 input)."""
    table = E3M3 if kind == "razer_w" else E4M3
    cases = []
    for j, s_t in enumerate(S_T_LIST):
        d = rn32(6 * F(s_t))
        blocks = []
        # every midpoint for two tensor scales, every fourth for the others
        step = 1 if j < 2 else 4
        for c in range(0, len(table) - 1, step):
            mid = (table[c] + table[c + 1]) / 2
            for a in _f32_neighbours(float(rn32(mid * d)), 2):
                rest = [float(a) * f for f in (0.5, -0.25, 0.75, -1.0, 0.3, 0.0, 0.9, -0.6, 0.1,
                                               0.45, -0.05, 0.2, -0.8, 0.66, 0.01)]
                blocks.append([float(a)] + [float(F32(v)) for v in rest])
        cases.append((blocks, s_t, kind, True))
    return cases


MIDPOINTS = [F(1, 4), F(3, 4), F(5, 4), F(7, 4), F(5, 2), F(7, 2), F(5)]
RAZER_EDGES = {"plain": [], "razer": [F(9, 2), F(11, 2)],
               "razer_w": [F(9, 2), F(11, 2), PAIR - F(1, 4), PAIR + F(1, 4)]}


def element_midpoint_cases(kind):
    """fp32 blocks with elements whose scaled value x r falls on an E2M1
    midpoint (or a RaZeR decision edge), and within a few ulps of it; block
    scales not powers of two, so that r is rounded."""
    table = E3M3 if kind == "razer_w" else E4M3
    codes = [20, 37, 43, 50, 61, 75, 91, 101] if kind != "razer_w" else [11, 19, 27, 35, 42]
    cases = []
    for s_t in (fp32(0.0123), fp32(3.1e-5), 1.0, float(np.nextafter(F32(2.0 ** -10), F32(1)))):
        d = rn32(6 * F(s_t))
        blocks = []
        for c in codes:
            amax = float(rn32(table[c] * d))  # s_raw rounds to code c
            s_eff = rn32(table[c] * F(s_t))
            for mu in MIDPOINTS + RAZER_EDGES[kind]:
                cand = []
                for sign in (1, -1):
                    cand += [sign * float(x) for x in _f32_neighbours(float(rn32(mu * s_eff)), 3)]
                for i in range(0, len(cand), 15):
                    chunk = cand[i:i + 15]
                    chunk += [0.0] * (15 - len(chunk))
                    blocks.append([amax] + chunk)
        cases.append((blocks, s_t, kind, True))
    return cases


def _bf16_near(v):
    """The bf16 value nearest to v (Python float)."""
    return float(inputs.bf16_bits_to_f32(_to_bf16_round(v))[0])


def bf16_targeted_cases(kind, n=40, seed=7):
    """bf16 blocks (the quantizer's usual input) placed on the edges by the
    choice of the tensor scale: bf16 values are too coarse to fall within an
    ulp of a midpoint by chance, so for a bf16 element x, a target value mu and
    a block-scale code c, s_t is taken near x / (mu e(c)) and stepped by ulps,
    which sweeps x r across mu (the block maximum, near 6 e(c) s_t, keeps the
    block-scale code c); likewise s_t near amax / (6 m) sweeps the quotient
    amax / RN(6 s_t) across a midpoint m of two block-scale values."""
    rng = np.random.default_rng(seed)
    table = E3M3 if kind == "razer_w" else E4M3
    targets = MIDPOINTS + RAZER_EDGES[kind]
    lo_c, hi_c = (12, 62) if kind == "razer_w" else (24, 125)
    cases = []
    for _ in range(n):
        c = int(rng.integers(lo_c, hi_c))
        mu = targets[int(rng.integers(len(targets)))]
        x = _bf16_near(float(rng.uniform(1, 2)) * 2.0 ** int(rng.integers(-12, 4)))
        for s_t in _f32_neighbours(float(F(x) / (mu * table[c])), 3):
            s_t = float(s_t)
            amax = _bf16_near(float(table[c] * 6 * F(s_t)))
            rest = [_bf16_near(x * f) for f in (-1.0, 0.5, -0.75, 0.3, 0.9, -0.2, 0.6, 0.0,
                                                 -0.45, 0.15, 0.8, -0.33, 0.05, 0.7)]
            cases.append(([[amax, x] + rest], s_t, kind, False))
    for _ in range(n):
        c = int(rng.integers(lo_c - 16, hi_c))
        m = (table[c] + table[c + 1]) / 2
        amax = _bf16_near(float(rng.uniform(1, 2)) * 2.0 ** int(rng.integers(-12, 4)))
        for s_t in _f32_neighbours(float(F(amax) / (6 * m)), 3):
            rest = [_bf16_near(amax * f) for f in (0.5, -0.25, 0.75, -1.0, 0.3, 0.0, 0.9, -0.6,
                                                   0.1, 0.45, -0.05, 0.2, -0.8, 0.66)]
            cases.append(([[amax] + rest + [-amax * 0.125]], float(s_t), kind, False))
    return cases


def _to_bf16_round(v):
    return inputs.f64_to_bf16_bits(np.array([float(v)], np.float64))


def random_cases(kind, f32):
    """Random blocks: the small NVFP4 weight recipe, and blocks whose
    elements span many binades (subnormal block scales, saturation)."""
    rng = np.random.default_rng(11 if f32 else 12)
    out = []
    x = inputs.gen_c2(rows=8, cols=256, seed=5)
    xf = _bf16_floats(x).reshape(-1, 16)
    if f32:  # off the bf16 grid
        xf = (xf * (1 + rng.uniform(-1e-3, 1e-3, xf.shape))).astype(F32).astype(np.float64)
    out.append(([list(b) for b in xf], None, kind, f32))
    wide = rng.standard_normal((96, 16)) * np.exp2(rng.uniform(-24, 12, (96, 1)))
    wide[::7, 3] = 0.0
    wide[::11, 5] = -0.0
    wide = wide.astype(F32).astype(np.float64)
    if not f32:
        wide = _bf16_floats(inputs.f64_to_bf16_bits(wide))
    for s_t in (1.0, 2.0 ** -7, float(np.nextafter(F32(2.0 ** -7), F32(0))), fp32(1e-3)):
        out.append(([list(b) for b in wide], s_t, kind, f32))
    return out


def _resolve(cases):
    """Computed tensor scales (None) replaced by the restated rule."""
    res = []
    for blocks, s_t, kind, f32 in cases:
        if s_t is None:
            s_t = model_tensor_scale([v for b in blocks for v in b], kind)
        res.append((blocks, s_t, kind, f32))
    return res


@pytest.fixture(scope="module")
def oracle_fns(orc):
    return _entry_points(orc._load())


ALL_KINDS = [("plain", False), ("razer", False), ("plain", True), ("razer", True),
             ("razer_w", False)]


# ----------------------------------------------------------------- tests ----


@pytest.mark.parametrize("kind,f32", ALL_KINDS)
def test_random_blocks_match_steps(oracle_fns, kind, f32):
    cases = _resolve(random_cases(kind, f32))
    assert sum(len(c[0]) for c in cases) >= 400
    assert _mismatches(oracle_fns, cases) == 0


@pytest.mark.parametrize("kind,f32", ALL_KINDS)
def test_tensor_scale_rule(orc, kind, f32):
    """s_t computed by the oracle = RN(amax / 2688) (weights: / 180), and the
    whole tensor quantized with it matches the restated steps."""
    x = inputs.gen_c2(rows=4, cols=128, seed=9)
    if kind == "razer_w":
        c, s, ts = orc.nvw_quantize(x, float(PAIR))
    elif f32:
        y = inputs.bf16_bits_to_f32(x) * F32(1.0007)
        c, s, ts = orc.nv_quantize_f32(y, kind == "razer")
        x = None
    else:
        c, s, ts = orc.nv_quantize(x, kind == "razer")
    vals = _bf16_floats(x) if x is not None else y.astype(np.float64)
    want = model_tensor_scale(vals.ravel(), kind)
    assert ts == want
    cd = _unpack(c).reshape(-1, 16)
    sc = s.reshape(-1)
    for i, blk in enumerate(vals.reshape(-1, 16)):
        b, cc = model_block(list(blk), want, kind)
        assert sc[i] == b and tuple(cd[i]) == cc


@pytest.mark.parametrize("kind", ["plain", "razer", "razer_w"])
def test_scale_midpoints_match_steps(oracle_fns, kind):
    cases = scale_midpoint_cases(kind)
    if kind == "razer_w":  # the weight quantizer has a bf16 entry point only
        cases = [([[float(inputs.bf16_bits_to_f32(_to_bf16_round(v))[0]) for v in b]
                   for b in blocks], s_t, kind, False) for blocks, s_t, kind, _ in cases]
    assert _mismatches(oracle_fns, cases) == 0


@pytest.mark.parametrize("kind", ["plain", "razer"])
def test_element_midpoints_match_steps(oracle_fns, kind):
    assert _mismatches(oracle_fns, element_midpoint_cases(kind)) == 0


@pytest.mark.parametrize("kind", ["plain", "razer", "razer_w"])
def test_bf16_targeted_blocks_match_steps(oracle_fns, kind):
    cases = bf16_targeted_cases(kind)
    assert sum(len(c[0]) for c in cases) >= 100
    assert _mismatches(oracle_fns, cases) == 0


@functools.lru_cache(maxsize=None)
def _slip_sets():
    """Adversarial sets per entry point of the quantizer."""
    return {
        "bf16 plain": bf16_targeted_cases("plain"),
        "bf16 razer": bf16_targeted_cases("razer"),
        "bf16 razer_w": bf16_targeted_cases("razer_w"),
        "f32 plain": element_midpoint_cases("plain") + scale_midpoint_cases("plain"),
        "f32 razer": element_midpoint_cases("razer"),
    }


@pytest.mark.parametrize("slip", ["div", "div6", "eff"])
def test_adversarial_sets_separate_each_slip(slip):
    """Each slip in the step sequence changes some byte of every entry point's
    set, so an oracle that made it would fail the tests above."""
    for name, cases in _slip_sets().items():
        if slip == "div6" and name == "f32 razer":
            continue  # its blocks hold s_raw on block-scale values, not midpoints
        assert _separating(cases, slip) >= 3, name


# the planted slips: (pattern in the oracle's C source, replacement)
PLANTS = {
    "div": (r"y\[i\] = xv\[i\] \* rcp;", "y[i] = xv[i] / s_eff;"),
    "div6": (r"float s_raw = amax / d;", "float s_raw = amax / 6.0f / s_t;"),
    "eff": (r"float s_eff = \(float\)orc_e([34])m3_value\(sb\) \* s_t;",
            r"double s_eff = orc_e\1m3_value(sb) * (double)s_t;"),
}


@pytest.mark.parametrize("slip", ["div", "div6", "eff"])
def test_planted_slip_is_rejected(tmp_path, slip):
    """The slip planted in a copy of the oracle's source (CPU build) makes
    the comparison with the restated steps fail."""
    with open(os.path.join(ROOT, "oracle", "fp4_oracle.c")) as fh:
        src = fh.read()
    pat, rep = PLANTS[slip]
    planted, n = re.subn(pat, rep, src)
    assert n == 2, "the lines to plant the slip in (NVFP4 and weight blocks) are gone"
    path = tmp_path / "planted.c"
    path.write_text(planted)
    shutil_h = os.path.join(ROOT, "oracle", "fp4_oracle.h")
    (tmp_path / "fp4_oracle.h").write_text(open(shutil_h).read())
    so = tmp_path / "libplanted.so"
    subprocess.run(["gcc", "-O2", "-std=gnu99", "-ffp-contract=off", "-fno-fast-math",
                    "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(so), str(path), "-lm"],
                   check=True)
    fns = _entry_points(ctypes.CDLL(str(so)))
    for name, cases in _slip_sets().items():
        if slip == "div6" and name == "f32 razer":
            continue
        assert _mismatches(fns, cases) > 0, name
