"""Plain CPU oracle for block-scaled FP4 quantization (ctypes over fp4_oracle.c).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(the HIP library and its Python binding) never imports it, and this package
imports nothing from the product.

Parity status of each oracle function, i.e. what pins it to something other
than itself (the pins live in ``tests/test_oracle_*.py``):

* ``e2m1_value``: pinned to the value set printed on the RaZeR page (technical
  summary sec. 1), stored in ``tests/golden/e2m1_value_set.txt``, and to the
  textbook E2M1 formula.
* ``e2m1_nearest`` / ``e2m1_nearest_razer``: pinned to exact Fraction brute
  force and to an independent round-half-even rule, over every bf16 pattern.
* ``e4m3_value`` / ``e4m3_encode``: decoder pinned to ``torch.float8_e4m3fn``;
  encoder pinned at every midpoint and one ulp either side.
* ``e8m0_scale``: pinned exhaustively by the minimality property; decoder pinned
  to ``torch.float8_e8m0fnu``.
* ``mx_quantize*``, ``dequantize*``: pinned by the nearest-grid property,
  scale invariance, sign symmetry and idempotence.
* ``nv_quantize``, ``nv_quantize_f32``, ``nvw_quantize``, ``nv_tensor_scale``,
  ``nvw_tensor_scale``: every scale byte and code pinned to a restatement of
  the per-block fp32 steps (tensor scale, RN(6 s_t), the block quotient, the
  E4M3 / E3M3 code, s_eff, its reciprocal, the scaled elements, the nearest
  code and the RaZeR choice) in exact rational arithmetic with its own fp32
  rounding, E4M3 values from ``torch.float8_e4m3fn``, on random blocks and on
  blocks that sit on every rounding edge of the sequence; those blocks are
  shown to separate the plausible slips (x / s_eff, amax / 6 / s_t, an
  unrounded s_eff), and each slip planted in a copy of the C source is
  rejected. Also by error bounds, scale invariance and sign symmetry.
* ``nv_tensor_amax_f32``: pinned to numpy's maximum of magnitudes.
* ``int4_value`` / ``int4_nearest`` / ``mxint4_scale`` / ``mxint4_quantize*``:
  decoder pinned to numpy's two's complement sign extension; nearest search
  to ``np.rint`` (round half to even) and exact Fraction brute force; the
  scale pinned exhaustively by minimality over every bf16 magnitude; whole
  tensors by the nearest-grid property, the half-step error bound, scale
  invariance and sign symmetry.
* ``gemm_f64``: pinned to an exact rational evaluation (Fraction) of the
  block-scaled dot products on small operands, one-hot operands and the
  bilinearity of the block scales.
* ``razer_block``: pinned by exact Fraction SSE arg-min and exhaustive tiny-block
  enumeration.
* ``rotate`` / ``unrotate_f64``: pinned to ``scipy.linalg.hadamard`` (orders 16
  and 32) and norm preservation.
* ``e3m3_value`` / ``e3m3_encode`` / ``razer_block_set``: decoder pinned to
  its closed form; encoder at every midpoint and one ulp either side; the
  block choice to an exact Fraction arg-min and exhaustive tiny-block
  enumeration (``nvw_quantize``: see the NVFP4 entry above). The second
  special-value pair is not on the pages: parity unpinned for that value (an
  offline search picks it).
* ``rotate_r`` / ``unrotate_r_f64``: pinned by special matrices (identity,
  permutation, Sylvester-Hadamard from scipy, one Givens rotation in closed
  form), a random orthogonal matrix against numpy's product, and the inverse.
* ``occupancy``: pinned to an exact Fraction search of the scale and the
  nearest magnitude, and to uniform and all-zero cases.
* ``apply_givens``: pinned to a dense product of the Givens matrices (numpy),
  closed forms for one rotation and for angles 0 and pi/2 (a swap with a sign),
  norm preservation and the inverse (the transposed rotations in reverse).
* ``build_perm``: pinned by bijectivity, block-energy balancing, a replay of the
  greedy invariant (every unit goes to an open block of least load) and, for
  aligned channel runs, the run structure.
* Whole-pipeline bit patterns on the five synthetic workloads: parity unpinned
  beyond the properties above, since the pages print no worked example.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4_oracle.c")
_HDR = os.path.join(_HERE, "fp4_oracle.h")
_LIB = os.path.join(_HERE, "_build", "liboracle_fp4.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= max(
        os.path.getmtime(_SRC), os.path.getmtime(_HDR)
    ):
        return _LIB
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = [
        "gcc", "-O2", "-std=gnu99", "-ffp-contract=off", "-fno-fast-math",
        "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    i64, i32, f32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
    vp = ctypes.c_void_p
    sig = {
        "orc_version": (i32, []),
        "orc_set_threads": (None, [i32]),
        "orc_get_threads": (i32, []),
        "orc_e2m1_value": (f64, [i32]),
        "orc_e2m1_nearest": (i32, [f64]),
        "orc_e2m1_nearest_razer": (i32, [f64, f64]),
        "orc_e4m3_value": (f64, [i32]),
        "orc_e4m3_encode": (i32, [f64]),
        "orc_e8m0_value": (f64, [i32]),
        "orc_e8m0_scale": (i32, [f64, i32]),
        "orc_bf16_to_f32": (f32, [ctypes.c_uint16]),
        "orc_f32_to_bf16": (ctypes.c_uint16, [f32]),
        "orc_mx_quantize_f32": (None, [vp, i64, i64, i64, i32, vp, i64, vp, i64]),
        "orc_mx_quantize_bf16": (None, [vp, i64, i64, i64, i32, vp, i64, vp, i64]),
        "orc_int4_value": (f64, [i32]),
        "orc_int4_nearest": (i32, [f64]),
        "orc_mxint4_scale": (i32, [f64, i32]),
        "orc_mxint4_quantize_f32": (None, [vp, i64, i64, i64, i32, vp, i64, vp, i64]),
        "orc_mxint4_quantize_bf16": (None, [vp, i64, i64, i64, i32, vp, i64, vp, i64]),
        "orc_nv_tensor_amax": (f32, [vp, i64, i64, i64]),
        "orc_nv_tensor_scale": (f32, [f32]),
        "orc_nv_quantize_bf16": (None, [vp, i64, i64, i64, i32, f32, vp, i64, vp, i64]),
        "orc_nv_quantize_f32": (None, [vp, i64, i64, i64, i32, f32, vp, i64, vp, i64]),
        "orc_nv_tensor_amax_f32": (f32, [vp, i64, i64, i64]),
        "orc_razer_block": (i32, [vp, i32, vp, vp, vp]),
        "orc_dequantize": (None, [vp, i64, vp, i64, f32, i64, i64, i32, i32, f64, vp, i64]),
        "orc_dequantize_f64": (None, [vp, i64, vp, i64, f32, i64, i64, i32, i32, f64, vp, i64]),
        "orc_e3m3_value": (f64, [i32]),
        "orc_e3m3_encode": (i32, [f64]),
        "orc_nvw_tensor_scale": (f32, [f32]),
        "orc_razer_block_set": (i32, [vp, i32, vp, i32, vp]),
        "orc_nvw_quantize_bf16": (None, [vp, i64, i64, i64, f32, f64, vp, i64, vp, i64]),
        "orc_nvw_value": (f64, [i32, i32, f64]),
        "orc_rotate": (None, [vp, i64, i64, i64, vp, i32, vp, i64]),
        "orc_unrotate_f64": (None, [vp, i64, i64, i64, vp, i32, vp, i64]),
        "orc_channel_energy": (None, [vp, i64, i64, i64, vp]),
        "orc_rotate_r": (None, [vp, i64, i64, i64, vp, vp, vp, i64]),
        "orc_apply_givens": (None, [vp, i64, i64, i64, vp, i64, vp, vp, vp, i64]),
        "orc_unrotate_r_f64": (None, [vp, i64, i64, i64, vp, vp, vp, i64]),
        "orc_occupancy": (f64, [vp, i64, i64, i64, vp]),
        "orc_build_perm": (None, [vp, i64, i32, i32, vp]),
        "orc_hadamard_entry": (f64, [i32, i32, i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _ld(a: np.ndarray) -> int:
    """Row stride in elements of a 2-D array whose rows are contiguous."""
    assert a.ndim == 2 and a.strides[1] == a.itemsize, "rows must be contiguous"
    return a.strides[0] // a.itemsize


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return _load().orc_get_threads()


# ---- scalar format helpers -------------------------------------------------
def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(int(code))


def e2m1_nearest(y: float) -> int:
    return _load().orc_e2m1_nearest(float(y))


def e2m1_nearest_razer(y: float, special: float) -> int:
    return _load().orc_e2m1_nearest_razer(float(y), float(special))


def e4m3_value(code: int) -> float:
    return _load().orc_e4m3_value(int(code))


def e4m3_encode(v: float) -> int:
    return _load().orc_e4m3_encode(float(v))


def e8m0_value(byte: int) -> float:
    return _load().orc_e8m0_value(int(byte))


def e8m0_scale(amax: float, floor_rule: bool = False) -> int:
    return _load().orc_e8m0_scale(float(amax), int(bool(floor_rule)))


def bf16_to_f32(h: int) -> float:
    return _load().orc_bf16_to_f32(int(h))


def f32_to_bf16(f: float) -> int:
    return _load().orc_f32_to_bf16(float(f))


# ---- tensor operations -------------------------------------------------------
def mx_quantize(x_bf16: np.ndarray, floor_rule: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """MXFP4 codes [rows, cols/2] and E8M0 scales [rows, cols/32] of bf16 bits."""
    assert x_bf16.dtype == np.uint16
    rows, cols = x_bf16.shape
    assert cols % 32 == 0
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 32), np.uint8)
    _load().orc_mx_quantize_bf16(_ptr(x_bf16), rows, cols, _ld(x_bf16), int(floor_rule),
                                 _ptr(codes), cols // 2, _ptr(scales), cols // 32)
    return codes, scales


def mx_quantize_f32(x: np.ndarray, floor_rule: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    assert x.dtype == np.float32
    rows, cols = x.shape
    assert cols % 32 == 0
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 32), np.uint8)
    _load().orc_mx_quantize_f32(_ptr(x), rows, cols, _ld(x), int(floor_rule),
                                _ptr(codes), cols // 2, _ptr(scales), cols // 32)
    return codes, scales


def int4_value(code: int) -> float:
    return _load().orc_int4_value(int(code))


def int4_nearest(y: float) -> int:
    return _load().orc_int4_nearest(float(y))


def mxint4_scale(amax: float, floor_rule: bool = False) -> int:
    return _load().orc_mxint4_scale(float(amax), int(floor_rule))


def mxint4_quantize(x_bf16: np.ndarray, floor_rule: bool = False
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """MXINT4 codes [rows, cols/2] and E8M0 scale bytes [rows, cols/32] of bf16 bits."""
    assert x_bf16.dtype == np.uint16
    rows, cols = x_bf16.shape
    assert cols % 32 == 0
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 32), np.uint8)
    _load().orc_mxint4_quantize_bf16(_ptr(x_bf16), rows, cols, _ld(x_bf16), int(floor_rule),
                                     _ptr(codes), cols // 2, _ptr(scales), cols // 32)
    return codes, scales


def mxint4_quantize_f32(x: np.ndarray, floor_rule: bool = False
                        ) -> Tuple[np.ndarray, np.ndarray]:
    x = np.ascontiguousarray(x, np.float32)
    rows, cols = x.shape
    assert cols % 32 == 0
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 32), np.uint8)
    _load().orc_mxint4_quantize_f32(_ptr(x), rows, cols, cols, int(floor_rule), _ptr(codes),
                                    cols // 2, _ptr(scales), cols // 32)
    return codes, scales


def nv_tensor_amax(x_bf16: np.ndarray) -> float:
    rows, cols = x_bf16.shape
    return _load().orc_nv_tensor_amax(_ptr(x_bf16), rows, cols, _ld(x_bf16))


def nv_tensor_scale(amax: float) -> float:
    return _load().orc_nv_tensor_scale(float(amax))


def nv_quantize(x_bf16: np.ndarray, razer: bool, tensor_scale: Optional[float] = None
                ) -> Tuple[np.ndarray, np.ndarray, float]:
    """NVFP4 codes, E4M3 scale bytes (RaZeR selector in bit 7) and s_t."""
    assert x_bf16.dtype == np.uint16
    rows, cols = x_bf16.shape
    assert cols % 16 == 0
    if tensor_scale is None:
        tensor_scale = nv_tensor_scale(nv_tensor_amax(x_bf16))
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    _load().orc_nv_quantize_bf16(_ptr(x_bf16), rows, cols, _ld(x_bf16), int(razer),
                                 float(tensor_scale), _ptr(codes), cols // 2,
                                 _ptr(scales), cols // 16)
    return codes, scales, float(np.float32(tensor_scale))


def razer_block(y: np.ndarray) -> Tuple[np.ndarray, int, float, float]:
    """Unpacked codes, selector bit, chosen SSE and plain-E2M1 SSE of scaled values."""
    y = np.ascontiguousarray(y, np.float32)
    n = y.size
    assert 0 < n <= 64
    codes = np.zeros(n, np.uint8)
    sse = np.zeros(1, np.float64)
    sse0 = np.zeros(1, np.float64)
    sel = _load().orc_razer_block(_ptr(y), n, _ptr(codes), _ptr(sse), _ptr(sse0))
    return codes, int(sel), float(sse[0]), float(sse0[0])


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: int, razer: int = 0,
               tensor_scale: float = 1.0, pair: float = 0.0) -> np.ndarray:
    """bf16 bits [rows, cols] of the decoded values (fmt 0 = MXFP4, 1 = NVFP4,
    2 = MXINT4; NVFP4 razer 1 = RaZeR, 2 = the weight variant with second
    special pair +-pair)."""
    rows = codes.shape[0]
    cols = codes.shape[1] * 2
    out = np.zeros((rows, cols), np.uint16)
    _load().orc_dequantize(_ptr(codes), _ld(codes), _ptr(scales), _ld(scales),
                           float(tensor_scale), rows, cols, int(fmt), int(razer), float(pair),
                           _ptr(out), cols)
    return out


def dequantize_f64(codes: np.ndarray, scales: np.ndarray, fmt: int, razer: int = 0,
                   tensor_scale: float = 1.0, pair: float = 0.0) -> np.ndarray:
    rows = codes.shape[0]
    cols = codes.shape[1] * 2
    out = np.zeros((rows, cols), np.float64)
    _load().orc_dequantize_f64(_ptr(codes), _ld(codes), _ptr(scales), _ld(scales),
                               float(tensor_scale), rows, cols, int(fmt), int(razer),
                               float(pair), _ptr(out), cols)
    return out


# ---- RaZeR for weights: E3M3 block scale, four special values --------------
def e3m3_value(code: int) -> float:
    return _load().orc_e3m3_value(int(code))


def e3m3_encode(v: float) -> int:
    return _load().orc_e3m3_encode(float(v))


def nvw_tensor_scale(amax: float) -> float:
    return float(_load().orc_nvw_tensor_scale(float(amax)))


def razer_block_set(y: np.ndarray, specials) -> Tuple[np.ndarray, int]:
    y = np.ascontiguousarray(y, np.float32)
    sp = np.ascontiguousarray(specials, np.float64)
    codes = np.zeros(y.size, np.uint8)
    sel = _load().orc_razer_block_set(_ptr(y), y.size, _ptr(sp), sp.size, _ptr(codes))
    return codes, int(sel)


def nvw_quantize(x_bf16: np.ndarray, pair: float, tensor_scale: Optional[float] = None
                 ) -> Tuple[np.ndarray, np.ndarray, float]:
    """RaZeR weight quantization: codes, scale bytes (E3M3 | selector << 6), s_t."""
    assert x_bf16.dtype == np.uint16
    rows, cols = x_bf16.shape
    assert cols % 16 == 0
    if tensor_scale is None:
        tensor_scale = nvw_tensor_scale(nv_tensor_amax(x_bf16))
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    _load().orc_nvw_quantize_bf16(_ptr(x_bf16), rows, cols, _ld(x_bf16), float(tensor_scale),
                                  float(pair), _ptr(codes), cols // 2, _ptr(scales), cols // 16)
    return codes, scales, float(tensor_scale)


def nv_tensor_amax_f32(y: np.ndarray) -> float:
    y = np.ascontiguousarray(y, np.float32)
    rows, cols = y.shape
    return float(_load().orc_nv_tensor_amax_f32(_ptr(y), rows, cols, cols))


def nv_quantize_f32(y: np.ndarray, razer: bool, tensor_scale: Optional[float] = None
                    ) -> Tuple[np.ndarray, np.ndarray, float]:
    """NVFP4 of fp32 values: codes, E4M3 scale bytes (RaZeR selector in bit 7), s_t."""
    y = np.ascontiguousarray(y, np.float32)
    rows, cols = y.shape
    assert cols % 16 == 0
    if tensor_scale is None:
        tensor_scale = nv_tensor_scale(nv_tensor_amax_f32(y))
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    _load().orc_nv_quantize_f32(_ptr(y), rows, cols, cols, int(razer), float(tensor_scale),
                                _ptr(codes), cols // 2, _ptr(scales), cols // 16)
    return codes, scales, float(tensor_scale)


def rotate(x_bf16: np.ndarray, perm: Optional[np.ndarray], hadamard: int) -> np.ndarray:
    """fp32 [rows, cols]: permute channels, then Hadamard inside each block."""
    rows, cols = x_bf16.shape
    if perm is not None:
        perm = np.ascontiguousarray(perm, np.int32)
        assert perm.shape == (cols,)
    out = np.zeros((rows, cols), np.float32)
    _load().orc_rotate(_ptr(x_bf16), rows, cols, _ld(x_bf16), _ptr(perm), int(hadamard),
                       _ptr(out), cols)
    return out


def rotate_quantize(x_bf16: np.ndarray, perm: Optional[np.ndarray], hadamard: int,
                    floor_rule: bool = False):
    """Rotation then MXFP4 quantization of the fp32 rotated values."""
    y = rotate(x_bf16, perm, hadamard)
    codes, scales = mx_quantize_f32(y, floor_rule)
    return codes, scales, y


def rotate_quantize_nv(x_bf16: np.ndarray, perm: Optional[np.ndarray], hadamard: int,
                       razer: bool, tensor_scale: Optional[float] = None):
    """Rotation (block-16 Hadamard) then NVFP4 of the fp32 rotated values:
    (codes, scales, s_t, rotated). s_t from the rotated tensor's amax unless given."""
    y = rotate(x_bf16, perm, hadamard)
    codes, scales, ts = nv_quantize_f32(y, razer, tensor_scale)
    return codes, scales, ts, y


def rotate_quantize_mxint4(x_bf16: np.ndarray, perm: Optional[np.ndarray], hadamard: int,
                           floor_rule: bool = False):
    """Rotation then MXINT4 quantization of the fp32 rotated values."""
    y = rotate(x_bf16, perm, hadamard)
    codes, scales = mxint4_quantize_f32(y, floor_rule)
    return codes, scales, y


def decode_exact(codes: np.ndarray, scales: np.ndarray, fmt: int, razer: int = 0,
                 tensor_scale: float = 1.0, pair: float = 0.0) -> np.ndarray:
    """float64 [rows, cols] of the exact element values (no rounding at all):
    MXFP4 e2m1(code) 2^(e-127); NVFP4 e2m1(code) e4m3(scale) s_t, RaZeR code
    0x8 reading +5 or -5 by the scale's top bit. Exact in float64: at most 3
    significant bits times 4 times 24. razer 2: the weight variant (E3M3
    scale, special {+5, -5, +pair, -pair}[selector])."""
    codes = np.ascontiguousarray(codes)
    rows, half = codes.shape
    nib = np.empty((rows, 2 * half), np.int64)
    nib[:, 0::2] = codes & 15
    nib[:, 1::2] = codes >> 4
    e2m1 = np.array([e2m1_value(c) for c in range(16)])
    val = e2m1[nib]
    if fmt == 0:
        e = np.repeat(scales.astype(np.int64), 32, axis=1)[:, :2 * half] - 127
        return np.ldexp(val, e)
    assert fmt == 1
    sb = np.repeat(scales.astype(np.int64), 16, axis=1)[:, :2 * half]
    if razer == 2:
        sp = np.array([5.0, -5.0, pair, -pair])
        val = np.where(nib == 8, sp[(sb >> 6) & 3], val)
        e3m3 = np.array([e3m3_value(b) for b in range(64)])
        return val * e3m3[sb & 63] * float(tensor_scale)
    e4m3 = np.array([e4m3_value(b) for b in range(256)])
    if razer:
        special = np.where(sb & 0x80, -5.0, 5.0)
        val = np.where(nib == 8, special, val)
        sb = sb & 0x7F
    return val * e4m3[sb] * float(tensor_scale)


def gemm_f64(a_codes: np.ndarray, a_scales: np.ndarray, b_codes: np.ndarray,
             b_scales: np.ndarray, fmt: int = 0, razer: int = 0, ts_a: float = 1.0,
             ts_b: float = 1.0, razer_b: Optional[int] = None, pair: float = 0.0) -> np.ndarray:
    """C = A B^T of two quantized operands, A [m, k] and B [n, k]: each decoded
    exactly (decode_exact), then a float64 library matmul (the RaZeR page,
    technical summary sec. 2.3: the GEMM consumes the quantized weights and
    activations). razer applies to A, and to B unless razer_b says otherwise."""
    a = decode_exact(a_codes, a_scales, fmt, razer, ts_a, pair)
    b = decode_exact(b_codes, b_scales, fmt, razer if razer_b is None else razer_b, ts_b, pair)
    return a @ b.T


def rotate_r(x_bf16: np.ndarray, perm: Optional[np.ndarray], R: np.ndarray) -> np.ndarray:
    """fp32 [rows, cols]: permute channels, then y_b = R x'_b in every 32-block."""
    rows, cols = x_bf16.shape
    R = np.ascontiguousarray(R, np.float64)
    assert R.shape == (32, 32) and cols % 32 == 0
    if perm is not None:
        perm = np.ascontiguousarray(perm, np.int32)
    out = np.zeros((rows, cols), np.float32)
    _load().orc_rotate_r(_ptr(x_bf16), rows, cols, _ld(x_bf16), _ptr(perm), _ptr(R), _ptr(out),
                         cols)
    return out


def rotate_quantize_r(x_bf16: np.ndarray, perm: Optional[np.ndarray], R: np.ndarray):
    """Permutation and block matrix R, then MXFP4 quantization of the fp32 y."""
    y = rotate_r(x_bf16, perm, R)
    codes, scales = mx_quantize_f32(y)
    return codes, scales, y


def unrotate_r_f64(y: np.ndarray, perm: Optional[np.ndarray], R: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, np.float64)
    rows, cols = y.shape
    R = np.ascontiguousarray(R, np.float64)
    if perm is not None:
        perm = np.ascontiguousarray(perm, np.int32)
    out = np.zeros((rows, cols), np.float64)
    _load().orc_unrotate_r_f64(_ptr(y), rows, cols, cols, _ptr(perm), _ptr(R), _ptr(out), cols)
    return out


def apply_givens(x_bf16: np.ndarray, perm: Optional[np.ndarray], pairs: np.ndarray,
                 cs: np.ndarray) -> np.ndarray:
    """fp64 [rows, cols]: permute channels, then the Givens rotations in order
    (pairs int [n, 2] = (i, j), cs [n, 2] = (c, s))."""
    rows, cols = x_bf16.shape
    pairs = np.ascontiguousarray(pairs, np.int32).reshape(-1, 2)
    cs = np.ascontiguousarray(cs, np.float64).reshape(-1, 2)
    assert pairs.shape == cs.shape
    assert pairs.size == 0 or (pairs.min() >= 0 and pairs.max() < cols)
    if perm is not None:
        perm = np.ascontiguousarray(perm, np.int32)
    out = np.zeros((rows, cols), np.float64)
    _load().orc_apply_givens(_ptr(x_bf16), rows, cols, _ld(x_bf16), _ptr(perm), len(pairs),
                             _ptr(pairs), _ptr(cs), _ptr(out), cols)
    return out


def occupancy(y: np.ndarray) -> Tuple[np.ndarray, float]:
    """MXFP4 code-book occupancy of fp32 values (fractions per E2M1 magnitude
    index) and the occupancy-equilibrium loss (squared distance from 1/8)."""
    y = np.ascontiguousarray(y, np.float32)
    rows, cols = y.shape
    hist = np.zeros(8, np.float64)
    loss = _load().orc_occupancy(_ptr(y), rows, cols, cols, _ptr(hist))
    return hist, float(loss)


def unrotate_f64(y: np.ndarray, perm: Optional[np.ndarray], hadamard: int) -> np.ndarray:
    y = np.ascontiguousarray(y, np.float64)
    rows, cols = y.shape
    if perm is not None:
        perm = np.ascontiguousarray(perm, np.int32)
    out = np.zeros((rows, cols), np.float64)
    _load().orc_unrotate_f64(_ptr(y), rows, cols, cols, _ptr(perm), int(hadamard),
                             _ptr(out), cols)
    return out


def channel_energy(x_bf16: np.ndarray) -> np.ndarray:
    rows, cols = x_bf16.shape
    e = np.zeros(cols, np.float64)
    _load().orc_channel_energy(_ptr(x_bf16), rows, cols, _ld(x_bf16), _ptr(e))
    return e


def build_perm(energy: np.ndarray, block: int = 32, group: int = 1) -> np.ndarray:
    """Balancing permutation moving aligned runs of ``group`` channels."""
    energy = np.ascontiguousarray(energy, np.float32)
    cols = energy.size
    assert cols % block == 0 and block % group == 0
    perm = np.zeros(cols, np.int32)
    _load().orc_build_perm(_ptr(energy), cols, int(block), int(group), _ptr(perm))
    return perm


def hadamard_matrix(n: int) -> np.ndarray:
    lib = _load()
    return np.array([[lib.orc_hadamard_entry(n, i, j) for j in range(n)] for i in range(n)])


def bf16_to_f64(x_bf16: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return (x_bf16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def sqnr_db(x: np.ndarray, xhat: np.ndarray) -> float:
    """10 log10(sum x^2 / sum (x - xhat)^2) in double over the whole tensor."""
    x = np.asarray(x, np.float64)
    xhat = np.asarray(xhat, np.float64)
    num = float(np.sum(x * x))
    den = float(np.sum((x - xhat) ** 2))
    return math.inf if den == 0.0 else 10.0 * math.log10(num / den)
