"""Block-scaled 4-bit (MXFP4 / NVFP4 / MXINT4, RaZeR, two-level rotation) for MI355X.

Thin Python binding over the C ABI in ``include/fp4.h`` (``libfp4.so``, built
in-tree by ``block_scaled_fp4_absmax_amd.build``). Every step of the path runs
in the library's HIP kernels; this module only allocates outputs with torch,
passes pointers, sizes and torch's current stream, and turns a non-zero status
into an exception. There is no fallback: if the library is missing, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "MXFP4", "NVFP4", "MXINT4", "PLAIN", "RAZER", "RAZER_W", "FLAG_TENSOR_SCALE_GIVEN", "FLAG_SCALE_OCP_FLOOR",
    "FLAG_SCALES_GEMM", "gemm_scale_shape",
    "Fp4Error", "lib", "library_path", "quantize", "dequantize", "rotate_quantize",
    "channel_energy", "build_permutation", "block_of", "gemm", "OUT_F32", "OUT_BF16",
    "rotate_quantize_r", "dequantize_r", "calibrate_block_rotation",
    "calibrate_macro_rotation", "apply_channel_rotation", "MacroRotation", "Prepared",
]

MXFP4, NVFP4, MXINT4 = 0, 1, 2
PLAIN, RAZER, RAZER_W = 0, 1, 2
FLAG_TENSOR_SCALE_GIVEN = 1
FLAG_SCALE_OCP_FLOOR = 2
FLAG_SCALES_GEMM = 0x100
OUT_F32, OUT_BF16 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfp4.so")
_lib = None


class Fp4Error(RuntimeError):
    """A libfp4 call returned a non-zero fp4_status."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libfp4.so with argument types set (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -m block_scaled_fp4_absmax_amd.build` "
            "or __graft_entry__.build() first")
    L = ctypes.CDLL(_LIB_PATH)
    i64, i32, u32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p
    sig = {
        "fp4_version": (i32, []),
        "fp4_status_string": (ctypes.c_char_p, [i32]),
        "fp4_quantize": (i32, [vp, i64, i64, i64, i32, i32, i32, u32, vp, i64, vp, i64, vp, vp]),
        "fp4_dequantize": (i32, [vp, i64, vp, i64, vp, i64, i64, i32, i32, i32, vp, i32, vp, i64,
                                 vp]),
        "fp4_rotate_quantize": (i32, [vp, i64, i64, i64, vp, i32, i32, i32, i32, u32, vp, i64, vp,
                                      i64, vp, vp, i64, vp]),
        "fp4_channel_energy": (i32, [vp, i64, i64, i64, vp, vp]),
        "fp4_gemm": (i32, [vp, i64, vp, i64, vp, i32, vp, i64, vp, i64, vp, i32, i64, i64, i64,
                           i32, i32, vp, i64, vp]),
        "fp4_build_permutation": (i32, [vp, i64, i32, i32, vp]),
        "fp4_rotate_quantize_r": (i32, [vp, i64, i64, i64, vp, vp, vp, i64, vp, i64, vp, i64,
                                        vp]),
        "fp4_dequantize_r": (i32, [vp, i64, vp, i64, i64, i64, vp, vp, vp, i64, vp]),
        "fp4_calibrate_block_rotation": (i32, [vp, i64, i64, i64, vp, i32, i32, vp, vp]),
        "fp4_calibrate_macro_rotation": (i32, [vp, i64, i64, i64, vp, i32, ctypes.c_double, i32,
                                               vp, vp, vp, vp, vp, vp]),
        "fp4_apply_channel_rotation": (i32, [vp, i64, i64, i64, vp, vp, vp, vp, i32, i32, vp,
                                             i64, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise Fp4Error(fn, status, lib().fp4_status_string(status).decode())


class Prepared:
    """A checked library call bound to its tensors, for loops that repeat the
    same call (serving, benchmarks): ``run()`` enqueues it again with no
    argument checks and no allocation and returns the same output tensors.
    It runs on the stream given when it was prepared, else on the caller's
    current stream at each run (so it can be captured in a graph). The
    tensors must stay alive and unchanged in shape and storage."""

    def __init__(self, name: str, args: tuple, outputs, stream_given: bool):
        fn = getattr(lib(), name)
        # arguments converted to their ctypes types once (the stream is last)
        self._fn = fn
        self._args = [a if a is None or isinstance(a, ctypes._SimpleCData) else t(a)
                      for t, a in zip(fn.argtypes, args)]
        self._name = name
        self._fixed_stream = stream_given
        self.outputs = outputs

    def run(self, stream=None):
        if stream is not None or not self._fixed_stream:
            self._args[-1] = _stream(stream)
        st = self._fn(*self._args)
        if st:
            _check(self._name, st)
        return self.outputs


def _call(name: str, args: tuple, outputs, prepare: bool, stream=None):
    """Run a checked call now, or return it as a Prepared call."""
    if prepare:
        return Prepared(name, args, outputs, stream is not None)
    _check(name, getattr(lib(), name)(*args))
    return outputs


def block_of(fmt: int) -> int:
    return 16 if fmt == NVFP4 else 32


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


# ---- argument checks --------------------------------------------------------
# The C ABI sees pointers, sizes and strides only, so a tensor of the wrong
# dtype, device or size would be read or written out of bounds. Every
# argument is checked here before its pointer is passed: dtype, 2-D with
# contiguous rows (or a contiguous vector), enough rows and columns, and the
# device of the call.


def _mat(t, name, dtype, device, rows=None, min_cols=0, exact_rows=True):
    """Check a 2-D argument; returns (rows, cols, row stride)."""
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1) or t.stride(0) < 0:
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    if rows is not None and (t.shape[0] != rows if exact_rows else t.shape[0] < rows):
        raise ValueError(f"{name} has {t.shape[0]} rows, {rows} needed")
    if t.shape[1] < min_cols:
        raise ValueError(f"{name} has {t.shape[1]} columns, at least {min_cols} needed")
    _on(t, name, device)
    return t.shape[0], t.shape[1], t.stride(0)


def _vec(t, name, dtype, n, device):
    """Check a contiguous vector argument of at least n elements."""
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < n:
        raise ValueError(f"{name} has {t.numel()} elements, at least {n} needed")
    _on(t, name, device)


def _on(t, name, device):
    if device is None:  # host argument
        if t.device.type != "cpu":
            raise ValueError(f"{name} must be a host tensor")
        return
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")


def _device_of(x):
    """The device of the call: the first tensor argument's (checked to be a
    HIP device by the first _mat / _vec on it)."""
    return x.device


def _check_fmt(fmt, mode):
    if fmt not in (MXFP4, NVFP4, MXINT4):
        raise ValueError(f"unknown format {fmt}")
    if mode not in (PLAIN, RAZER, RAZER_W):
        raise ValueError(f"unknown mode {mode}")


def gemm_scale_shape(rows: int, cols: int):
    """Shape of an MXFP4 scale array in the GEMM order (FLAG_SCALES_GEMM):
    one row of 256-byte steps per group of 32 rows, a step per 256 columns."""
    return ((rows + 31) // 32, 256 * ((cols + 255) // 256))


def _outputs(rows, cols, fmt, device, codes=None, scales=None, gemm_scales=False):
    import torch
    if gemm_scales and fmt != MXFP4:
        raise ValueError("scales in the GEMM order are MXFP4 only")
    sshape = gemm_scale_shape(rows, cols) if gemm_scales else (rows, cols // block_of(fmt))
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.uint8, device=device)
    _mat(codes, "codes", torch.uint8, device, rows, cols // 2)
    _mat(scales, "scales", torch.uint8, device, *sshape)
    return codes, scales


def _tensor_scale(tensor_scale, device):
    import torch
    if tensor_scale is None:
        return torch.empty(1, dtype=torch.float32, device=device)
    _vec(tensor_scale, "tensor_scale", torch.float32, 1, device)
    return tensor_scale


def quantize(x, fmt: int = MXFP4, mode: int = PLAIN, floor_rule: bool = False,
             tensor_scale=None, scale_given: Optional[bool] = None, codes=None, scales=None,
             stream=None, prepare: bool = False, gemm_scales: bool = False):
    """Quantize a bf16 [rows, cols] CUDA tensor.

    Returns (codes uint8 [rows, cols/2], scales uint8 [rows, cols/block],
    tensor_scale fp32 [1] for NVFP4 else None); with ``gemm_scales`` (MXFP4)
    the scales come in the GEMM order, shape :func:`gemm_scale_shape`. For
    NVFP4, ``tensor_scale`` is
    a 1-element fp32 device tensor: read as s_t when ``scale_given`` (the
    default when it is passed), otherwise it receives the computed s_t
    (allocated when None). ``prepare=True`` returns a :class:`Prepared` call
    instead of running it (so does every other entry point that enqueues work).
    """
    import torch
    _check_fmt(fmt, mode)
    dev = _device_of(x)
    rows, cols, ld = _mat(x, "x", torch.bfloat16, dev)
    codes, scales = _outputs(rows, cols, fmt, dev, codes, scales, gemm_scales)
    flags = (FLAG_SCALE_OCP_FLOOR if floor_rule else 0) | (FLAG_SCALES_GEMM if gemm_scales else 0)
    ts = None
    if fmt == NVFP4:
        if scale_given is None:
            scale_given = tensor_scale is not None
        if scale_given:
            if tensor_scale is None:
                raise ValueError("scale_given needs a tensor_scale")
            flags |= FLAG_TENSOR_SCALE_GIVEN
        ts = _tensor_scale(tensor_scale, dev)
    return _call("fp4_quantize",
                 (_ptr(x), rows, cols, ld, fmt, block_of(fmt), mode, flags, _ptr(codes),
                  codes.stride(0), _ptr(scales), scales.stride(0), _ptr(ts), _stream(stream)),
                 (codes, scales, ts), prepare, stream)


def dequantize(codes, scales, fmt: int = MXFP4, mode: int = PLAIN, tensor_scale=None,
               perm=None, hadamard: int = 0, out=None, stream=None, prepare: bool = False):
    """Decode to a bf16 [rows, cols] tensor (optionally undoing a rotation)."""
    import torch
    _check_fmt(fmt, mode)
    dev = _device_of(codes)
    rows, half, ldc = _mat(codes, "codes", torch.uint8, dev)
    cols = half * 2
    _mat(scales, "scales", torch.uint8, dev, rows, cols // block_of(fmt))
    if fmt == NVFP4:
        if tensor_scale is None:
            raise ValueError("NVFP4 needs its tensor_scale")
        _vec(tensor_scale, "tensor_scale", torch.float32, 1, dev)
    if perm is not None:
        _vec(perm, "perm", torch.int32, cols, dev)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    _mat(out, "out", torch.bfloat16, dev, rows, cols)
    return _call("fp4_dequantize",
                 (_ptr(codes), ldc, _ptr(scales), scales.stride(0), _ptr(tensor_scale), rows,
                  cols, fmt, block_of(fmt), mode, _ptr(perm), hadamard, _ptr(out), out.stride(0),
                  _stream(stream)), out, prepare, stream)


def rotate_quantize(x, perm=None, hadamard: Optional[int] = None, floor_rule: bool = False,
                    want_rotated: bool = False, codes=None, scales=None, rotated=None,
                    fmt: int = MXFP4, mode: int = PLAIN, tensor_scale=None,
                    scale_given: Optional[bool] = None, stream=None, prepare: bool = False,
                    gemm_scales: bool = False):
    """Permutation + block Hadamard fused with FP4 quantize + pack.

    ``hadamard`` defaults to the format's block size (32 MXFP4, 16 NVFP4); 0
    turns the transform off. NVFP4 takes ``mode`` (PLAIN or RAZER) and a
    tensor scale as in :func:`quantize`. Returns (codes, scales, rotated fp32
    [rows, cols] or None) for MXFP4 and MXINT4, and (codes, scales, rotated,
    tensor_scale) for NVFP4. ``gemm_scales`` (MXFP4): scales in the GEMM
    order, as for :func:`quantize`.
    """
    import torch
    _check_fmt(fmt, mode)
    dev = _device_of(x)
    rows, cols, ld = _mat(x, "x", torch.bfloat16, dev)
    if hadamard is None:
        hadamard = block_of(fmt)
    if perm is not None:
        _vec(perm, "perm", torch.int32, cols, dev)
    codes, scales = _outputs(rows, cols, fmt, dev, codes, scales, gemm_scales)
    if want_rotated and rotated is None:
        rotated = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    if rotated is not None:
        _mat(rotated, "rotated", torch.float32, dev, rows, cols)
    flags = (FLAG_SCALE_OCP_FLOOR if floor_rule else 0) | (FLAG_SCALES_GEMM if gemm_scales else 0)
    ts = None
    if fmt == NVFP4:
        if scale_given is None:
            scale_given = tensor_scale is not None
        if scale_given:
            if tensor_scale is None:
                raise ValueError("scale_given needs a tensor_scale")
            flags |= FLAG_TENSOR_SCALE_GIVEN
        ts = _tensor_scale(tensor_scale, dev)
    return _call("fp4_rotate_quantize",
                 (_ptr(x), rows, cols, ld, _ptr(perm), hadamard, fmt, block_of(fmt), mode, flags,
                  _ptr(codes), codes.stride(0), _ptr(scales), scales.stride(0), _ptr(ts),
                  _ptr(rotated), rotated.stride(0) if rotated is not None else 0,
                  _stream(stream)),
                 (codes, scales, rotated, ts) if fmt == NVFP4 else (codes, scales, rotated),
                 prepare, stream)


def gemm(a_codes, a_scales, b_codes, b_scales, k: Optional[int] = None, fmt: int = MXFP4,
         a_ts=None, b_ts=None, mode_a: int = PLAIN, mode_b: int = PLAIN, out_dtype=None,
         out=None, stream=None, prepare: bool = False, a_gemm_scales: bool = False,
         b_gemm_scales: bool = False):
    """C = A B^T for quantized A [m, k] and B [n, k] (codes and scales as the
    quantizer returns them; NVFP4 also takes the two tensor scales and a mode
    per operand); fp32 [m, n] unless ``out_dtype`` is bfloat16.
    ``a_gemm_scales`` / ``b_gemm_scales`` (MXFP4): that operand's scales are
    in the GEMM order (a quantizer called with ``gemm_scales=True``)."""
    import torch
    if fmt not in (MXFP4, NVFP4):
        raise ValueError(f"fp4_gemm takes MXFP4 or NVFP4, got format {fmt}")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"out_dtype must be torch.float32 or torch.bfloat16, got {out_dtype}")
    dev = _device_of(a_codes)
    m, ha, lda = _mat(a_codes, "a_codes", torch.uint8, dev)
    n, hb, ldb = _mat(b_codes, "b_codes", torch.uint8, dev)
    if k is None:
        k = 2 * ha
    if k > 2 * ha or k > 2 * hb:
        raise ValueError(f"k = {k} exceeds the code rows ({2 * ha}, {2 * hb} elements)")
    blk = block_of(fmt)
    if (a_gemm_scales or b_gemm_scales) and fmt != MXFP4:
        raise ValueError("scales in the GEMM order are MXFP4 only")
    _mat(a_scales, "a_scales", torch.uint8, dev,
         *(gemm_scale_shape(m, k) if a_gemm_scales else (m, k // blk)))
    _mat(b_scales, "b_scales", torch.uint8, dev,
         *(gemm_scale_shape(n, k) if b_gemm_scales else (n, k // blk)))
    mode_a |= FLAG_SCALES_GEMM if a_gemm_scales else 0
    mode_b |= FLAG_SCALES_GEMM if b_gemm_scales else 0
    if fmt == NVFP4:
        if a_ts is None or b_ts is None:
            raise ValueError("NVFP4 needs both tensor scales")
        _vec(a_ts, "a_ts", torch.float32, 1, dev)
        _vec(b_ts, "b_ts", torch.float32, 1, dev)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    if out.dtype != out_dtype:
        raise ValueError(f"out is {out.dtype}, out_dtype is {out_dtype}")
    _mat(out, "out", out_dtype, dev, m, n)
    od = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    return _call("fp4_gemm",
                 (_ptr(a_codes), lda, _ptr(a_scales), a_scales.stride(0), _ptr(a_ts), mode_a,
                  _ptr(b_codes), ldb, _ptr(b_scales), b_scales.stride(0), _ptr(b_ts), mode_b,
                  m, n, k, fmt, od, _ptr(out), out.stride(0), _stream(stream)), out, prepare, stream)


def channel_energy(x, out=None, stream=None, prepare: bool = False):
    """fp32 [cols]: sum over rows of x^2 per channel (fp64 accumulation)."""
    import torch
    dev = _device_of(x)
    rows, cols, ld = _mat(x, "x", torch.bfloat16, dev)
    if out is None:
        out = torch.empty(cols, dtype=torch.float32, device=dev)
    _vec(out, "out", torch.float32, cols, dev)
    return _call("fp4_channel_energy", (_ptr(x), rows, cols, ld, _ptr(out), _stream(stream)),
                 out, prepare, stream)


def build_permutation(energy, block: int = 32, group: int = 1):
    """int32 [cols] host tensor: magnitude-balancing permutation (host code)
    moving aligned runs of ``group`` channels (1, 2, 4 or 8)."""
    import torch
    e = energy.detach().to("cpu", torch.float32).contiguous()
    perm = torch.empty(e.numel(), dtype=torch.int32)
    st = lib().fp4_build_permutation(_ptr(e), e.numel(), block, group, _ptr(perm))
    _check("fp4_build_permutation", st)
    return perm


def rotate_quantize_r(x, perm, rotation, want_rotated: bool = False, codes=None, scales=None,
                      rotated=None, stream=None, prepare: bool = False):
    """Permutation + learned 32x32 block matrix (fp32 [32, 32] device tensor,
    R row-major) fused with MXFP4 quantize + pack. Returns (codes, scales,
    rotated fp32 [rows, cols] or None)."""
    import torch
    dev = _device_of(x)
    rows, cols, ld = _mat(x, "x", torch.bfloat16, dev)
    _vec(perm, "perm", torch.int32, cols, dev)
    _vec(rotation, "rotation", torch.float32, 32 * 32, dev)
    codes, scales = _outputs(rows, cols, MXFP4, dev, codes, scales)
    if want_rotated and rotated is None:
        rotated = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    if rotated is not None:
        _mat(rotated, "rotated", torch.float32, dev, rows, cols)
    return _call("fp4_rotate_quantize_r",
                 (_ptr(x), rows, cols, ld, _ptr(perm), _ptr(rotation), _ptr(codes),
                  codes.stride(0), _ptr(scales), scales.stride(0), _ptr(rotated),
                  rotated.stride(0) if rotated is not None else 0, _stream(stream)),
                 (codes, scales, rotated), prepare, stream)


def dequantize_r(codes, scales, perm, rotation, out=None, stream=None, prepare: bool = False):
    """Inverse of :func:`rotate_quantize_r`: decode, R^T per block, undo the
    permutation; bf16 [rows, cols]."""
    import torch
    dev = _device_of(codes)
    rows, half, ldc = _mat(codes, "codes", torch.uint8, dev)
    cols = half * 2
    _mat(scales, "scales", torch.uint8, dev, rows, cols // 32)
    _vec(perm, "perm", torch.int32, cols, dev)
    _vec(rotation, "rotation", torch.float32, 32 * 32, dev)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    _mat(out, "out", torch.bfloat16, dev, rows, cols)
    return _call("fp4_dequantize_r",
                 (_ptr(codes), ldc, _ptr(scales), scales.stride(0), rows, cols, _ptr(perm),
                  _ptr(rotation), _ptr(out), out.stride(0), _stream(stream)), out, prepare, stream)


def calibrate_block_rotation(x, perm=None, iters: int = 60, angles: int = 32):
    """Learn the block matrix R on a bf16 calibration sample (host code).

    ``x`` is a bf16 tensor (any device; copied to the host) and ``perm`` the
    permutation that will be used online (host or device int32, or None).
    The cost grows as iters * angles * x.numel() / 32: pass a sample of rows
    (a few hundred rows of 8192 take seconds). Returns (R fp32 [32, 32] host
    tensor, (loss of H / sqrt(32), loss of R)).
    """
    import torch
    xh = x.detach().to("cpu").contiguous()
    rows, cols, ld = _mat(xh, "x", torch.bfloat16, None)
    ph = None if perm is None else perm.detach().to("cpu", torch.int32).contiguous()
    if ph is not None and ph.numel() != cols:
        raise ValueError(f"perm has {ph.numel()} entries, {cols} needed")
    R = torch.empty((32, 32), dtype=torch.float32)
    loss = (ctypes.c_double * 2)()
    st = lib().fp4_calibrate_block_rotation(_ptr(xh), rows, cols, ld, _ptr(ph), iters, angles,
                                            _ptr(R), ctypes.cast(loss, ctypes.c_void_p))
    _check("fp4_calibrate_block_rotation", st)
    return R, (loss[0], loss[1])


class MacroRotation:
    """The inter-block Givens transform: ``pairs`` int32 [n, 2], ``cs`` fp32
    [n, 2] (cos, sin), ``layer_start`` int32 [layers + 1] (host tensors), and
    the relative block-variance spread before and after."""

    def __init__(self, pairs, cs, layer_start, spread):
        self.pairs, self.cs, self.layer_start, self.spread = pairs, cs, layer_start, spread

    @property
    def n_rot(self) -> int:
        return int(self.pairs.shape[0])

    @property
    def n_layers(self) -> int:
        return int(self.layer_start.numel()) - 1

    def to(self, device):
        return MacroRotation(self.pairs.to(device), self.cs.to(device),
                             self.layer_start.to(device), self.spread)


def calibrate_macro_rotation(x, perm=None, block: int = 32, tol: float = 1e-6,
                             max_rot: Optional[int] = None) -> MacroRotation:
    """Givens rotations that equalise the block variances of the bf16 sample
    ``x`` after ``perm`` (host code; x is copied to the host)."""
    import torch
    xh = x.detach().to("cpu").contiguous()
    rows, cols, ld = _mat(xh, "x", torch.bfloat16, None)
    if max_rot is None:
        max_rot = 4 * (cols // block)
    ph = None if perm is None else perm.detach().to("cpu", torch.int32).contiguous()
    if ph is not None and ph.numel() != cols:
        raise ValueError(f"perm has {ph.numel()} entries, {cols} needed")
    pairs = torch.empty((max_rot, 2), dtype=torch.int32)
    cs = torch.empty((max_rot, 2), dtype=torch.float32)
    starts = torch.empty(max_rot + 1, dtype=torch.int32)
    n_rot, n_layers = ctypes.c_int(0), ctypes.c_int(0)
    spread = (ctypes.c_double * 2)()
    st = lib().fp4_calibrate_macro_rotation(
        _ptr(xh), rows, cols, ld, _ptr(ph), block, float(tol), max_rot, _ptr(pairs), _ptr(cs),
        _ptr(starts), ctypes.byref(n_rot), ctypes.byref(n_layers),
        ctypes.cast(spread, ctypes.c_void_p))
    _check("fp4_calibrate_macro_rotation", st)
    n, nl = n_rot.value, n_layers.value
    return MacroRotation(pairs[:n].clone(), cs[:n].clone(), starts[:nl + 1].clone(),
                         (spread[0], spread[1]))


def apply_channel_rotation(x, macro: MacroRotation, perm=None, out=None, stream=None,
                           prepare: bool = False):
    """bf16 [rows, cols]: permutation, then the Givens layers of ``macro``
    (device tensors, see :meth:`MacroRotation.to`), on every row."""
    import torch
    dev = _device_of(x)
    rows, cols, ld = _mat(x, "x", torch.bfloat16, dev)
    if perm is not None:
        _vec(perm, "perm", torch.int32, cols, dev)
    _vec(macro.pairs, "pairs", torch.int32, 2 * macro.n_rot, dev)
    _vec(macro.cs, "cs", torch.float32, 2 * macro.n_rot, dev)
    _vec(macro.layer_start, "layer_start", torch.int32, macro.n_layers + 1, dev)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    _mat(out, "out", torch.bfloat16, dev, rows, cols)
    return _call("fp4_apply_channel_rotation",
                 (_ptr(x), rows, cols, ld, _ptr(perm), _ptr(macro.pairs), _ptr(macro.cs),
                  _ptr(macro.layer_start), macro.n_layers, macro.n_rot, _ptr(out), out.stride(0),
                  _stream(stream)), out, prepare, stream)
