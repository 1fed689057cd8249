"""C ABI checks that need no GPU: exports, argument validation, host code."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_scaled_fp4_absmax_amd as fp4
from block_scaled_fp4_absmax_amd import build as hip_build
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "fp4.h")


@pytest.fixture(scope="module")
def L():
    if hip_build.is_stale():
        hip_build.build()
    return fp4.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fp4_quantize", "fp4_dequantize", "fp4_rotate_quantize", "fp4_channel_energy",
              "fp4_build_permutation", "fp4_status_string", "fp4_version"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n
    assert L.fp4_version() == 1


def test_status_strings(L):
    for st in (0, -1, -2, -3, -4, -5, -99):
        assert L.fp4_status_string(st)


# fp4_quantize(x, rows, cols, ld_x, format, block, mode, flags, codes, ld_codes,
#              scales, ld_scales, tensor_scale, stream)
FAKE = 0x10000  # never dereferenced: every case below fails before any launch
TS = FAKE + 0x100


@pytest.mark.parametrize("args,want", [
    ((FAKE, 4, 64, 64, 3, 32, 0, 0, FAKE, 32, FAKE, 2, None), -4),      # bad format
    ((FAKE, 4, 64, 64, 2, 16, 0, 0, FAKE, 32, FAKE, 4, None), -4),      # MXINT4 block is 32
    ((FAKE, 4, 64, 64, 2, 32, 1, 0, FAKE, 32, FAKE, 2, None), -4),      # RaZeR on MXINT4
    ((FAKE, 4, 64, 64, 2, 32, 0, 1, FAKE, 32, FAKE, 2, None), -4),      # given s_t on MXINT4
    ((FAKE, 4, 64, 64, 0, 16, 0, 0, FAKE, 32, FAKE, 4, None), -4),      # MXFP4 needs block 32
    ((FAKE, 4, 64, 64, 1, 32, 0, 0, FAKE, 32, FAKE, 2, TS), -4),        # NVFP4 needs block 16
    ((FAKE, 4, 64, 64, 0, 32, 1, 0, FAKE, 32, FAKE, 2, None), -4),      # RaZeR needs NVFP4
    ((FAKE, 4, 64, 64, 0, 32, 0, 8, FAKE, 32, FAKE, 2, None), -4),      # unknown flag
    ((FAKE, 4, 64, 64, 0, 32, 0, 1, FAKE, 32, FAKE, 2, None), -4),      # scale-given on MXFP4
    ((FAKE, 4, 64, 64, 1, 16, 0, 2, FAKE, 32, FAKE, 4, TS), -4),        # floor rule on NVFP4
    ((FAKE, -1, 64, 64, 0, 32, 0, 0, FAKE, 32, FAKE, 2, None), -2),     # negative rows
    ((FAKE, 4, 48, 48, 0, 32, 0, 0, FAKE, 24, FAKE, 2, None), -2),      # cols % block
    ((FAKE, 4, 64, 32, 0, 32, 0, 0, FAKE, 32, FAKE, 2, None), -2),      # ld_x < cols
    ((FAKE, 4, 64, 64, 0, 32, 0, 0, FAKE, 16, FAKE, 2, None), -2),      # ld_codes < cols/2
    ((FAKE, 4, 64, 64, 0, 32, 0, 0, FAKE, 32, FAKE, 1, None), -2),      # ld_scales < cols/32
    ((None, 4, 64, 64, 0, 32, 0, 0, FAKE, 32, FAKE, 2, None), -1),      # null input
    ((FAKE, 4, 64, 64, 1, 16, 0, 0, FAKE, 32, FAKE, 4, None), -1),      # NVFP4 needs s_t slot
    ((FAKE + 2, 4, 64, 64, 0, 32, 0, 0, FAKE, 32, FAKE, 2, None), -3),  # misaligned input
    ((FAKE, 4, 64, 68, 0, 32, 0, 0, FAKE, 32, FAKE, 2, None), -3),      # ld_x % 8
    ((FAKE, 4, 64, 64, 0, 32, 0, 0, FAKE + 1, 32, FAKE, 2, None), -3),  # misaligned codes
    ((FAKE, 1 << 20, 1 << 14, 1 << 14, 0, 32, 0, 0, FAKE, 1 << 13, FAKE, 512, None), -4),  # too big
])
def test_quantize_validation(L, args, want):
    assert L.fp4_quantize(*args, None) == want


def test_empty_mxfp4_is_a_no_op(L):
    # rows == 0: nothing to do and nothing enqueued, even with NULL buffers
    assert L.fp4_quantize(None, 0, 64, 64, 0, 32, 0, 0, None, 32, None, 2, None, None) == 0


def test_rotate_and_dequant_validation(L):
    # rotate_quantize(x, rows, cols, ld, perm, had, fmt, block, mode, flags, codes, ldc,
    #                 scales, lds, ts, rot, ld_rot, stream)
    R = L.fp4_rotate_quantize
    assert R(FAKE, 4, 64, 64, None, 16, 0, 32, 0, 0, FAKE, 32, FAKE, 2, None, None, 0, None) == -4
    assert R(FAKE, 4, 64, 64, None, 32, 1, 16, 0, 0, FAKE, 32, FAKE, 4, TS, None, 0, None) == -4
    # NVFP4 rotation works on 32-element segments: cols % 32
    assert R(FAKE, 4, 48, 48, None, 16, 1, 16, 1, 0, FAKE, 24, FAKE, 3, TS, None, 0, None) == -2
    assert R(FAKE, 4, 32800, 32800, FAKE, 32, 0, 32, 0, 0, FAKE, 16400, FAKE, 1025, None, None,
             0, None) == -4  # permutation wider than the LDS row buffer (32768)
    assert R(FAKE, 4, 64, 64, None, 32, 0, 32, 0, 0, FAKE, 32, FAKE, 2, None, FAKE, 32,
             None) == -2
    assert R(FAKE, 4, 64, 64, None, 32, 0, 32, 0, 0, FAKE, 32, FAKE, 2, None, FAKE + 4, 64,
             None) == -3
    # dequantize(codes, ldc, scales, lds, ts, rows, cols, fmt, block, mode, perm, had, out, ldo, s)
    D = L.fp4_dequantize
    assert D(FAKE, 32, FAKE, 4, TS, 4, 64, 1, 16, 0, None, 32, FAKE, 64, None) == -4
    assert D(FAKE, 24, FAKE, 3, TS, 4, 48, 1, 16, 1, None, 16, FAKE, 48, None) == -2
    assert D(FAKE, 32, FAKE, 2, None, 4, 64, 0, 32, 1, None, 0, FAKE, 64, None) == -4
    assert D(FAKE, 32, FAKE, 4, None, 4, 64, 1, 16, 0, None, 0, FAKE, 64, None) == -1
    assert D(FAKE, 32, FAKE, 2, None, 4, 64, 0, 32, 0, None, 0, FAKE + 8, 64, None) == -3
    assert D(FAKE, 32, FAKE, 2, None, 0, 64, 0, 32, 0, None, 0, None, 64, None) == 0
    # gemm(a, ld_a, sa, ld_sa, ta, mode_a, b, ld_b, sb, ld_sb, tb, mode_b, m, n, k, fmt,
    #      out_dtype, c, ld_c, stream)
    def G(a=FAKE, lda=32, sa=FAKE, ldsa=4, ta=None, ma=0, b=FAKE, ldb=32, sb=FAKE, ldsb=4,
          tb=None, mb=0, m=8, n=8, k=64, fmt=0, od=0, c=FAKE, ldc=8):
        return L.fp4_gemm(a, lda, sa, ldsa, ta, ma, b, ldb, sb, ldsb, tb, mb, m, n, k, fmt, od,
                          c, ldc, None)
    assert G(fmt=2) == -4                        # MXINT4 has no GEMM
    assert G(od=2) == -4                         # output type
    assert G(ma=1) == -4                         # RaZeR needs NVFP4
    assert G(k=48) == -2                         # k % 32
    assert G(lda=16) == -2                       # ld_a < k / 2
    assert G(ldc=4) == -2                        # ld_c < n
    assert G(lda=40) == -3                       # ld_a % 16
    assert G(ldsa=6) == -3                       # MXFP4 scale rows: ld_s % 4
    assert G(a=FAKE + 8) == -3
    assert G(a=None) == -1
    assert G(a=None, sa=None, b=None, sb=None, c=None, m=0) == 0
    assert G(fmt=1, ldsa=4, ldsb=4) == -1        # NVFP4 needs both tensor scales
    assert G(fmt=1, ta=TS, tb=TS, ldsa=5, ldsb=4) == -3  # NVFP4 scale rows: ld_s % 2
    # rotate_quantize_r(x, rows, cols, ld, perm, rotation, codes, ldc, scales, lds, rot, ld_rot,
    #                   stream)
    Q = L.fp4_rotate_quantize_r
    assert Q(FAKE, 4, 48, 48, FAKE, FAKE, FAKE, 24, FAKE, 2, None, 0, None) == -2  # cols % 32
    assert Q(FAKE, 4, 64, 64, None, FAKE, FAKE, 32, FAKE, 2, None, 0, None) == -1  # perm needed
    assert Q(FAKE, 4, 64, 64, FAKE, None, FAKE, 32, FAKE, 2, None, 0, None) == -1  # matrix needed
    assert Q(FAKE, 4, 64, 64, FAKE, FAKE + 2, FAKE, 32, FAKE, 2, None, 0, None) == -3
    assert Q(FAKE, 4, 64, 64, FAKE, FAKE, FAKE, 32, FAKE, 2, FAKE, 32, None) == -2  # ld_rot
    assert Q(FAKE, 4, 32800, 32800, FAKE, FAKE, FAKE, 16400, FAKE, 1025, None, 0, None) == -4
    assert Q(None, 0, 64, 64, None, None, None, 32, None, 2, None, 0, None) == 0
    # dequantize_r(codes, ldc, scales, lds, rows, cols, perm, rotation, out, ldo, stream)
    U = L.fp4_dequantize_r
    assert U(FAKE, 24, FAKE, 2, 4, 48, FAKE, FAKE, FAKE, 48, None) == -2
    assert U(FAKE, 32, FAKE, 2, 4, 64, None, FAKE, FAKE, 64, None) == -1
    assert U(FAKE, 32, FAKE, 2, 4, 64, FAKE, FAKE, FAKE + 8, 64, None) == -3
    assert U(FAKE, 32, FAKE, 2, 4, 64, FAKE, FAKE + 1, FAKE, 64, None) == -3
    assert U(None, 32, None, 2, 0, 64, None, None, None, 64, None) == 0
    # apply_channel_rotation(x, rows, cols, ld, perm, pairs, cs, layer_start, n_layers, n_rot,
    #                        out, ld_out, stream)
    A = L.fp4_apply_channel_rotation
    assert A(FAKE, 4, 60, 64, None, FAKE, FAKE, FAKE, 1, 2, FAKE, 64, None) == -2  # cols % 8
    assert A(FAKE, 4, 64, 64, None, FAKE, FAKE, FAKE, -1, 2, FAKE, 64, None) == -2
    assert A(FAKE, 4, 32768, 32768, None, FAKE, FAKE, FAKE, 1, 2, FAKE, 32768, None) == -4
    assert A(FAKE, 4, 64, 64, None, None, FAKE, FAKE, 1, 2, FAKE, 64, None) == -1  # pairs
    assert A(FAKE, 4, 64, 64, None, FAKE, FAKE, None, 1, 2, FAKE, 64, None) == -1  # layers
    assert A(FAKE, 4, 64, 64, None, FAKE, FAKE, FAKE, 0, 2, FAKE, 64, None) == -1  # no layer
    assert A(FAKE + 2, 4, 64, 64, None, FAKE, FAKE, FAKE, 1, 2, FAKE, 64, None) == -3
    assert A(FAKE, 4, 64, 64, FAKE + 1, FAKE, FAKE, FAKE, 1, 2, FAKE, 64, None) == -3
    assert A(FAKE, 4, 64, 64, None, FAKE, FAKE, FAKE, 1, 2, FAKE, 72, None) == -4  # in place
    assert A(None, 0, 64, 64, None, None, None, None, 0, 0, None, 64, None) == 0
    E = L.fp4_channel_energy
    assert E(FAKE, 4, 48, 48, FAKE, None) == -2
    assert E(None, 4, 64, 64, FAKE, None) == -1


def test_gemm_scale_order_validation(L):
    """FP4_FLAG_SCALES_GEMM: MXFP4 only, ld_scales a multiple of 256 covering
    ceil(cols / 256) steps; in fp4_gemm it is OR-ed into an operand's mode."""
    Fg = 0x100
    Q = L.fp4_quantize
    assert Q(FAKE, 4, 64, 64, 1, 16, 0, Fg, FAKE, 32, FAKE, 256, TS, None) == -4   # NVFP4
    assert Q(FAKE, 4, 64, 64, 2, 32, 0, Fg, FAKE, 32, FAKE, 256, None, None) == -4  # MXINT4
    assert Q(FAKE, 4, 64, 64, 0, 32, 0, Fg, FAKE, 32, FAKE, 2, None, None) == -2    # < 256
    assert Q(FAKE, 4, 64, 64, 0, 32, 0, Fg, FAKE, 32, FAKE, 300, None, None) == -2  # % 256
    assert Q(FAKE, 4, 512, 512, 0, 32, 0, Fg, FAKE, 256, FAKE, 256, None, None) == -2  # 2 steps
    assert Q(None, 0, 512, 512, 0, 32, 0, Fg, None, 256, None, 512, None, None) == 0
    assert Q(None, 0, 544, 544, 0, 32, 0, Fg | 2, None, 272, None, 768, None, None) == 0
    R = L.fp4_rotate_quantize
    assert R(FAKE, 4, 64, 64, None, 16, 1, 16, 0, Fg, FAKE, 32, FAKE, 256, TS, None, 0,
             None) == -4
    assert R(FAKE, 4, 64, 64, None, 32, 0, 32, 0, Fg, FAKE, 32, FAKE, 2, None, None, 0,
             None) == -2
    assert R(None, 0, 64, 64, None, 32, 0, 32, 0, Fg, None, 32, None, 256, None, None, 0,
             None) == 0

    def G(ma=0, mb=0, ldsa=4, ldsb=4, k=64, fmt=0, m=8, ta=None, tb=None):
        return L.fp4_gemm(FAKE, 512, FAKE, ldsa, ta, ma, FAKE, 512, FAKE, ldsb, tb, mb, m, 8, k,
                          fmt, 0, FAKE, 8, None)
    assert G(ma=Fg, fmt=1, ta=TS, tb=TS) == -4   # NVFP4 scales have no GEMM order
    assert G(ma=Fg) == -2                        # ld_sa must be a 256-byte step multiple
    assert G(mb=Fg, ldsb=260) == -2
    assert G(ma=Fg, ldsa=256, k=512) == -2       # two steps of 256 k need 512
    assert G(ma=Fg | 1, ldsa=256) == -4          # RaZeR needs NVFP4
    assert G(ma=Fg, mb=Fg, ldsa=512, ldsb=512, k=512, m=0) == 0


def test_gemm_scale_shape_and_binding():
    import torch
    assert fp4.gemm_scale_shape(100, 8192) == (4, 8192)
    assert fp4.gemm_scale_shape(32, 544) == (1, 768)
    assert fp4.gemm_scale_shape(0, 0) == (0, 0)
    with pytest.raises(ValueError, match="MXFP4"):
        fp4._outputs(4, 64, fp4.NVFP4, None, gemm_scales=True)
    c, s = fp4._outputs(33, 512, fp4.MXFP4, None, torch.zeros(33, 256, dtype=torch.uint8),
                        torch.zeros(2, 512, dtype=torch.uint8), gemm_scales=True)
    assert tuple(s.shape) == (2, 512)
    with pytest.raises(ValueError, match="rows"):
        fp4._outputs(33, 512, fp4.MXFP4, None, torch.zeros(33, 256, dtype=torch.uint8),
                     torch.zeros(1, 512, dtype=torch.uint8), gemm_scales=True)


def test_binding_raises_without_gpu_work():
    with pytest.raises(fp4.Fp4Error):
        fp4._check("fp4_quantize", -2)


def test_binding_argument_checks():
    """The binding rejects wrong dtypes, host tensors, short outputs and
    unsupported output dtypes before any pointer reaches the library (the
    device-side cases are in test_gpu_binding.py)."""
    import torch
    bf = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="bfloat16"):
        fp4.quantize(bf.float())
    with pytest.raises(ValueError, match="CUDA"):
        fp4.quantize(bf)
    with pytest.raises(ValueError, match="contiguous rows"):
        fp4.quantize(bf.t())
    with pytest.raises(ValueError, match="format"):
        fp4.quantize(bf, fmt=7)
    u8 = torch.zeros(4, 32, dtype=torch.uint8)
    with pytest.raises(ValueError, match="out_dtype"):
        fp4.gemm(u8, u8, u8, u8, out_dtype=torch.float16)
    with pytest.raises(ValueError, match="out_dtype"):
        fp4.gemm(u8, u8, u8, u8, out=torch.zeros(4, 4, dtype=torch.float16))
    with pytest.raises(ValueError, match="uint8"):
        fp4.dequantize(u8.to(torch.int8), u8)
    # the helpers on host tensors (device None)
    with pytest.raises(ValueError, match="rows"):
        fp4._mat(u8, "codes", torch.uint8, None, rows=5)
    with pytest.raises(ValueError, match="columns"):
        fp4._mat(u8, "codes", torch.uint8, None, rows=4, min_cols=33)
    assert fp4._mat(u8, "codes", torch.uint8, None, rows=4, min_cols=32) == (4, 32, 32)
    with pytest.raises(ValueError, match="elements"):
        fp4._vec(torch.zeros(63, dtype=torch.int32), "perm", torch.int32, 64, None)
    with pytest.raises(ValueError, match="int32"):
        fp4._vec(torch.zeros(64, dtype=torch.int64), "perm", torch.int32, 64, None)
    with pytest.raises(ValueError, match="contiguous"):
        fp4._vec(torch.zeros(128, dtype=torch.int32)[::2], "perm", torch.int32, 64, None)


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_host_permutation_matches_oracle(L, orc, group):
    rng = np.random.default_rng(3 + group)
    for cols, block in ((64, 32), (8192, 32), (1024, 16), (28672, 32)):
        if block % group:
            continue
        e = np.exp(3 * rng.standard_normal(cols)).astype(np.float32)
        e[rng.integers(0, cols, cols // 8)] = e[0]  # plenty of exact ties
        want = orc.build_perm(e, block, group)
        got = np.zeros(cols, np.int32)
        assert L.fp4_build_permutation(e.ctypes.data, cols, block, group, got.ctypes.data) == 0
        assert np.array_equal(got, want)
    bad = np.zeros(64, np.int32)
    assert L.fp4_build_permutation(e.ctypes.data, 48, 32, group, bad.ctypes.data) == -2
    assert L.fp4_build_permutation(None, 64, 32, group, bad.ctypes.data) == -1
    assert L.fp4_build_permutation(e.ctypes.data, 64, 32, 3, bad.ctypes.data) == -4
