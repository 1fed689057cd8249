"""The binding's argument checks on device tensors: a short or mistyped
output, permutation or tensor scale raises ValueError before the library is
called, so nothing is read or written out of bounds."""
import pytest
import torch

import block_scaled_fp4_absmax_amd as fp4

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available()
    fp4.lib()
    return torch.device("cuda:0")


def test_quantize_rejects_short_outputs(dev):
    x = torch.zeros(8, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="codes"):
        fp4.quantize(x, codes=torch.empty(8, 31, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError, match="codes"):
        fp4.quantize(x, codes=torch.empty(7, 32, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError, match="scales"):
        fp4.quantize(x, fp4.NVFP4, scales=torch.empty(8, 2, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError, match="tensor_scale"):
        fp4.quantize(x, fp4.NVFP4, tensor_scale=torch.ones(1, dtype=torch.float64, device=dev))
    with pytest.raises(ValueError, match="CUDA"):
        fp4.quantize(x, codes=torch.empty(8, 32, dtype=torch.uint8))


def test_rotate_and_dequantize_reject_bad_arguments(dev):
    x = torch.zeros(8, 64, dtype=torch.bfloat16, device=dev)
    perm64 = torch.arange(64, dtype=torch.int64, device=dev)
    with pytest.raises(ValueError, match="perm"):
        fp4.rotate_quantize(x, perm64, 32)
    with pytest.raises(ValueError, match="perm"):
        fp4.rotate_quantize(x, perm64[:32].int(), 32)
    with pytest.raises(ValueError, match="rotated"):
        fp4.rotate_quantize(x, None, 32,
                            rotated=torch.empty(8, 64, dtype=torch.float16, device=dev))
    c, s, _ = fp4.quantize(x)
    with pytest.raises(ValueError, match="scales"):
        fp4.dequantize(c, s[:4])
    with pytest.raises(ValueError, match="out"):
        fp4.dequantize(c, s, out=torch.empty(8, 63, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError, match="tensor_scale"):
        fp4.dequantize(c, torch.zeros(8, 4, dtype=torch.uint8, device=dev), fp4.NVFP4)


def test_gemm_rejects_bad_arguments(dev):
    # k = 128: 64 code bytes and 4 E8M0 scale bytes (MXFP4 scale rows are
    # read as dwords) or 8 E4M3 bytes (NVFP4) per row
    a = torch.zeros(4, 64, dtype=torch.uint8, device=dev)
    sa = torch.zeros(4, 4, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="out_dtype"):
        fp4.gemm(a, sa, a, sa, out_dtype=torch.float16)
    with pytest.raises(ValueError, match="out"):
        fp4.gemm(a, sa, a, sa, out=torch.empty(4, 3, dtype=torch.float32, device=dev))
    with pytest.raises(ValueError, match="a_scales"):
        fp4.gemm(a, sa[:, :3], a, sa)
    with pytest.raises(ValueError, match="k"):
        fp4.gemm(a, sa, a, sa, k=160)
    s8 = torch.zeros(4, 8, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="tensor scales"):
        fp4.gemm(a, s8, a, s8, fmt=fp4.NVFP4)
    out = fp4.gemm(a, sa, a, sa, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16 and out.shape == (4, 4)
    assert not out.float().any()


def test_prepared_calls_repeat_the_checked_call(dev):
    """A prepared call reruns the same launch on new contents of its inputs
    and gives what the checked call gives."""
    import numpy as np
    from block_scaled_fp4_absmax_amd import inputs
    x = torch.from_numpy(inputs.gen_c4(rows=64, cols=2048).view(np.int16)).to(dev)
    x = x.view(torch.bfloat16)
    perm = torch.randperm(2048, generator=torch.Generator().manual_seed(1)).int().to(dev)
    pq = fp4.rotate_quantize(x, perm, 32, prepare=True)
    pn = fp4.quantize(x, fp4.NVFP4, fp4.RAZER, prepare=True)
    c, s, _ = pq.run()
    cn, sn, tn = pn.run()
    pd = fp4.dequantize(c, s, fp4.MXFP4, perm=perm, hadamard=32, prepare=True)
    d = pd.run()
    pg = fp4.gemm(c, s, c, s, prepare=True)
    g = pg.run()
    for scale in (1.0, 0.5, 3.0):
        x.mul_(scale)
        c2, s2, _ = pq.run()
        cn2, sn2, tn2 = pn.run()
        d2 = pd.run()
        g2 = pg.run()
        rc, rs, _ = fp4.rotate_quantize(x, perm, 32)
        rcn, rsn, rtn = fp4.quantize(x, fp4.NVFP4, fp4.RAZER)
        rd = fp4.dequantize(rc, rs, fp4.MXFP4, perm=perm, hadamard=32)
        rg = fp4.gemm(rc, rs, rc, rs)
        torch.cuda.synchronize()
        assert c2 is c and torch.equal(c2, rc) and torch.equal(s2, rs)
        assert torch.equal(cn2, rcn) and torch.equal(sn2, rsn) and torch.equal(tn2, rtn)
        assert torch.equal(d2, rd) and torch.equal(g2, rg)
