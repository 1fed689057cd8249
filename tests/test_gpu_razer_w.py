"""GPU parity of RaZeR for weights (E3M3 block scale, four special values).

"RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
Remapping", technical summary sec. 2.1-2.2. Codes, scale bytes, tensor scale
and decoded bf16 must be bit-exact with the oracle; the GEMM with weight-
RaZeR B operands meets the fp32 accumulation bound of the GEMM tests.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_scaled_fp4_absmax_amd as fp4
from block_scaled_fp4_absmax_amd import inputs
from conftest import read_golden
from parity_util import bf16_bits, note, same_bf16, to_dev

pytestmark = pytest.mark.gpu


def _pair():
    for ln in read_golden("razer_w_pair.txt"):
        if ln.startswith("pair"):
            return float(ln.split()[1])
    raise AssertionError("no pair in razer_w_pair.txt")


PAIR = _pair()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp4.lib()


def np_u8(t):
    return t.cpu().numpy()


def _f32_bits(v):
    return np.float32(v).view(np.uint32)


@pytest.mark.parametrize("t,rows", [(0, 512), (1, 256), (4, 128), (6, 64)])
def test_razer_w_layer_weights(orc, t, rows):
    name, _, cols = inputs.C5_SHAPES[t]
    note(f"case: RaZeR-W weights {name} {rows}x{cols}")
    x = inputs.gen_c5(t, rows=rows)
    c, s, ts = fp4.quantize(to_dev(x), fp4.NVFP4, fp4.RAZER_W)
    d = fp4.dequantize(c, s, fp4.NVFP4, fp4.RAZER_W, ts)
    torch.cuda.synchronize()
    oc, os_, ots = orc.nvw_quantize(x, PAIR)
    assert _f32_bits(ts.cpu().numpy()[0]) == _f32_bits(ots)
    assert np.array_equal(np_u8(s), os_)
    assert np.array_equal(np_u8(c), oc)
    assert np.array_equal(bf16_bits(d), orc.dequantize(oc, os_, 1, 2, ots, PAIR))
    assert ((os_ >> 6) >= 2).any() and ((os_ >> 6) < 2).any()


@pytest.mark.parametrize("shrink", [1.0, 1e-3])
def test_razer_w_given_tensor_scale(orc, shrink):
    note(f"case: RaZeR-W with a given tensor scale x{shrink}")
    x = inputs.gen_c2(rows=256, cols=2048)
    st = np.float32(orc.nvw_tensor_scale(orc.nv_tensor_amax(x)) * shrink)
    tst = torch.tensor([st], device="cuda")
    c, s, _ = fp4.quantize(to_dev(x), fp4.NVFP4, fp4.RAZER_W, tensor_scale=tst)
    torch.cuda.synchronize()
    oc, os_, _ = orc.nvw_quantize(x, PAIR, float(st))
    assert np.array_equal(np_u8(s), os_) and np.array_equal(np_u8(c), oc)


def test_razer_w_dequant_every_code_and_scale(orc):
    note("case: RaZeR-W dequantize every code x scale byte")
    rows, cols = 256, 512
    codes = np.tile(np.arange(256, dtype=np.uint8), (rows, 1))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], cols // 16, axis=1)
    ts = np.float32(0.37109375)
    d = fp4.dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                       fp4.NVFP4, fp4.RAZER_W, torch.tensor([ts], device="cuda"))
    torch.cuda.synchronize()
    assert same_bf16(bf16_bits(d), orc.dequantize(codes, scales, 1, 2, float(ts), PAIR))


@pytest.mark.parametrize("rows,cols", [(1, 16), (7, 96), (33, 160), (129, 4128)])
def test_razer_w_strided_ragged(orc, rows, cols):
    note(f"case: RaZeR-W strided {rows}x{cols}")
    x_full = inputs.gen_c5(2, rows=rows, cols=cols + 24)
    xt = to_dev(x_full)[:, :cols]
    x = np.ascontiguousarray(x_full[:, :cols])
    cbuf = torch.full((rows, cols // 2 + 12), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((rows, cols // 16 + 5), 0xCD, dtype=torch.uint8, device="cuda")
    c, s = cbuf[:, :cols // 2], sbuf[:, :cols // 16]
    _, _, ts = fp4.quantize(xt, fp4.NVFP4, fp4.RAZER_W, codes=c, scales=s)
    torch.cuda.synchronize()
    oc, os_, ots = orc.nvw_quantize(x, PAIR)
    assert float(ts.cpu()[0]) == ots
    assert np.array_equal(np_u8(c), oc) and np.array_equal(np_u8(s), os_)
    assert np.all(np_u8(cbuf)[:, cols // 2:] == 0xAB) and np.all(np_u8(sbuf)[:, cols // 16:] == 0xCD)


def test_razer_w_zero_tensor(orc):
    note("case: RaZeR-W all-zero tensor")
    x = np.zeros((8, 64), np.uint16)
    c, s, ts = fp4.quantize(to_dev(x), fp4.NVFP4, fp4.RAZER_W)
    torch.cuda.synchronize()
    assert float(ts.cpu()[0]) == 1.0 and not np_u8(c).any() and not np_u8(s).any()


@pytest.mark.parametrize("m,n,k", [(128, 256, 1024), (2048, 2048, 512), (16, 512, 2048)])
def test_gemm_razer_activations_razer_w_weights(orc, m, n, k):
    """The pages' weight-and-activation setting: activations NVFP4 + RaZeR,
    weights RaZeR for weights, both quantized on the GPU, then the GEMM."""
    note(f"case: GEMM RaZeR activations x RaZeR-W weights {m}x{n}x{k}")
    xa = inputs.gen_c3(rows=m, cols=k)
    xw = inputs.gen_c5(0, rows=n, cols=k)
    ca, sa, ta = fp4.quantize(to_dev(xa), fp4.NVFP4, fp4.RAZER)
    cw, sw, tw = fp4.quantize(to_dev(xw), fp4.NVFP4, fp4.RAZER_W)
    out = fp4.gemm(ca, sa, cw, sw, fmt=fp4.NVFP4, a_ts=ta, b_ts=tw, mode_a=fp4.RAZER,
                   mode_b=fp4.RAZER_W)
    torch.cuda.synchronize()
    ac, as_, bc, bs = (t.cpu().numpy() for t in (ca, sa, cw, sw))
    fa, fb = float(ta.cpu()[0]), float(tw.cpu()[0])
    want = orc.gemm_f64(ac, as_, bc, bs, 1, 1, fa, fb, razer_b=2, pair=PAIR)
    a = np.abs(orc.decode_exact(ac, as_, 1, 1, fa))
    b = np.abs(orc.decode_exact(bc, bs, 1, 2, fb, PAIR))
    tol = 2.0 ** -22 * (k / 16 + 1) * (a @ b.T) + 2.0 ** -22 * np.abs(want)
    err = np.abs(out.cpu().numpy() - want)
    assert np.all(err <= tol), f"max err {err.max()}"
