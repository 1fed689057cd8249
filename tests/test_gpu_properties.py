"""Property tests of the quantizers (hypothesis): random shapes, row-stride
padding, formats, modes and scale rules, each through the C ABI on the GPU
and bit-exact against the oracle (codes, scale bytes, s_t, decoded bf16),
with the padding of every strided buffer left untouched. Derandomised, so a
run is reproducible."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import block_scaled_fp4_absmax_amd as fp4  # noqa: E402
from conftest import read_golden  # noqa: E402
from parity_util import bf16_bits, note, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu

PAIR = next(float(ln.split()[1]) for ln in read_golden("razer_w_pair.txt") if ln.startswith("pair"))

# (format, mode, floor rule)
VARIANTS = [(0, 0, False), (0, 0, True), (2, 0, False), (2, 0, True), (1, 0, False),
            (1, 1, False), (1, 2, False)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp4.lib()


def _tensor(seed, rows, cols, kind):
    rng = np.random.default_rng(seed)
    if kind == 0:    # Gaussian with outliers
        x = rng.standard_normal((rows, cols)) * 0.02
        k = max(1, rows * cols // 500)
        x.flat[rng.choice(rows * cols, k, replace=False)] *= 40
    elif kind == 1:  # heavy tails
        x = rng.standard_t(2, (rows, cols))
    else:            # blocks spanning many binades, with zero blocks
        x = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-40, 40, (rows, cols // 16)))\
            .repeat(16, axis=1)
        x[:, : cols // 4] *= rng.integers(0, 2, (rows, 1))
    return (x.astype(np.float32).view(np.uint32) + 0x8000 >> 16).astype(np.uint16)


@settings(max_examples=40, deadline=None, derandomize=True)
@given(rows=st.integers(1, 70), nblk=st.integers(1, 40), var=st.sampled_from(VARIANTS),
       pad_x=st.sampled_from([0, 8, 40]), pad_c=st.sampled_from([0, 4, 12]),
       pad_s=st.sampled_from([0, 1, 5]), kind=st.integers(0, 2), seed=st.integers(0, 10 ** 6))
def test_quantize_dequantize_properties(orc, rows, nblk, var, pad_x, pad_c, pad_s, kind, seed):
    fmt, mode, floor_rule = var
    blk = 16 if fmt == 1 else 32
    cols = nblk * 32
    note(f"case: property fmt={fmt} mode={mode} floor={floor_rule} {rows}x{cols} "
         f"pads={pad_x},{pad_c},{pad_s} kind={kind} seed={seed}")
    x = _tensor(seed, rows, cols, kind)
    xbuf = torch.zeros((rows, cols + pad_x), dtype=torch.bfloat16, device="cuda")
    xbuf[:, :cols] = to_dev(x)
    cbuf = torch.full((rows, cols // 2 + pad_c), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((rows, cols // blk + pad_s), 0xCD, dtype=torch.uint8, device="cuda")
    c, s = cbuf[:, :cols // 2], sbuf[:, :cols // blk]
    _, _, ts = fp4.quantize(xbuf[:, :cols], fmt, mode, floor_rule=floor_rule, codes=c, scales=s)
    obuf = torch.full((rows, cols + 8), 1.0, dtype=torch.bfloat16, device="cuda")
    fp4.dequantize(c, s, fmt, mode, ts, out=obuf[:, :cols])
    torch.cuda.synchronize()
    if fmt == 0:
        oc, os_ = orc.mx_quantize(x, floor_rule)
        od = orc.dequantize(oc, os_, 0)
    elif fmt == 2:
        oc, os_ = orc.mxint4_quantize(x, floor_rule)
        od = orc.dequantize(oc, os_, 2)
    elif mode == 2:
        oc, os_, ots = orc.nvw_quantize(x, PAIR)
        assert float(ts.cpu()[0]) == ots
        od = orc.dequantize(oc, os_, 1, 2, ots, PAIR)
    else:
        oc, os_, ots = orc.nv_quantize(x, mode == 1)
        assert float(ts.cpu()[0]) == ots
        od = orc.dequantize(oc, os_, 1, mode, ots)
    assert np.array_equal(c.cpu().numpy(), oc)
    assert np.array_equal(s.cpu().numpy(), os_)
    got = bf16_bits(obuf[:, :cols])
    nan_g = (got & 0x7F80) == 0x7F80
    assert np.array_equal(got[~nan_g], od[~nan_g]) and np.array_equal(nan_g, (od & 0x7F80) == 0x7F80)
    assert np.all(cbuf.cpu().numpy()[:, cols // 2:] == 0xAB)
    assert np.all(sbuf.cpu().numpy()[:, cols // blk:] == 0xCD)
    assert np.all(bf16_bits(obuf[:, cols:]) == 0x3F80)
