"""The seeded generators are deterministic and follow their stated recipes."""
import numpy as np

from block_scaled_fp4_absmax_amd import inputs


def test_deterministic():
    a = inputs.gen_c1()
    b = inputs.gen_c1()
    assert a.dtype == np.uint16 and a.shape == (256, 4096)
    assert np.array_equal(a, b)
    assert not np.array_equal(inputs.gen_c2(rows=64, cols=64), inputs.gen_c2(rows=64, cols=64, seed=9))


def test_bf16_rounding_is_rne():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, -0.0], np.float64)
    got = inputs.f64_to_bf16_bits(v)
    assert list(got) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0000, 0x8000]


def test_c1_outliers_count():
    x = inputs.bf16_bits_to_f32(inputs.gen_c1())
    # 1049 = round(0.1% of 1,048,576) positions x20 on top of 0.02 N(0,1)
    assert 0.019 < np.std(x[np.abs(x) < 0.2]) < 0.021
    big = np.abs(x) > 0.15
    assert 500 < big.sum() < 1049


def test_c3_outlier_channels_recovered():
    rows = 64
    x = inputs.bf16_bits_to_f32(inputs.gen_c3(rows=rows, cols=1024))
    ch = inputs.c3_outlier_channels(rows=rows, cols=1024)
    assert ch.size == 16
    m = np.abs(x).mean(0)
    assert set(np.argsort(-m)[:16]) == set(ch)


def test_c4_block_variance_structure():
    x = inputs.bf16_bits_to_f32(inputs.gen_c4(rows=256, cols=1024)).astype(np.float64)
    v = (x * x).mean(0).reshape(-1, 32)
    within = v.std(1) / v.mean(1)
    across = v.mean(1)
    assert np.all(within < 0.5) and across.max() / across.min() > 10


def test_c5_shapes():
    assert [s[1:] for s in inputs.C5_SHAPES] == [
        (8192, 8192), (1024, 8192), (1024, 8192), (8192, 8192),
        (28672, 8192), (28672, 8192), (8192, 28672)]
    x = inputs.gen_c5(1, rows=8)
    assert x.shape == (8, 8192)
