"""Pins of the W8A8 FP8 oracle: static per-tensor quantization, 128 x 128
weight blocks and the block-scaled fp32 reference (CPU)."""
import numpy as np
import pytest

from oracle import e4m3 as E4
from oracle import w8a8 as W8
from oracle.formats import e4m3_decode
from tests.conftest import golden_rows


def test_static_quantization_worked_example():
    # the walkthrough's row: amax 22.4 with scale 0.05 lands on 448
    (amax, scale, mult, top), = golden_rows("fp8_scale_example.txt")
    x = np.array([float(amax), -float(amax), float(amax) / 2], np.float32)
    c = W8.quantize_e4m3_static(x, float(scale))
    assert e4m3_decode(c)[0] == float(top) and e4m3_decode(c)[1] == -float(top)
    assert e4m3_decode(c)[2] == 224.0
    # unscaled, 0.0005 falls below half the smallest subnormal and 0.001 becomes 2^-9
    c = W8.quantize_e4m3_static(np.array([0.0005, 0.001], np.float32), 1.0)
    assert list(e4m3_decode(c)) == [0.0, 2.0 ** -9]
    # saturation instead of overflow
    c = W8.quantize_e4m3_static(np.array([1e6, -1e30], np.float32), 0.5)
    assert list(c) == [0x7E, 0xFE]


def test_static_equals_dynamic_per_tensor_with_its_scale():
    g = np.random.default_rng(1)
    x = (g.standard_normal((16, 256)) * 3).astype(np.float32)
    s = E4.e4m3_scale(np.abs(x).max())
    c_dyn, s_dyn = E4.quantize_e4m3(x.reshape(1, -1), -1)
    assert s_dyn[0, 0] == s
    assert np.array_equal(W8.quantize_e4m3_static(x, float(s)).reshape(1, -1), c_dyn)
    with pytest.raises(ValueError):
        W8.quantize_e4m3_static(x, 0.0)


def test_weight_blocks():
    g = np.random.default_rng(2)
    N, K = 300, 512
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    # one block holds a planted maximum 448 * 2^-5: its scale is exactly 2^-5
    w[130, 260] = 448 * 2.0 ** -5
    codes, s = W8.quantize_e4m3_block2d(w)
    assert s.shape == (3, 4)
    assert s[1, 2] == 2.0 ** -5 and codes[130, 260] == 0x7E
    for i in range(3):
        for j in range(4):
            blk = w[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            assert s[i, j] == np.float32(np.abs(blk).max() / np.float32(448))
    deq = e4m3_decode(codes) * np.repeat(np.repeat(s, 128, axis=0)[:N], 128, axis=1)
    ref = w.astype(np.float64)
    normal = np.abs(ref) >= 2.0 ** -6 * np.repeat(np.repeat(s, 128, axis=0)[:N], 128, axis=1)
    assert np.all(np.abs(deq - ref)[normal] <= np.abs(ref)[normal] * 2.0 ** -4)


def test_block_scaled_reference_is_the_dequantized_matmul():
    g = np.random.default_rng(3)
    M, N, K = 37, 260, 384
    x = (g.standard_normal((M, K)) * np.exp2(g.integers(-4, 4, (M, 1)))).astype(np.float32)
    w = (g.standard_normal((N, K)) * 0.05).astype(np.float32)
    a, sa = E4.quantize_e4m3(x, 128)                           # per token x 128-K group
    b, sb = W8.quantize_e4m3_block2d(w)                        # 128 x 128 blocks
    y, asum = W8.reference(a, W8.expand_scales(sa, M, K // 128), b, W8.expand_scales(sb, N, K // 128, 128))
    xd = e4m3_decode(a) * np.repeat(sa.astype(np.float64), 128, axis=1)
    wd = e4m3_decode(b) * np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0)[:N], 128, axis=1)
    assert np.allclose(y, xd @ wd.T, rtol=1e-12, atol=1e-12 * (np.abs(xd) @ np.abs(wd).T).max())
    assert np.allclose(asum, np.abs(xd) @ np.abs(wd).T, rtol=1e-12)
    # a transposed weight-scale matrix is caught
    bad, _ = W8.reference(a, W8.expand_scales(sa, M, K // 128), b,
                          W8.expand_scales(sb[::-1].copy(), N, K // 128, 128))
    assert not np.allclose(bad, y)


def test_scales_that_factor_out():
    g = np.random.default_rng(4)
    M, N, K = 5, 40, 256
    a = g.integers(0, 0x7E, (M, K)).astype(np.uint8)
    b = g.integers(0, 0x7E, (N, K)).astype(np.uint8) | (g.integers(0, 2, (N, K)) << 7).astype(np.uint8)
    base = e4m3_decode(a) @ e4m3_decode(b).T
    y, _ = W8.reference(a, W8.expand_scales(0.25, M, 2), b, W8.expand_scales(3.0, N, 2))
    assert np.allclose(y, 0.75 * base, rtol=1e-13)
    sm = g.uniform(0.5, 2, M)
    sn = g.uniform(0.5, 2, N)
    y, _ = W8.reference(a, W8.expand_scales(sm, M, 2), b, W8.expand_scales(sn, N, 2))
    assert np.allclose(y, sm[:, None] * base * sn[None, :], rtol=1e-13)
