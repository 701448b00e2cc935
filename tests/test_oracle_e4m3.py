"""Pins of the oracle's fp32 -> E4M3 conversion and scaled E4M3 quantizer (CPU)."""
import numpy as np
import pytest
import torch

from oracle import e4m3 as Q
from oracle.formats import E4M3_POS_VALUES, e4m3_decode
from synthetic import all_bf16_patterns, bf16_bits_to_f32
from tests.conftest import golden_rows


def _double_rounding(x):
    """Negative control: fp32 -RTZ-> fp16 -RNE-> E4M3 (the sm_89 lowering)."""
    x = np.asarray(x, np.float32)
    h = np.float16(x)                                   # RNE to fp16
    # replace by the round-toward-zero fp16 value
    hv = h.astype(np.float32)
    over = np.abs(hv) > np.abs(x)
    h = np.where(over, np.nextafter(h, np.float16(0)), h)
    return Q.e4m3_from_f32(h.astype(np.float32))


def test_page_cases():
    for row in golden_rows("e4m3_cases.txt"):
        key, want = row[0], float(row[1])
        if key.startswith("double_rounding:"):
            x = np.float32(float(key.split(":")[1]))
            got = e4m3_decode(_double_rounding([x]))[0]
            assert got == want, "negative control must reproduce the double-rounding bug"
            assert e4m3_decode(Q.e4m3_from_f32([x]))[0] != want
        else:
            x = np.float32(float(key))
            assert e4m3_decode(Q.e4m3_from_f32([x]))[0] == want
            assert e4m3_decode(Q.e4m3_from_f32([-x]))[0] == -want


def test_200_04_code():
    assert Q.e4m3_from_f32([np.float32(200.04)])[0] == 0x75
    assert Q.e4m3_from_f32([np.float32(192.0)])[0] == 0x74


def test_saturation_nan_signed_zero():
    x = np.array([448, 449, 463.99, 464, 465, 480, 1e30, np.inf, -np.inf, np.nan, -np.nan, 0.0, -0.0, -1e-9],
                 np.float32)
    got = Q.e4m3_from_f32(x)
    assert list(got[:9]) == [0x7E] * 7 + [0x7E, 0xFE]
    assert got[9] & 0x7F == 0x7F and got[10] & 0x7F == 0x7F
    assert got[11] == 0x00 and got[12] == 0x80 and got[13] == 0x80


def test_all_bf16_patterns_two_derivations():
    x = bf16_bits_to_f32(all_bf16_patterns())
    a = Q.e4m3_from_f32(x)
    b = Q.e4m3_from_f32_bruteforce(x)
    assert np.array_equal(a, b)


def test_all_bf16_patterns_vs_torch():
    x = bf16_bits_to_f32(all_bf16_patterns())
    ok = np.isfinite(x) & (np.abs(x) <= 464)        # torch's cast is not satfinite above 464
    mine = Q.e4m3_from_f32(x[ok])
    lib = torch.from_numpy(x[ok].copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, lib)


def _fp32_sweep():
    """Grid values, midpoints, one and two fp32 ulps either side, uniform samples
    over the range and over the subnormals, both signs."""
    v = E4M3_POS_VALUES
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    pts = [v.astype(np.float32), mid]
    for d in (1, 2):
        up, dn = mid.copy(), mid.copy()
        for _ in range(d):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(0))
        pts += [up, dn]
    g = np.random.default_rng(11)
    pts += [g.uniform(0, 470, 400000).astype(np.float32), g.uniform(0, 2.0 ** -6, 100000).astype(np.float32)]
    p = np.concatenate(pts)
    return np.concatenate([p, -p])


def test_fp32_sweep_two_derivations_and_torch():
    x = _fp32_sweep()
    a = Q.e4m3_from_f32(x)
    assert np.array_equal(a, Q.e4m3_from_f32_bruteforce(x))
    ok = np.abs(x) <= 464
    lib = torch.from_numpy(x[ok].copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(a[ok], lib)


def test_scale_example_22_4():
    rows = golden_rows("fp8_scale_example.txt")
    amax, scale, mult, top = (float(v) for v in rows[0])
    x = np.array([[amax, 1.0, -3.0, 0.0]], np.float32)
    codes, s = Q.quantize_e4m3(x, -1)
    assert abs(float(s[0, 0]) - scale) < 1e-8
    assert abs(1.0 / float(s[0, 0]) - mult) < 1e-5
    assert e4m3_decode(codes)[0, 0] == top


def test_block_max_lands_on_448_and_error_bound():
    g = np.random.default_rng(5)
    x = (g.standard_normal((64, 512)) * np.exp2(g.integers(-20, 20, (64, 1)))).astype(np.float32)
    codes, s = Q.quantize_e4m3(x, 128)
    c = codes.reshape(64, 4, 128)
    top = np.take_along_axis(c & 0x7F, np.abs(x.reshape(64, 4, 128)).argmax(axis=2)[..., None], 2)
    assert np.all(top == 0x7E)
    # element error <= half an E4M3 spacing (in scaled units), times the scale
    v = e4m3_decode(codes).reshape(64, 4, 128) * s[:, :, None].astype(np.float64)
    err = np.abs(v - x.reshape(64, 4, 128).astype(np.float64)) / s[:, :, None]
    q = np.abs(x.reshape(64, 4, 128) / s[:, :, None]).astype(np.float64)
    _, ex = np.frexp(np.maximum(q, 2.0 ** -6))
    spacing = np.exp2(ex - 1 - 3.0)
    assert np.all(err <= spacing / 2 * (1 + 1e-6) + 1e-7 * q)


def test_zero_block_scale_one_and_nonfinite_rejected():
    x = np.zeros((2, 256), np.float32)
    codes, s = Q.quantize_e4m3(x, 128)
    assert np.all(s == 1.0) and np.all(codes == 0)
    x[1, 3] = np.inf
    with pytest.raises(ValueError):
        Q.quantize_e4m3(x, 128)


def test_per_row_equals_block_of_full_width():
    g = np.random.default_rng(9)
    x = g.standard_normal((8, 384)).astype(np.float32)
    a, sa = Q.quantize_e4m3(x, -1)
    b, sb = Q.quantize_e4m3(x, 384)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_scaled_quotient_is_correctly_rounded_fp32():
    # fp64 holds x and s exactly; rounding the fp64 quotient to fp32 gives the
    # correctly rounded fp32 quotient (53 >= 2*24 + 2), an independent route to
    # RN_f32(x / s) and RN_f32(amax / 448)
    g = np.random.default_rng(1)
    x = (g.standard_normal((32, 1024)) * np.exp2(g.integers(-30, 30, (32, 1)))).astype(np.float32)
    codes, s = Q.quantize_e4m3(x, 128)
    amax = np.abs(x.reshape(32, 8, 128)).max(axis=2).astype(np.float64)
    s64 = (amax / 448.0).astype(np.float32)
    assert np.array_equal(s, s64)
    q = (x.reshape(32, 8, 128).astype(np.float64) / s64[:, :, None].astype(np.float64)).astype(np.float32)
    assert np.array_equal(codes, Q.e4m3_from_f32_bruteforce(q).reshape(32, 1024))
