"""Pins of the NVFP4 oracle (E2M1 blocks of 16 with an E4M3 scale) on the CPU."""
import numpy as np
import pytest

from oracle import mx as MX
from oracle import mxfp4 as M4
from oracle import nvfp4 as NV
from oracle.e4m3 import e4m3_from_f32_bruteforce
from oracle.formats import E2M1_GRID, E4M3_POS_CODES, E4M3_POS_VALUES, bf16_decode, e2m1_decode, e4m3_decode


def _blocks(seed, rows=40, cols=256, lo=-8, hi=8):
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(g.integers(lo, hi, (rows, cols // 16, 1))).repeat(16, axis=2).reshape(rows, cols).astype(np.float32)
    return x


def test_every_e4m3_value_round_trips_as_a_scale():
    # a block whose maximum is 6 v has scale v exactly, for every E4M3 value v
    v = E4M3_POS_VALUES[1:]
    amax = (6.0 * v).astype(np.float32)
    s8, d = NV.block_scale(amax)
    assert np.array_equal(s8, E4M3_POS_CODES[1:].astype(np.uint8))
    assert np.array_equal(d.astype(np.float64), v)


def test_scale_is_the_nearest_e4m3_value_of_amax_over_6g():
    g = np.random.default_rng(1)
    amax = np.exp2(g.uniform(-14, 12, 20000)).astype(np.float32)
    for gs in (1.0, 0.37, 2.0 ** -7, 3.1e-4):
        s8, d = NV.block_scale(amax, gs)
        target = (amax.astype(np.float64) / 6.0 / gs)
        # brute force over the whole E4M3 table, on the fp32 quotient
        want = e4m3_from_f32_bruteforce(((amax / np.float32(6)).astype(np.float32) / np.float32(gs)).astype(np.float32))
        assert np.array_equal(s8, want)
        # and within half an E4M3 step of the real quotient (normal range, below 448)
        val = e4m3_decode(s8)
        ok = (target >= 2.0 ** -6) & (target < 448)
        assert np.all(np.abs(val[ok] - target[ok]) <= target[ok] * 2.0 ** -4 * (1 + 1e-6))
        assert np.array_equal(d, (val * np.float32(gs)).astype(np.float32))


def test_elements_divide_by_the_dequantized_scale():
    x = _blocks(2, lo=-16, hi=8)
    for gs in (1.0, 0.01):
        packed, s8 = NV.quantize_nvfp4(x, gs)
        d = (e4m3_decode(s8).astype(np.float32) * np.float32(gs)).astype(np.float32)[:, :, None]
        assert (d > 0).any() and (gs != 1.0 or (d == 0).any())   # some scales underflow E4M3
        with np.errstate(divide="ignore", invalid="ignore"):
            v = np.where(d > 0, x.reshape(x.shape[0], -1, 16) / d, 0.0).astype(np.float32).reshape(x.shape)
        ref = M4.e2m1_from_f64_bruteforce(v.astype(np.float64), np.signbit(x).astype(np.uint8))
        assert np.array_equal(M4.unpack_nibbles(packed), ref)
        # negative control: dividing by the unrounded scale gives other codes
        s = ((np.abs(x.reshape(x.shape[0], -1, 16)).max(axis=2) / np.float32(6)).astype(np.float32))
        with np.errstate(divide="ignore", invalid="ignore"):
            v_bad = np.where(d > 0, x.reshape(x.shape[0], -1, 16) / (s * np.float32(gs))[:, :, None],
                             0.0).astype(np.float32).reshape(x.shape)
        bad = M4.e2m1_from_f64_bruteforce(v_bad.astype(np.float64), np.signbit(x).astype(np.uint8))
        assert not np.array_equal(bad, ref)


def test_power_of_two_scales_match_the_mx_ceil_rule():
    # amax = 6 * 2^k: the E4M3 scale is the power 2^k, which is the round-up
    # division rule's E8M0 scale; the element codes must then coincide
    g = np.random.default_rng(3)
    x = g.uniform(-1, 1, (64, 16 * 8)).astype(np.float32)
    k = g.integers(-6, 7, (64, 8))
    xb = x.reshape(64, 8, 16)
    pos = g.integers(0, 16, (64, 8))
    np.put_along_axis(xb, pos[..., None], 1.0, axis=2)
    xb *= (6.0 * np.exp2(k))[..., None].astype(np.float32)
    x = xb.reshape(64, -1)
    p_nv, s8 = NV.quantize_nvfp4(x)
    p_mx, c_mx = MX.quantize_mx(x, 16, "e2m1", "ceil_div")
    assert np.array_equal(e4m3_decode(s8), np.exp2(c_mx.astype(np.float64) - 127))
    assert np.array_equal(p_nv, p_mx)


def test_scale_lands_between_powers_of_two():
    # the block maximum maps to within an E4M3 step of 6, where every E8M0
    # rule leaves a factor-2 range
    x = _blocks(4, lo=0, hi=8)                           # block scales in the E4M3 normal range
    packed, s8 = NV.quantize_nvfp4(x)
    assert np.all((s8 >> 3) > 0) and np.all(s8 < 0x7E)
    amax = np.abs(x.reshape(x.shape[0], -1, 16)).max(axis=2).astype(np.float64)
    r = amax / e4m3_decode(s8)
    assert r.min() >= 6 / (1 + 2.0 ** -4) and r.max() <= 6 / (1 - 2.0 ** -4)
    mant = s8 & 7
    assert np.mean(mant != 0) > 0.5
    # with r in that range the block maximum always takes the top code (6)
    codes = M4.unpack_nibbles(packed).reshape(x.shape[0], -1, 16) & 7
    top = np.take_along_axis(codes, np.abs(x.reshape(codes.shape)).argmax(axis=2)[..., None], 2)[..., 0]
    assert set(np.unique(top)) == {7}


def test_power_of_two_tensor_scale_invariance():
    x = _blocks(5)
    base = NV.quantize_nvfp4(x, 0.125)
    for j in (-5, 3, 9):
        p, s = NV.quantize_nvfp4((x * np.float32(2.0 ** j)).astype(np.float32), 0.125 * 2.0 ** j)
        assert np.array_equal(p, base[0]) and np.array_equal(s, base[1])


def test_operand_products_are_bf16_numbers():
    e = np.concatenate([E2M1_GRID, -E2M1_GRID])
    p = (e[:, None] * E4M3_POS_VALUES[None, :]).reshape(-1)
    from oracle.formats import bf16_round
    assert np.array_equal(bf16_decode(bf16_round(p)), p)
    # the dequantized operand equals the product of the decoded parts
    x = _blocks(6, rows=8)
    packed, s8 = NV.quantize_nvfp4(x)
    want = e2m1_decode(M4.unpack_nibbles(packed)).reshape(8, -1, 16) * e4m3_decode(s8)[..., None]
    assert np.array_equal(bf16_decode(NV.dequant_nvfp4(packed, s8)), want.reshape(8, -1))


def test_reconstruction_error_bound():
    x = _blocks(7)
    for gs in (1.0, 2.0 ** -3):
        packed, s8 = NV.quantize_nvfp4(x, gs)
        d = e4m3_decode(s8)[..., None] * gs
        rec = (e2m1_decode(M4.unpack_nibbles(packed)).reshape(x.shape[0], -1, 16) * d).reshape(x.shape)
        dd = np.repeat(d[..., 0], 16, axis=1)
        assert np.all(rec[dd == 0] == 0)
        with np.errstate(divide="ignore", invalid="ignore"):
            v = np.where(dd > 0, np.abs(x) / np.where(dd > 0, dd, 1.0), 0.0)
        # half the E2M1 spacing: 0.25 below 2, 0.5 in [2, 4), 1 in [4, 6]
        half = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0)) * dd
        ok = (v <= 6) & (dd > 0)
        sat = (v > 6) & (dd > 0)
        assert np.all(np.abs(rec - x)[ok] <= half[ok] * (1 + 1e-6))
        assert np.all(np.abs(rec[sat]) == 6 * dd[sat])


def test_zero_tiny_and_saturated_blocks():
    x = np.zeros((2, 64), np.float32)
    x[0, 16:32] = -0.0
    x[0, 32:48] = np.float32(1e-4) * np.arange(16, dtype=np.float32)   # amax/6 below 2^-10: scale 0
    x[1, :16] = 1e5                                                     # amax/6 above 448: saturates
    x[1, 16:32] = -2.0 ** -126
    packed, s8 = NV.quantize_nvfp4(x)
    c = M4.unpack_nibbles(packed)
    assert s8[0, 0] == 0 and np.all(c[0, :16] == 0)
    assert np.all(c[0, 16:32] == 8)                      # zeros keep their sign
    assert s8[0, 2] == 0 and np.all(c[0, 32:48] == 0)
    assert s8[1, 0] == 0x7E and np.all(c[1, :16] == 7)
    assert s8[1, 1] == 0 and np.all(c[1, 16:32] == 8)
    with pytest.raises(ValueError):
        NV.quantize_nvfp4(x, 0.0)
    with pytest.raises(ValueError):
        NV.quantize_nvfp4(x, float("inf"))
    with pytest.raises(ValueError):
        NV.block_scale(np.array([np.nan], np.float32))
