"""Pins of the oracle's E8M0 rule, E2M1 rounding and MXFP4 quantizer (CPU)."""
import numpy as np
import pytest

from oracle import e8m0 as R
from oracle import mxfp4 as MX
from oracle.dequant import dequant_mxfp4
from oracle.formats import E2M1_GRID, bf16_decode, e2m1_decode, f32_bits, f32_from_bits
from synthetic import all_bf16_patterns, bf16_bits_to_f32, mxfp4_gemv_inputs
from tests.conftest import golden_rows


def _old_rule(vecmax):
    """Negative control: biased exponent of vecMax * (1/6) in fp32."""
    v = np.asarray(vecmax, np.float32) * np.float32(1.0 / 6.0)
    return ((f32_bits(v) >> 23) & 0xFF).astype(np.uint8)


def _rule_with_constant(vecmax, add):
    bits = f32_bits(np.abs(np.asarray(vecmax, np.float32))).astype(np.uint64)
    be = (((bits + add) & 0xFF800000) >> 23) & 0xFF
    return np.where(be > 2, be - 2, 0).astype(np.int64)


def test_worked_table():
    for vm, old, fixed, r_old, r_fixed in golden_rows("e8m0_worked_table.txt"):
        v = np.array([float(vm)], np.float32)
        assert R.e8m0_code_bits(v)[0] == int(fixed)
        assert R.e8m0_code_arith(v)[0] == int(fixed)
        assert _old_rule(v)[0] == int(old)
        assert abs(float(v[0]) / R.e8m0_scale(int(fixed)) - float(r_fixed)) < 1e-5
        assert abs(float(v[0]) / R.e8m0_scale(int(old)) - float(r_old)) < 1e-5


def test_two_derivations_all_bf16_patterns():
    x = bf16_bits_to_f32(all_bf16_patterns())
    x = x[np.isfinite(x)]
    assert np.array_equal(R.e8m0_code_bits(x), R.e8m0_code_arith(x))


def test_two_derivations_fp32_sweep():
    g = np.random.default_rng(4)
    bits = g.integers(0, 0x7F800000, 2_000_000, dtype=np.uint32)
    # dense around the 0.75 threshold of every binade
    e = g.integers(1, 255, 200000).astype(np.uint32)
    edge = (e << 23) | (0x600000 + g.integers(-3, 3, 200000)).astype(np.uint32)
    x = f32_from_bits(np.concatenate([bits, edge, np.array([0, 1, 0x7F7FFFFF, 0x00600000], np.uint32)]))
    assert np.array_equal(R.e8m0_code_bits(x), R.e8m0_code_arith(x))


def test_ratio_invariant_and_clip_share():
    # every mantissa of one binade (2^23 patterns), exponent field 130
    m = np.arange(1 << 23, dtype=np.uint32)
    x = f32_from_bits((np.uint32(130) << 23) | m)
    f = m.astype(np.float64) / 2.0 ** 23
    zones = golden_rows("e8m0_clip_zones.txt")
    for add, lo, hi, rlo, rhi, share in zones:
        code = _rule_with_constant(x, int(add))
        ratio = x.astype(np.float64) / np.exp2(code - 127.0)
        clip = ratio >= 6.0
        assert abs(clip.mean() - float(share)) < 1e-12
        if lo != "-":
            assert np.array_equal(clip, (f >= float(lo)) & (f < float(hi)))
            assert ratio[clip].min() >= float(rlo) and ratio[clip].max() < float(rhi)
    # the oracle uses the 0.75 constant: its codes equal the 1<<21 variant
    assert np.array_equal(R.e8m0_code_bits(x).astype(np.int64), _rule_with_constant(x, 1 << 21))
    ratio = x.astype(np.float64) / R.e8m0_scale(R.e8m0_code_bits(x))
    assert ratio.min() >= 3.5 and ratio.max() < 7.0


def test_zero_and_tiny_blocks():
    assert R.e8m0_code_bits(np.array([0.0], np.float32))[0] == 0
    assert R.e8m0_code_arith(np.array([0.0], np.float32))[0] == 0
    tiny = f32_from_bits(np.array([1, 0x00700000, 0x00800000, 0x01000000, 0x01600000], np.uint32))
    assert np.array_equal(R.e8m0_code_bits(tiny), R.e8m0_code_arith(tiny))
    with pytest.raises(ValueError):
        R.e8m0_code_bits(np.array([np.inf], np.float32))


def test_e2m1_grid_ties_and_saturation():
    rows = {r[0]: r[1:] for r in golden_rows("e2m1_grid.txt")}
    grid = np.array([float(v) for v in rows["values"]])
    bounds = np.array([float(v) for v in rows["bounds"]])
    c = MX.e2m1_from_f64(grid, np.zeros(8, np.uint8))
    assert list(c) == list(range(8))
    tie = MX.e2m1_from_f64(bounds, np.zeros(7, np.uint8))
    assert list(e2m1_decode(tie)) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    sat = MX.e2m1_from_f64(np.array([6.0, 6.5, 7.0, 100.0, 1e300]), np.zeros(5, np.uint8))
    assert list(sat) == [7] * 5
    neg = MX.e2m1_from_f64(np.array([-0.1, -0.0, -3.2]), np.array([1, 1, 1], np.uint8))
    assert list(neg) == [0x8, 0x8, 0x8 | 5]


def test_e2m1_two_derivations_all_bf16_patterns():
    x = bf16_bits_to_f32(all_bf16_patterns())
    x = x[np.isfinite(x)].astype(np.float64)
    s = np.signbit(x).astype(np.uint8)
    for code in (127, 120, 130, 1):
        v = x * 2.0 ** (127 - code)
        assert np.array_equal(MX.e2m1_from_f64(v, s), MX.e2m1_from_f64_bruteforce(v, s))


def test_pack_unpack_identity():
    g = np.random.default_rng(2)
    c = g.integers(0, 16, (5, 64), dtype=np.uint8)
    assert np.array_equal(MX.unpack_nibbles(MX.pack_nibbles(c)), c)


def test_block_max_gets_top_codes_and_reconstruction():
    x, W = mxfp4_gemv_inputs(0)
    for block in (32, 16):
        packed, sc = MX.quantize_mxfp4(W, block)
        codes = MX.unpack_nibbles(packed).reshape(W.shape[0], -1, block)
        amax_pos = np.abs(W.reshape(W.shape[0], -1, block)).argmax(axis=2)
        top = np.take_along_axis(codes & 7, amax_pos[..., None], 2)[..., 0]
        assert set(np.unique(top)) <= {6, 7}
        # reconstruction error of non-saturated elements <= half the E2M1 spacing
        deq = bf16_decode(dequant_mxfp4(packed, sc, block)).reshape(W.shape[0], -1, block)
        s = np.exp2(sc.astype(np.float64) - 127.0)[..., None]
        v = W.reshape(deq.shape).astype(np.float64) / s
        a = np.abs(v)
        spacing = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
        ok = a <= 6
        assert np.all(np.abs(deq / s - v)[ok] <= spacing[ok] / 2 + 1e-12)


def test_quantize_matches_elementwise_definition():
    g = np.random.default_rng(8)
    x = (g.standard_normal((16, 256)) * np.exp2(g.integers(-40, 40, (16, 1)))).astype(np.float32)
    packed, sc = MX.quantize_mxfp4(x, 32)
    vmax = np.abs(x.reshape(16, 8, 32)).max(axis=2)
    assert np.array_equal(sc, R.e8m0_code_arith(vmax))
    v = x.reshape(16, 8, 32).astype(np.float64) / np.exp2(sc.astype(np.float64) - 127.0)[..., None]
    want = MX.e2m1_from_f64_bruteforce(v, np.signbit(x).reshape(v.shape).astype(np.uint8)).reshape(16, 256)
    assert np.array_equal(MX.unpack_nibbles(packed), want)


def test_rejects_bad_block_and_nonfinite():
    with pytest.raises(ValueError):
        MX.quantize_mxfp4(np.zeros((2, 48), np.float32), 32)
    x = np.zeros((2, 64), np.float32)
    x[0, 0] = np.nan
    with pytest.raises(ValueError):
        MX.quantize_mxfp4(x, 32)
