"""Pins of the MX scale-rule variants and the MXFP8 (E4M3 element) quantizer (CPU)."""
import numpy as np
import pytest

from oracle import e4m3 as E4
from oracle import mx as MX
from oracle import mxfp4 as M4
from oracle.formats import e4m3_decode, f32_bits, f32_from_bits
from synthetic import all_bf16_patterns, bf16_bits_to_f32
from tests.conftest import golden_rows


def _binade(exp_field=130):
    m = np.arange(1 << 23, dtype=np.uint32)
    return f32_from_bits((np.uint32(exp_field) << 23) | m), m.astype(np.float64) / 2.0 ** 23


def _ratio(x, code):
    return x.astype(np.float64) / np.exp2(code.astype(np.float64) - 127.0)


def test_worked_table_old_and_fixed_rules():
    # the old rule is floor_div with E2M1 elements, the fixed one is round
    for vm, old, fixed, r_old, r_fixed in golden_rows("e8m0_worked_table.txt"):
        v = np.array([float(vm)], np.float32)
        for fn in (MX.scale_code, MX.scale_code_arith):
            assert fn(v, "floor_div", "e2m1")[0] == int(old)
            assert fn(v, "round", "e2m1")[0] == int(fixed)
        assert abs(_ratio(v, MX.scale_code(v, "floor_div", "e2m1"))[0] - float(r_old)) < 1e-5
        assert abs(_ratio(v, MX.scale_code(v, "round", "e2m1"))[0] - float(r_fixed)) < 1e-5


def test_clip_zones_of_the_three_constants():
    x, f = _binade()
    zones = golden_rows("e8m0_clip_zones.txt")
    for (add, lo, hi, rlo, rhi, share), rule in zip(zones, ("ocp", "round", "half")):
        code = MX.scale_code(x, rule, "e2m1")
        ratio = _ratio(x, code)
        clip = ratio >= 6.0
        assert abs(clip.mean() - float(share)) < 1e-12
        if lo != "-":
            assert np.array_equal(clip, (f >= float(lo)) & (f < float(hi)))
            assert ratio[clip].min() >= float(rlo) and ratio[clip].max() < float(rhi)


@pytest.mark.parametrize("elem,rule,lo,hi", [
    ("e2m1", "round", 3.5, 7.0),
    ("e2m1", "half", 3.0, 6.0),
    ("e2m1", "ocp", 4.0, 8.0),
    ("e4m3", "round", 248.0, 496.0),
    ("e4m3", "half", 192.0, 384.0),
    ("e4m3", "ocp", 256.0, 512.0),
])
def test_ratio_range_exponent_rules(elem, rule, lo, hi):
    # vmax / scale over every mantissa of two binades: the range each rule maps
    # the block maximum to, with both ends reached
    for e in (130, 20):
        x, _ = _binade(e)
        r = _ratio(x, MX.scale_code(x, rule, elem))
        assert r.min() == lo and r.max() < hi
        assert r.max() > hi * (1 - 2.0 ** -22)


def test_e4m3_round_rule_clip_share():
    # with m = 3 the carry happens for fractions >= 1 - 2^-4; the maximum then
    # exceeds 448 (1.75 * 2^8) for fractions in [0.75, 0.9375)
    x, f = _binade()
    r = _ratio(x, MX.scale_code(x, "round", "e4m3"))
    clip = r > 448.0
    assert np.array_equal(clip, (f > 0.75) & (f < 0.9375))
    assert abs(clip.mean() - 0.1875) < 1e-6


@pytest.mark.parametrize("elem,emax", [("e2m1", 6.0), ("e4m3", 448.0)])
def test_division_rules_bracket_the_quotient(elem, emax):
    g = np.random.default_rng(11)
    bits = np.concatenate([g.integers(0, 0x7F800000, 400000, dtype=np.uint32),
                           f32_bits(np.float32(emax) * np.exp2(np.arange(-140, 120)).astype(np.float32)),
                           np.array([0, 1, 2, 0x00400000, 0x00400001, 0x7F7FFFFF], np.uint32)])
    x = f32_from_bits(bits)
    qf = (x * (np.float32(1) / np.float32(emax))).astype(np.float32).astype(np.float64)
    qc = (x / np.float32(emax)).astype(np.float32).astype(np.float64)
    cf = MX.scale_code(x, "floor_div", elem).astype(np.float64)
    cc = MX.scale_code(x, "ceil_div", elem).astype(np.float64)
    # floor: 2^(c-127) <= q < 2^(c-126) for normal q; code 0 otherwise
    norm = qf >= 2.0 ** -126
    assert np.all(np.exp2(cf[norm] - 127) <= qf[norm]) and np.all(qf[norm] < np.exp2(cf[norm] - 126))
    assert np.all(cf[~norm] == 0)
    # ceil: the smallest power 2^k >= q with k >= -127
    assert np.all(np.exp2(cc - 127) >= qc)
    above = cc > 0
    assert np.all(np.exp2(cc[above] - 128) < qc[above])
    assert np.all(qc[~above] <= 2.0 ** -127)


def test_ceil_rule_never_clips_and_exact_powers():
    # rounding the quotient up keeps vmax / scale <= the element maximum
    x, _ = _binade()
    for elem, emax in (("e2m1", 6.0), ("e4m3", 448.0)):
        r = _ratio(x, MX.scale_code(x, "ceil_div", elem))
        assert r.max() <= emax * (1 + 2.0 ** -23) and r.min() > emax / 2 * (1 - 2.0 ** -23)
        for k in (-3, 0, 7):
            v = np.array([emax * 2.0 ** k], np.float32)
            assert MX.scale_code(v, "ceil_div", elem)[0] == 127 + k
            # a quotient a few ulps above the power (one ulp of vmax can round away)
            up = (v * np.float32(1 + 2.0 ** -20)).astype(np.float32)
            assert MX.scale_code(up, "ceil_div", elem)[0] == 128 + k


@pytest.mark.parametrize("rule", MX.RULES)
@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_two_derivations_all_bf16_patterns(rule, elem):
    x = bf16_bits_to_f32(all_bf16_patterns())
    x = x[np.isfinite(x)]
    assert np.array_equal(MX.scale_code(x, rule, elem), MX.scale_code_arith(x, rule, elem))


@pytest.mark.parametrize("rule", MX.RULES)
def test_two_derivations_fp32_edges(rule):
    g = np.random.default_rng(5)
    e = g.integers(0, 255, 300000).astype(np.uint32)
    frac = np.array([0, 0x400000, 0x600000, 0x700000, 0x780000], np.uint32)
    m = (frac[g.integers(0, 5, 300000)].astype(np.int64) + g.integers(-2, 3, 300000)) & 0x7FFFFF
    x = f32_from_bits((e << 23) | m.astype(np.uint32))
    for elem in ("e2m1", "e4m3"):
        assert np.array_equal(MX.scale_code(x, rule, elem), MX.scale_code_arith(x, rule, elem))


def test_zero_tiny_and_nonfinite():
    tiny = f32_from_bits(np.array([0, 1, 0x00400000, 0x00700000, 0x00800000, 0x01000000], np.uint32))
    for rule in MX.RULES:
        for elem in ("e2m1", "e4m3"):
            c = MX.scale_code(tiny, rule, elem)
            assert c[0] == 0
            assert np.array_equal(c, MX.scale_code_arith(tiny, rule, elem))
            with pytest.raises(ValueError):
                MX.scale_code(np.array([np.nan], np.float32), rule, elem)


def _rows(seed, rows=24, cols=256):
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, cols)).astype(np.float32) * np.exp2(g.integers(-20, 20, (rows, 1))).astype(np.float32)
    x[0, :32] = 0.0
    x[1, 5] = 6.0 * 2.0 ** 3
    x[2, :] = -x[2, :]
    return x


def test_round_rule_e2m1_is_quantize_mxfp4():
    # the fixed rule with E2M1 elements is the MXFP4 quantizer pinned on its own
    x = _rows(1)
    for block in (16, 32):
        p, c = MX.quantize_mx(x, block, "e2m1", "round")
        p0, c0 = M4.quantize_mxfp4(x, block)
        assert np.array_equal(p, p0) and np.array_equal(c, c0)


@pytest.mark.parametrize("rule", MX.RULES)
def test_e2m1_elements_any_rule_bruteforce(rule):
    x = _rows(2)
    p, c = MX.quantize_mx(x, 32, "e2m1", rule)
    v = x.astype(np.float64).reshape(x.shape[0], -1, 32) / np.exp2(c.astype(np.float64) - 127)[..., None]
    ref = M4.e2m1_from_f64_bruteforce(v.reshape(x.shape), np.signbit(x).astype(np.uint8))
    assert np.array_equal(M4.unpack_nibbles(p), ref)


@pytest.mark.parametrize("rule", MX.RULES)
@pytest.mark.parametrize("block", [16, 32])
def test_e4m3_elements_bruteforce_and_error(rule, block):
    x = _rows(3)
    q, c = MX.quantize_mx(x, block, "e4m3", rule)
    s = np.exp2(c.astype(np.float64) - 127)
    v = (x.astype(np.float64).reshape(x.shape[0], -1, block) / s[..., None]).reshape(x.shape)
    assert np.array_equal(q, E4.e4m3_from_f32_bruteforce(v.astype(np.float32)))
    # dequantized error: half a spacing of E4M3 (relative 2^-4) for values in the
    # normal range and below 448, absolute 2^-10 * scale below it
    deq = (e4m3_decode(q).reshape(x.shape[0], -1, block) * s[..., None]).reshape(x.shape)
    av = np.abs(v)
    ok = av < 448
    err = np.abs(deq - x)[ok]
    bound = np.maximum(np.abs(x)[ok] * 2.0 ** -4, (2.0 ** -10 * np.repeat(s, block, axis=1))[ok])
    assert np.all(err <= bound)


def test_e4m3_ocp_block_max_in_top_binade_and_saturation():
    x = _rows(4)
    q, c = MX.quantize_mx(x, 32, "e4m3", "ocp")
    codes = q.reshape(x.shape[0], -1, 32)
    amax_pos = np.abs(x.reshape(codes.shape)).argmax(axis=2)
    top = np.take_along_axis(codes & 0x7F, amax_pos[..., None], 2)[..., 0]
    nz = np.abs(x.reshape(codes.shape)).max(axis=2) > 0
    # the maximum lands in [256, 448] (exponent field 15) under the OCP rule
    assert np.all((top[nz] >> 3) == 15)
    assert np.all(top[~nz] == 0)
