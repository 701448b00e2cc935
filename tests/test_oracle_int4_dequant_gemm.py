"""Pins of the oracle's INT4 quantizer, dequantizers and reference GEMM (CPU)."""
import numpy as np
import pytest
import torch

from oracle import dequant as D
from oracle import gemm as G
from oracle import int4 as I4
from oracle.formats import bf16_decode, bf16_round, e2m1_decode, e8m0_decode, int_range
from synthetic import all_bf16_patterns, to_bf16_bits
from tests.conftest import golden_rows


def _torch_bf16_bits(v64):
    return torch.from_numpy(np.asarray(v64, np.float64)).to(torch.float32).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_int4_range_and_overhead():
    assert int_range(4) == (-8, 7)
    rows = {r[0]: r[1:] for r in golden_rows("int4_overhead.txt")}
    group, sbits = int(rows["group"][0]), int(rows["scale_bits"][0])
    assert sbits / group == float(rows["extra_bits_per_weight"][0])
    assert round((4 + sbits / group) / 8, 3) == float(rows["bytes_per_weight"][0])
    g = np.random.default_rng(0)
    w = (g.standard_normal((64, 512)) * 0.02).astype(np.float32)
    packed, sb, q = I4.quantize_int4(w, group)
    assert packed.nbytes + sb.nbytes == w.size * (4 + sbits / group) / 8
    assert q.min() >= -8 and q.max() <= 7


_SHORT_BF16 = np.arange(8, 0x7F80, 8, dtype=np.uint32).astype(np.uint16)      # low 3 mantissa bits zero


def _nearest_short_bf16(v):
    """Brute force: the positive bf16 value with 3 trailing zero mantissa bits
    nearest to each v (fp64), ties to the one whose bit 3 is clear."""
    cand = bf16_decode(_SHORT_BF16).astype(np.float64)
    i = np.clip(np.searchsorted(cand, v), 1, len(cand) - 1)
    lo, hi = cand[i - 1], cand[i]
    pick_hi = (hi - v < v - lo) | ((hi - v == v - lo) & ((_SHORT_BF16[i] & 8) == 0))
    return np.where(pick_hi, _SHORT_BF16[i], _SHORT_BF16[i - 1])


def test_int4_scale_makes_every_product_exact_in_bf16():
    # every stored scale has 3 trailing zero mantissa bits, and then q * s is a
    # bf16 value for every code: dequantization involves no rounding
    g = np.random.default_rng(3)
    w = (g.standard_normal((16, 1024)) * np.exp2(g.integers(-40, 40, (16, 1)))).astype(np.float32)
    _, sb, _ = I4.quantize_int4(w, 128)
    assert np.all(sb & 7 == 0)
    s = bf16_decode(sb).astype(np.float64)
    prods = s[..., None] * np.arange(-8, 8)
    assert np.array_equal(bf16_decode(bf16_round(prods)), prods)
    # a 6-bit significand would not have this property (negative control)
    s6 = bf16_decode(sb | 4).astype(np.float64)
    p6 = s6[..., None] * np.arange(-8, 8)
    assert not np.array_equal(bf16_decode(bf16_round(p6)), p6)


def test_int4_bruteforce_and_bound():
    g = np.random.default_rng(1)
    w = (g.standard_normal((8, 256)) * np.exp2(g.integers(-10, 10, (8, 1)))).astype(np.float32)
    for group in (32, 64, 128):
        packed, sb, q = I4.quantize_int4(w, group)
        s = bf16_decode(sb).astype(np.float32)
        r = (w.reshape(8, -1, group) / s[:, :, None]).astype(np.float64)
        cand = np.arange(-8, 8)
        d = np.abs(r[..., None] - cand)
        best = d.min(axis=-1, keepdims=True)
        ties = d == best
        even = ties & (cand % 2 == 0)
        pick = np.where(even.any(-1), even.argmax(-1), ties.argmax(-1))
        assert np.array_equal(q.reshape(r.shape), cand[pick])
        # self-consistency: |x - q*s| <= s/2 for unclamped elements
        err = np.abs(w.reshape(r.shape) - q.reshape(r.shape) * s[:, :, None].astype(np.float64))
        unclamped = np.abs(r) <= 7.5
        bound = np.broadcast_to(s[:, :, None].astype(np.float64) * 0.5 * (1 + 2.0 ** -20), r.shape)
        assert np.all(err[unclamped] <= bound[unclamped])
        # the scale is the bf16 value with a 5-bit significand nearest to
        # RN_f32(amax/7), ties to the even significand, found here by a search
        # over every such positive bf16 value
        amax = np.abs(w.reshape(r.shape)).max(axis=2)
        v = (amax / np.float32(7)).astype(np.float32).astype(np.float64).ravel()
        assert np.array_equal(sb.ravel(), _nearest_short_bf16(v))
        # the largest element of every group gets |q| = 7
        qg = np.abs(q.reshape(r.shape).astype(np.int64))
        at_max = np.abs(w.reshape(r.shape)) == amax[:, :, None]
        assert np.all(qg[at_max] == 7)


def test_int4_zero_group_and_pack():
    w = np.zeros((2, 128), np.float32)
    w[1, :64] = 0.5
    packed, sb, q = I4.quantize_int4(w, 64)
    assert bf16_decode(sb)[0, 0] == 1.0 and bf16_decode(sb)[0, 1] == 1.0
    assert np.all(q[0] == 0)
    g = np.random.default_rng(2)
    q = g.integers(-8, 8, (3, 64)).astype(np.int8)
    assert np.array_equal(I4.unpack_int4(I4.pack_int4(q)), q)
    # element 8i+j in bits 4j..4j+3 of word i, two's complement
    one = np.zeros((1, 8), np.int8); one[0, 3] = -1
    assert I4.pack_int4(one)[0, 0] == 0xF << 12


def test_dequant_e2m1_all_codes():
    # 16 element codes x 256 scale codes against the closed form, rounded by torch
    codes = np.arange(16, dtype=np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).reshape(1, 8)
    for sc in range(255):
        got = D.dequant_mxfp4(np.repeat(packed, 1, 0), np.full((1, 1), sc, np.uint8), 16)
        exact = e2m1_decode(codes) * 2.0 ** (sc - 127)
        with np.errstate(over="ignore"):
            want = _torch_bf16_bits(exact)
        assert np.array_equal(got[0], want), sc
    nan = D.dequant_mxfp4(packed, np.full((1, 1), 255, np.uint8), 16)
    assert np.all(np.isnan(bf16_decode(nan)))


def test_dequant_e4m3_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8).reshape(16, 16)
    got = D.dequant_e4m3(codes)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    gv, lv = bf16_decode(got), bf16_decode(lib)
    assert np.array_equal(np.isnan(gv), np.isnan(lv))
    assert np.array_equal(got[~np.isnan(gv)], lib[~np.isnan(lv)])


def test_dequant_int4_every_scale_pattern():
    s = all_bf16_patterns()
    sv = bf16_decode(s)
    s = s[np.isfinite(sv)]
    q = np.arange(-8, 8, dtype=np.int8)
    N = s.size
    packed = I4.pack_int4(np.tile(q, (N, 1)))
    got = D.dequant_int4(packed, s.reshape(N, 1), 16)
    exact = q[None, :].astype(np.float64) * bf16_decode(s)[:, None]      # exact product
    with np.errstate(over="ignore"):
        want = _torch_bf16_bits(exact)
    assert np.array_equal(got, want)


def test_accumulation_all_ones():
    rows = {r[0]: r[1] for r in golden_rows("accumulation.txt")}
    K = int(rows["terms"])
    one = to_bf16_bits(np.ones((1, K), np.float32))
    y, a = G.reference(one, one)
    assert y[0, 0] == float(rows["fp32_sum"]) and a[0, 0] == K
    # negative control: a serial bf16 accumulator stalls
    acc = np.uint16(0)
    for _ in range(K):
        acc = bf16_round(bf16_decode(acc) + 1.0)
    assert bf16_decode(acc) == float(rows["bf16_serial_sum"])


def test_reference_matmul_exact_on_integers():
    g = np.random.default_rng(3)
    x = g.integers(-8, 9, (7, 96)).astype(np.float32)
    w = g.integers(-8, 9, (11, 96)).astype(np.float32)
    y, a = G.reference(to_bf16_bits(x), to_bf16_bits(w), chan_scale=np.full(11, 2.0))
    want = np.zeros((7, 11))
    for i in range(7):
        for j in range(11):
            want[i, j] = 2 * sum(int(x[i, k]) * int(w[j, k]) for k in range(96))
    assert np.array_equal(y, want)
    assert np.array_equal(a, 2 * np.abs(x).astype(np.int64) @ np.abs(w).astype(np.int64).T)


def test_tolerance_bound():
    g = np.random.default_rng(4)
    x = to_bf16_bits(g.standard_normal((4, 4096)).astype(np.float32))
    w = to_bf16_bits((g.standard_normal((64, 4096)) * 0.02).astype(np.float32))
    y, a = G.reference(x, w)
    # an fp32 serial sum followed by a bf16 rounding is inside the bound
    xf, wf = bf16_decode(x).astype(np.float32), bf16_decode(w).astype(np.float32)
    acc = np.zeros((4, 64), np.float32)
    for k in range(4096):
        acc += xf[:, k:k + 1] * wf[:, k][None, :]
    yb = bf16_decode(bf16_round(acc.astype(np.float64)))
    assert G.within_tolerance(yb, y, a).all()
    u = 2.0 ** -24
    gamma = 4095 * u / (1 - 4095 * u)
    assert np.all(np.abs(acc - y) <= gamma * a)
    # an error of 2e-3 * sum|x w| is rejected
    assert not G.within_tolerance(y + 2e-3 * a + 1e-2 * np.abs(y), y, a).any()
    assert G.worst_ratio(yb, y, a) <= 1.0
