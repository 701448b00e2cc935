"""Pins of the oracle's W4A8 MoE pieces: routing, scale recipe, LUT, grouped GEMM (CPU)."""
import numpy as np

from oracle import int4 as I4
from oracle import w4a8 as W
from oracle.e4m3 import e4m3_from_f32
from oracle.formats import bf16_decode, e4m3_decode
from synthetic import moe_router_logits, to_bf16_bits


def test_routing_topk_bruteforce_and_ties():
    z = moe_router_logits(0, 256, 64)
    ids, w = W.route_topk(z, 8)
    for t in range(256):
        order = sorted(range(64), key=lambda e: (-float(z[t, e]), e))[:8]
        assert list(ids[t]) == order
        p = np.exp(z[t].astype(np.float64) - z[t].max()); p /= p.sum()
        assert np.allclose(w[t], p[order], rtol=1e-6)
    tie = np.zeros((1, 6), np.float32)
    tie[0, [1, 4]] = 1.0
    ids, _ = W.route_topk(tie, 4)
    assert list(ids[0]) == [1, 4, 0, 2]


def test_routing_weights_closed_forms():
    # logits ln(1), ln(2), ..., ln(E): the softmax is (e + 1) / (E (E + 1) / 2)
    E, k = 64, 8
    z = np.log(np.arange(1, E + 1, dtype=np.float64)).astype(np.float32)[None, :]
    ids, w = W.route_topk(z, k)
    assert list(ids[0]) == list(range(E - 1, E - 1 - k, -1))
    expect = (np.arange(E, E - k, -1) / (E * (E + 1) / 2)).astype(np.float64)
    assert np.allclose(w[0], expect, rtol=2e-6, atol=0)
    # two experts: logits (a, 0) give sigmoid(a) and 1 - sigmoid(a)
    a = np.float32(1.25)
    ids, w = W.route_topk(np.array([[a, 0.0]], np.float32), 2)
    sig = 1.0 / (1.0 + np.exp(-1.25))
    assert list(ids[0]) == [0, 1] and abs(w[0, 0] - sig) < 1e-7 and abs(w[0, 1] - (1 - sig)) < 1e-7
    # equal logits: every probability 1 / E, ids in increasing order
    ids, w = W.route_topk(np.full((1, 16), 3.5, np.float32), 4)
    assert list(ids[0]) == [0, 1, 2, 3] and np.all(w[0] == np.float32(1 / 16))
    # a constant added to every logit changes nothing
    g = np.random.default_rng(7)
    z = g.standard_normal((8, 64)).astype(np.float32) * 0.5
    i0, w0 = W.route_topk(z, 8)
    i1, w1 = W.route_topk(z + np.float32(4.0), 8)
    assert np.array_equal(i0, i1) and np.allclose(w0, w1, rtol=1e-6)


def test_channel_scale_closed_forms():
    # channels whose largest group scale is 448 * 2^j: ch = 8 * 2^j exactly and
    # that group's fp8 scale is 56 exactly; the other groups' codes round
    # s / ch to the nearest E4M3 value
    js = np.arange(-6, 3)
    smax = 448.0 * np.exp2(js)
    others = np.array([1.0, 3.0, 0.5, 100.0]) * np.exp2(js)[:, None]
    s = np.concatenate([smax[:, None], others], axis=1).astype(np.float32)
    bits = to_bf16_bits(s)
    assert np.array_equal(bf16_decode(bits), s)                   # every value exact in bf16
    s8, ch = W.scale_recipe(bits)
    assert np.array_equal(ch, (8.0 * np.exp2(js)).astype(np.float32))
    assert np.all(e4m3_decode(s8[:, 0]) == 56.0)
    ratio = others / (8.0 * np.exp2(js))[:, None]                 # exact: powers of two
    assert np.array_equal(s8[:, 1:], e4m3_from_f32(ratio.astype(np.float32)))
    # any channel: ch / 8 is the float nearest amax / 448 (checked in fp64)
    g = np.random.default_rng(3)
    sb = to_bf16_bits(np.abs(g.standard_normal((200, 16))).astype(np.float32) * 0.01)
    _, ch = W.scale_recipe(sb)
    amax = bf16_decode(sb).max(axis=1).astype(np.float64) / 448.0
    c8 = ch.astype(np.float64) / 8.0
    ulp = np.spacing(np.abs(c8).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(c8 - amax) <= ulp / 2)


def test_grouping_is_stable_and_complete():
    z = moe_router_logits(1, 300, 16)
    ids, _ = W.route_topk(z, 4)
    off, tok, slot = W.group_by_expert(ids, 16)
    assert off[0] == 0 and off[-1] == 300 * 4
    for e in range(16):
        rows = np.arange(off[e], off[e + 1])
        assert np.all(np.diff(tok[rows]) > 0)                  # increasing token ids
        assert np.all(ids[tok[rows], slot[rows]] == e)
        assert set(tok[rows]) == set(np.where((ids == e).any(axis=1))[0])


def test_scale_recipe_range_and_lut_no_clip():
    g = np.random.default_rng(0)
    w = (g.standard_normal((96, 512)) * 0.02).astype(np.float32)
    packed, sb, q = I4.quantize_int4(w, 128)
    s8, ch = W.scale_recipe(sb)
    v = e4m3_decode(s8)
    # the largest group scale of each channel maps to 448/8 = 56
    assert np.all(v.max(axis=1) == 56.0)
    assert np.all(v > 0)
    # (the channel scale itself: test_channel_scale_closed_forms)
    table = W.lut(s8)
    tv = e4m3_decode(table)
    # |w * s8| <= 8 * 56 = 448: no entry saturates, every entry is the rounded product
    wv = np.where(np.arange(16) >= 8, np.arange(16) - 16, np.arange(16))
    exact = v[..., None] * wv
    assert np.abs(exact).max() <= 448
    assert np.array_equal(table, e4m3_from_f32(exact.astype(np.float32)))
    # sign symmetry: entry(-w) = entry(w) with the sign bit, for w = 1..7
    for k in range(1, 8):
        assert np.array_equal(table[..., 16 - k], table[..., k] | 0x80)
    assert np.all(np.abs(tv - exact) <= np.abs(exact) * 2.0 ** -4 + 2.0 ** -10)


def test_grouped_gemm_reference_bruteforce_small():
    g = np.random.default_rng(5)
    T, H, N, E, k = 12, 256, 16, 4, 2
    logits = g.standard_normal((T, E)).astype(np.float32)
    ids, _ = W.route_topk(logits, k)
    off, tok, _ = W.group_by_expert(ids, E)
    x8, a = W.quantize_tokens(to_bf16_bits(g.standard_normal((T, H)).astype(np.float32)))
    experts = []
    for e in range(E):
        packed, sb, _ = I4.quantize_int4((g.standard_normal((N, H)) * 0.02).astype(np.float32), 128)
        s8, ch = W.scale_recipe(sb)
        experts.append((packed, s8, ch))
    y, absy = W.grouped_gemm_reference(x8, a, off, tok, experts, 128)
    # brute force triple loop in Python
    for r in range(off[-1]):
        e = int(np.searchsorted(off, r, side="right") - 1)
        packed, s8, ch = experts[e]
        q = I4.unpack_int4(packed)
        t = tok[r]
        for n in range(0, N, 5):
            acc = 0.0
            for kk in range(H):
                lutv = e4m3_decode(e4m3_from_f32(np.array([q[n, kk] * e4m3_decode(s8[n, kk // 128])], np.float32)))[0]
                acc += e4m3_decode(x8[t, kk]) * lutv
            want = acc * float(a[t]) * float(ch[n])
            assert abs(y[r, n] - want) <= 1e-12 * abs(want) + 1e-300
