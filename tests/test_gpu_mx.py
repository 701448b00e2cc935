"""GPU parity of the MX quantizer with a choice of E8M0 rule and E2M1 or E4M3
elements against the CPU oracle: codes and scales must match bit for bit."""
import numpy as np
import pytest
import torch

from oracle import mx as OX
from oracle import mxfp4 as OM
from oracle.formats import f32_from_bits
from synthetic import act_quant_inputs, all_bf16_patterns, bf16_bits_to_f32, to_bf16_bits
from tests.gpu_helpers import banner, dev_bf16, dev_f32, host_u8

pytestmark = pytest.mark.gpu

RULES = ("round", "half", "ocp", "floor_div", "ceil_div")
ELEMS = ("e2m1", "e4m3")


@pytest.fixture(scope="module")
def W():
    import weight_only_quantized_quant_amd as W
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return W


def _wide(rows, cols, seed, block):
    """Per-row exponent spread, outliers, zero, subnormal-range and huge blocks."""
    g = np.random.default_rng(seed)
    a = (g.standard_normal((rows, cols)) * np.exp2(g.integers(-60, 60, (rows, 1)))).astype(np.float32)
    idx = g.choice(a.size, size=a.size // 300, replace=False)
    a.reshape(-1)[idx] *= np.float32(100.0)
    a[0, :block] = 0.0
    a[3, block:2 * block] = 0.0
    a[1, :block] = (g.standard_normal(block) * 1e-40).astype(np.float32)
    a[2, :block] = (g.standard_normal(block) * 3e37).astype(np.float32)
    a[4, :block] = -np.abs(a[4, :block])
    return a


def _edge_maxima(block):
    """Blocks whose maximum sits on or next to every rule's decision point:
    fractions 0.5, 0.75, 0.9375 of a binade, e * 2^k for e in {6, 448}, the
    subnormal quotient thresholds, and the fp32 extremes."""
    fr = np.array([0, 0x400000, 0x600000, 0x780000, 0x7FFFFF], np.int64)
    e = np.array([1, 2, 3, 8, 9, 10, 100, 127, 130, 200, 253, 254], np.int64)
    m = (fr[None, :, None] + np.array([-1, 0, 1])[None, None, :]) & 0x7FFFFF
    bits = ((e[:, None, None] << 23) | m).reshape(-1)
    pw = np.concatenate([np.float32(6.0) * np.exp2(np.arange(-128, 125, 7.0)),
                         np.float32(448.0) * np.exp2(np.arange(-135, 118, 7.0))]).astype(np.float32)
    pw_bits = np.concatenate([f32_from_bits(np.zeros(1, np.uint32)), pw]).view(np.uint32).astype(np.int64)
    pw_bits = (pw_bits[:, None] + np.array([-1, 0, 1])[None, :]).reshape(-1)
    sub = np.array([1, 0x200000, 0x400000, 0x400001, 0x7FFFFF, 0x00C00000, 0x01400000, 0x7F7FFFFF], np.int64)
    vmax = f32_from_bits(np.concatenate([bits, pw_bits, sub]).clip(0, 0x7F7FFFFF).astype(np.uint32))
    n = vmax.size + (-vmax.size) % 16
    vmax = np.concatenate([vmax, np.ones(n - vmax.size, np.float32)])
    g = np.random.default_rng(9)
    blocks = (g.uniform(-1, 1, (n, block)) * vmax[:, None]).astype(np.float32)
    pos = g.integers(0, block, n)
    blocks[np.arange(n), pos] = vmax * np.where(g.integers(0, 2, n) == 1, -1, 1).astype(np.float32)
    return blocks.reshape(-1, 16 * block)


def _run(W, x_dev, ref_in, block, elem, rule):
    codes, scales = W.quantize_mx(x_dev, block, elem, rule)
    wc, ws = OX.quantize_mx(ref_in, block, elem, rule)
    assert np.array_equal(host_u8(scales), ws), (elem, rule, block)
    assert np.array_equal(host_u8(codes), wc), (elem, rule, block)


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("block", [16, 32])
@pytest.mark.parametrize("bf16", [False, True])
def test_mx_wide_values(W, rule, elem, block, bf16):
    a = _wide(37, 512, seed=block + 3 * bf16, block=block)
    if bf16:
        bits = to_bf16_bits(a)
        x, ref_in = dev_bf16(bits), bf16_bits_to_f32(bits)
    else:
        x, ref_in = dev_f32(a), a
    banner("quantize_mx", rule, elem, block, "bf16" if bf16 else "fp32", a.shape)
    _run(W, x, ref_in, block, elem, rule)


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("elem", ELEMS)
def test_mx_rule_decision_points(W, rule, elem):
    for block in (16, 32):
        a = _edge_maxima(block)
        banner("quantize_mx decision points", rule, elem, block, a.shape)
        _run(W, dev_f32(a), a, block, elem, rule)


@pytest.mark.parametrize("rule", RULES)
def test_mx_all_bf16_patterns_as_blocks(W, rule):
    bits = all_bf16_patterns()
    bits = bits[np.isfinite(bf16_bits_to_f32(bits))]
    bits = bits[: bits.size // 512 * 512].reshape(-1, 512)
    for elem in ELEMS:
        for block in (32, 16):
            banner("quantize_mx bf16 patterns", rule, elem, block, bits.shape)
            _run(W, dev_bf16(bits), bf16_bits_to_f32(bits), block, elem, rule)


def test_mx_round_e2m1_equals_quantize_mxfp4(W):
    a = _wide(64, 1024, seed=5, block=32)
    x = dev_f32(a)
    banner("quantize_mx round/e2m1 vs quantize_mxfp4", a.shape)
    for block in (16, 32):
        c0, s0 = W.quantize_mxfp4(x, block)
        c1, s1 = W.quantize_mx(x, block, "e2m1", "round")
        assert torch.equal(c0, c1) and torch.equal(s0, s1)


def test_mx_single_row_and_tail_chunk(W):
    # 32 columns: one block 32 per row, an odd number of 16-element chunks overall
    a = _wide(7, 32, seed=8, block=32)
    banner("quantize_mx 7x32")
    for elem in ELEMS:
        for rule in RULES:
            for block in (16, 32):
                _run(W, dev_f32(a), a, block, elem, rule)


@pytest.mark.parametrize("rule", ["round", "ceil_div"])
def test_mxfp8_activation_full_size_sampled_rows(W, rule):
    # 4096 x 7168 bf16 activations, MXFP8 block 32; the oracle checks 96 rows
    bits = act_quant_inputs(0)
    banner("quantize_mx e4m3 block 32, 4096x7168 bf16", rule)
    codes, scales = W.quantize_mx(dev_bf16(bits), 32, "e4m3", rule)
    hc, hs = host_u8(codes), host_u8(scales)
    rows = np.unique(np.concatenate([[0, 4095], np.random.default_rng(1).choice(4096, 94, replace=False)]))
    wc, ws = OX.quantize_mx(bf16_bits_to_f32(bits[rows]), 32, "e4m3", rule)
    assert np.array_equal(hs[rows], ws)
    assert np.array_equal(hc[rows], wc)


def test_mx_invalid_arguments(W):
    x = torch.zeros((4, 64), device="cuda")
    with pytest.raises(ValueError):
        W.quantize_mx(x, 32, "e5m2", "round")
    with pytest.raises(ValueError):
        W.quantize_mx(x, 32, "e4m3", "nearest")
    with pytest.raises(ValueError):
        W.quantize_mx(x, 64, "e4m3", "round")
    with pytest.raises(ValueError):
        W.quantize_mx(torch.zeros((4, 48), device="cuda"), 16, "e4m3", "round")
