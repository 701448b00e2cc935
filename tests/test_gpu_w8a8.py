"""GPU parity of the W8A8 FP8 path: the static per-tensor and 128 x 128 block
quantizers bit for bit, the GEMM within
|y - y_ref| <= 8e-3 |y_ref| + 1e-3 sum_k |a_k s_a b_k s_b| of the oracle's
block-scaled fp64 reference.  GEMM operands are quantized by the oracle."""
import numpy as np
import pytest
import torch

from oracle import e4m3 as OE
from oracle import gemm as OG
from oracle import w8a8 as O8
from oracle.formats import bf16_decode
from synthetic import prefill_inputs, to_bf16_bits, bf16_bits_to_f32
from tests.gpu_helpers import banner, dev_bf16, dev_f32, dev_u8, host_bits16, host_f32, host_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def W():
    import weight_only_quantized_quant_amd as W
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return W


def _wide(rows, cols, seed):
    g = np.random.default_rng(seed)
    a = (g.standard_normal((rows, cols)) * np.exp2(g.integers(-12, 12, (rows, 1)))).astype(np.float32)
    idx = g.choice(a.size, size=a.size // 200, replace=False)
    a.reshape(-1)[idx] *= np.float32(60.0)
    a[0, :64] = 0.0
    a[1, :32] = -0.0
    return a


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("scale", [0.05, 1.0, 3.7e-5, 2.0 ** -100, 1.0e30])
def test_static_quantizer(W, bf16, scale):
    a = _wide(33, 512, seed=int(bf16) + 1)
    if bf16:
        bits = to_bf16_bits(a)
        x, ref = dev_bf16(bits), bf16_bits_to_f32(bits)
    else:
        x, ref = dev_f32(a), a
    banner("quantize_e4m3_static", scale, "bf16" if bf16 else "fp32")
    s = torch.tensor([scale], dtype=torch.float32, device="cuda")
    codes = W.quantize_e4m3_static(x, s)
    assert np.array_equal(host_u8(codes), O8.quantize_e4m3_static(ref, float(np.float32(scale))))


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("N,K", [(300, 512), (128, 128), (17, 256), (1024, 1024)])
def test_block2d_quantizer(W, bf16, N, K):
    w = _wide(N, K, seed=N + K)
    w[-1, -128:] = 0.0                                   # an all-zero block row in the last block
    if bf16:
        bits = to_bf16_bits(w)
        x, ref = dev_bf16(bits), bf16_bits_to_f32(bits)
    else:
        x, ref = dev_f32(w), w
    banner("quantize_e4m3_block2d", N, K, "bf16" if bf16 else "fp32")
    codes, scales = W.quantize_e4m3_block2d(x)
    wc, ws = O8.quantize_e4m3_block2d(ref)
    assert np.array_equal(host_f32(scales), ws)
    assert np.array_equal(host_u8(codes), wc)


def _operands(M, N, K, seed, a_mode, b_mode):
    """Oracle-quantized operands, their device tensors, strides and the
    per-(row, K block) scale matrices of the reference."""
    g = np.random.default_rng(seed)
    x = (g.standard_normal((M, K)) * np.exp2(g.integers(-3, 3, (M, 1)))).astype(np.float32)
    x[:, g.choice(K, 2, replace=False)] *= 30
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[g.choice(N, 3, replace=False)] *= 20
    kb = K // 128
    if a_mode == "group":
        ac, sa = OE.quantize_e4m3(x, 128)
        a_args, a_full = (sa, kb, 1), O8.expand_scales(sa, M, kb)
    elif a_mode == "token":
        ac, sa = OE.quantize_e4m3(x, -1)
        a_args, a_full = (sa[:, 0], 1, 0), O8.expand_scales(sa[:, 0], M, kb)
    else:
        s = OE.e4m3_scale(np.abs(x).max())
        ac = O8.quantize_e4m3_static(x, float(s))
        a_args, a_full = (np.array([s], np.float32), 0, 0), O8.expand_scales(float(s), M, kb)
    if b_mode == "block":
        bc, sb = O8.quantize_e4m3_block2d(w)
        b_args, b_full = (sb, kb, 1, 128), O8.expand_scales(sb, N, kb, 128)
    elif b_mode == "channel":
        bc, sb = OE.quantize_e4m3(w, -1)
        b_args, b_full = (sb[:, 0], 1, 0, 1), O8.expand_scales(sb[:, 0], N, kb)
    else:
        s = OE.e4m3_scale(np.abs(w).max())
        bc = O8.quantize_e4m3_static(w, float(s))
        b_args, b_full = (np.array([s], np.float32), 0, 0, 1), O8.expand_scales(float(s), N, kb)
    return ac, a_args, a_full, bc, b_args, b_full


def _run(W, ac, a_args, bc, b_args):
    sa, as_m, as_k = a_args
    sb, bs_n, bs_k, gn = b_args
    return W.wq_gemm_w8a8(dev_u8(ac), dev_f32(np.ascontiguousarray(sa).reshape(-1)), as_m, as_k, dev_u8(bc),
                          dev_f32(np.ascontiguousarray(sb).reshape(-1)), bs_n, bs_k, gn)


def _check(y_dev, ac, a_full, bc, b_full, rows=None):
    y = bf16_decode(host_bits16(y_dev))
    if rows is not None:
        y, ac, a_full = y[rows], ac[rows], a_full[rows]
    ref, asum = O8.reference(ac, a_full, bc, b_full)
    ratio = OG.worst_ratio(y, ref, asum)
    assert np.isfinite(y).all()
    assert ratio <= 1.0, f"worst error / bound = {ratio:.3f}"


MODES = [("group", "block"), ("group", "channel"), ("token", "channel"), ("tensor", "tensor"), ("token", "block")]


@pytest.mark.parametrize("a_mode,b_mode", MODES)
@pytest.mark.parametrize("M,N,K", [(300, 520, 512), (17, 256, 256), (1, 384, 1024), (257, 33, 128), (512, 512, 1024),
                                   (64, 100, 384)])
def test_gemm_ragged(W, a_mode, b_mode, M, N, K):
    ac, a_args, a_full, bc, b_args, b_full = _operands(M, N, K, M + N + K, a_mode, b_mode)
    banner("w8a8", a_mode, b_mode, M, N, K)
    _check(_run(W, ac, a_args, bc, b_args), ac, a_full, bc, b_full)


def _random_w8a8_cases(n, seed=2028):
    """Seeded random shapes (M 1-600, N 3-3000, K a multiple of 128 up to
    4096) and scale layouts."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M, N, K = int(g.integers(1, 601)), int(g.integers(3, 3001)), 128 * int(g.integers(1, 33))
        if M * N * K > 1.5e9:
            continue
        a_mode, b_mode = MODES[len(out) % len(MODES)]
        out.append((a_mode, b_mode, M, N, K, int(g.integers(1 << 30))))
    return out


@pytest.mark.parametrize("a_mode,b_mode,M,N,K,seed", _random_w8a8_cases(15))
def test_gemm_random_shapes(W, a_mode, b_mode, M, N, K, seed):
    ac, a_args, a_full, bc, b_args, b_full = _operands(M, N, K, seed, a_mode, b_mode)
    banner("w8a8 random shape", a_mode, b_mode, M, N, K, seed)
    _check(_run(W, ac, a_args, bc, b_args), ac, a_full, bc, b_full)


def test_gemm_exact_small_integers(W):
    # unit scales and small E4M3 integers: every partial sum is exact in fp32,
    # so y is the single bf16 rounding of the exact product
    M, N, K = 64, 256, 512
    g = np.random.default_rng(5)
    vals = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0xC4], np.uint8)   # 0, 1, 2, 3, 4, -1, -2, -3
    ac = vals[g.integers(0, 8, (M, K))]
    bc = vals[g.integers(0, 8, (N, K))]
    one = np.ones(1, np.float32)
    banner("w8a8 exact integers")
    for a_args, b_args in (((one, 0, 0), (one, 0, 0, 1)), ((np.ones(M * 4, np.float32), 4, 1),
                                                          (np.ones(2 * 4, np.float32), 4, 1, 128))):
        y = _run(W, ac, a_args, bc, b_args)
        ref, _ = O8.reference(ac, np.ones((M, 4)), bc, np.ones((N, 4)))
        assert np.array_equal(host_bits16(y), to_bf16_bits(ref.astype(np.float32)))


def test_gemm_full_size_sampled_rows(W):
    # M = 8192, K = 4096, N = 14336: per-token-group activations x 128 x 128 weight blocks
    xbits, Wf = prefill_inputs(0)
    x = bf16_bits_to_f32(xbits)
    ac, sa = OE.quantize_e4m3(x, 128)
    bc, sb = O8.quantize_e4m3_block2d(Wf)
    banner("w8a8 full size 8192x4096 . 14336x4096, group x block")
    y = W.wq_gemm_w8a8(dev_u8(ac), dev_f32(sa.reshape(-1)), 32, 1, dev_u8(bc), dev_f32(sb.reshape(-1)), 32, 1, 128)
    # both rows at every 256-row tile boundary and 512 seed-chosen rows
    edges = np.concatenate([np.arange(0, 8192, 256), np.arange(255, 8192, 256)])
    rows = np.unique(np.concatenate([edges, np.random.default_rng(96).choice(8192, 512, replace=False)]))
    _check(y, ac, O8.expand_scales(sa, 8192, 32), bc, O8.expand_scales(sb, 14336, 32, 128), rows=rows)


def test_gemm_full_size_token_channel_sampled_rows(W):
    # M = 8192, K = 4096, N = 14336: per-token activations x per-channel weights
    # (the scales factor out of the K sum and apply in the epilogue)
    xbits, Wf = prefill_inputs(0)
    x = bf16_bits_to_f32(xbits)
    ac, sa = OE.quantize_e4m3(x, -1)
    bc, sb = OE.quantize_e4m3(Wf, -1)
    banner("w8a8 full size 8192x4096 . 14336x4096, token x channel")
    y = W.wq_gemm_w8a8(dev_u8(ac), dev_f32(sa[:, 0]), 1, 0, dev_u8(bc), dev_f32(sb[:, 0]), 1, 0, 1)
    edges = np.concatenate([np.arange(0, 8192, 256), np.arange(255, 8192, 256)])
    rows = np.unique(np.concatenate([edges, np.random.default_rng(97).choice(8192, 512, replace=False)]))
    _check(y, ac, O8.expand_scales(sa[:, 0], 8192, 32), bc, O8.expand_scales(sb[:, 0], 14336, 32), rows=rows)


def test_gemm_rejects_short_scale_arrays(W):
    a = torch.zeros((4, 256), dtype=torch.uint8, device="cuda")
    b = torch.zeros((8, 256), dtype=torch.uint8, device="cuda")
    s = torch.ones(1, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        W.wq_gemm_w8a8(a, s, 2, 1, b, s, 0, 0, 1)
