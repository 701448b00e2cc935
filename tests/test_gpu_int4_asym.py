"""GPU parity of asymmetric INT4 (x = s (q - z)): the quantizer and the
dequantized operand bit for bit, the matmul within
|y - y_ref| <= 8e-3 |y_ref| + 1e-3 sum_k |x_k w_k| of the oracle's fp64
reference.  Weights for the matmul are quantized by the oracle."""
import numpy as np
import pytest
import torch

from oracle import gemm as OG
from oracle import int4_asym as OA
from oracle.formats import bf16_decode
from synthetic import all_bf16_patterns, bf16_bits_to_f32, decode_inputs, prefill_inputs, to_bf16_bits
from tests.gpu_helpers import banner, check_all_rows, dev_bf16, dev_f32, dev_words, host_bits16, host_words

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def W():
    import weight_only_quantized_quant_amd as W
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return W


def scale_zero_words(sb, z):
    """The WQ_BF16Z layout: bf16 scale bits in the low half, z in bits 16..23."""
    return np.asarray(sb, np.uint32) | (np.asarray(z, np.uint32) << 16)


def _wide(rows, cols, seed, shift=0.0):
    g = np.random.default_rng(seed)
    a = g.standard_normal((rows, cols)) * np.exp2(g.integers(-30, 30, (rows, 1)))
    a = a + shift * np.abs(a).max(axis=1, keepdims=True)
    a = a.astype(np.float32)
    idx = g.choice(a.size, size=a.size // 300, replace=False)
    a.reshape(-1)[idx] *= np.float32(20.0)
    a[0, :128] = 0.0
    a[1, :128] = (g.standard_normal(128) * 1e-40).astype(np.float32)
    a[2, :128] = np.abs(a[2, :128])
    a[3, :128] = -np.abs(a[3, :128])
    return a


def _quant_check(W, x_dev, ref_in, group):
    packed, sz = W.quantize_int4_asym(x_dev, group)
    wp, sb, z = OA.quantize_int4_asym(ref_in, group)
    assert np.array_equal(host_words(sz), scale_zero_words(sb, z)), group
    assert np.array_equal(host_words(packed), wp), group


@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("shift", [0.0, 0.8, -0.6])
def test_quantize_wide_values(W, group, bf16, shift):
    a = _wide(37, 512, seed=group + int(bf16), shift=shift)
    if bf16:
        bits = to_bf16_bits(a)
        x, ref_in = dev_bf16(bits), bf16_bits_to_f32(bits)
    else:
        x, ref_in = dev_f32(a), a
    banner("quantize_int4_asym", group, "bf16" if bf16 else "fp32", shift, a.shape)
    _quant_check(W, x, ref_in, group)


def test_quantize_all_bf16_patterns_as_groups(W):
    # groups of consecutive patterns share a sign, so no group range overflows
    bits = all_bf16_patterns()
    bits = bits[np.isfinite(bf16_bits_to_f32(bits))]
    bits = bits[: bits.size // 512 * 512].reshape(-1, 512)
    for group in (32, 128):
        banner("quantize_int4_asym bf16 patterns", group, bits.shape)
        _quant_check(W, dev_bf16(bits), bf16_bits_to_f32(bits), group)


def test_quantize_full_size_weights(W):
    _, Wf = decode_inputs(1, 0)
    banner("quantize_int4_asym 14336x4096 fp32 group 128")
    _quant_check(W, dev_f32(Wf), Wf, 128)


def test_dequant_every_code_and_zero_point(W):
    # rows: zero-points 0..15 under three scales; every row holds every code
    K, group = 256, 32
    words = np.array([0x76543210, 0xFEDCBA98, 0x01234567, 0x89ABCDEF], np.uint32)
    packed = np.tile(np.resize(words, K // 8), (48, 1))
    sb = np.repeat(np.array([0x3F80, 0x3B24, 0x4A3D], np.uint16), 16)           # 1, ~2.5e-3, ~3.1e6
    z = np.tile(np.arange(16, dtype=np.uint8), 3)
    sbg = np.repeat(sb[:, None], K // group, axis=1)
    zg = np.repeat(z[:, None], K // group, axis=1)
    banner("dequant asymmetric int4 every code x zero-point")
    out = W.wq_dequant(dev_words(packed), W.WQ_UINT4X8, dev_words(scale_zero_words(sbg, zg)), W.WQ_BF16Z, group,
                       48, K)
    assert np.array_equal(host_bits16(out), OA.dequant_int4_asym(packed, sbg, zg, group))


def _args(W, Wf, group):
    packed, sb, z = OA.quantize_int4_asym(Wf, group)
    args = (dev_words(packed), W.WQ_UINT4X8, dev_words(scale_zero_words(sb, z)), W.WQ_BF16Z, group)
    return args, OA.dequant_int4_asym(packed, sb, z, group)


def _check(y_dev, xbits, wdeq, rows=None):
    y = bf16_decode(host_bits16(y_dev))
    xb = xbits if rows is None else xbits[rows]
    if rows is not None:
        y = y[rows]
    ref, asum = OG.reference(xb, wdeq)
    ratio = OG.worst_ratio(y, ref, asum)
    assert np.isfinite(y).all()
    assert ratio <= 1.0, f"worst error / bound = {ratio:.3f}"


@pytest.mark.parametrize("group", [32, 128])
@pytest.mark.parametrize("M,N,K", [(1, 1000, 384), (3, 520, 512), (4, 272, 8192), (1, 300, 8192), (8, 272, 1024),
                                   (16, 300, 4096), (5, 17, 128), (2, 4096, 2048), (17, 256, 256), (300, 520, 512),
                                   (257, 33, 128), (512, 512, 1024),
                                   (9, 300, 14336), (12, 4500, 1536)])
def test_gemm_ragged(W, group, M, N, K):
    r = np.random.default_rng(M * 5 + N + K + group)
    Wf = (r.standard_normal((N, K)) * 0.02 + 0.01 * r.standard_normal((N, 1))).astype(np.float32)
    Wf[:, r.choice(K, 3, replace=False)] *= 40
    xbits = to_bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    args, wdeq = _args(W, Wf, group)
    banner("gemm asymmetric int4", group, M, N, K)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq)


@pytest.mark.parametrize("group,M,N,K", [(32, 3, 9001, 4096), (128, 4, 8200, 2048), (32, 2, 4795, 4096),
                                         (128, 1, 3205, 8192)])
def test_gemv_more_shapes(W, group, M, N, K):
    # ragged last tiles and balancing rounds of 8-row tiles, K 2048 to 8192,
    # groups of 32 (128 scale-zero words per row at K = 4096) and 128
    r = np.random.default_rng(M * 3 + N + K + group)
    Wf = (r.standard_normal((N, K)) * 0.02 + 0.01 * r.standard_normal((N, 1))).astype(np.float32)
    Wf[:, r.choice(K, 3, replace=False)] *= 40
    xbits = to_bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    args, wdeq = _args(W, Wf, group)
    banner("gemv more shapes asymmetric int4", group, M, N, K)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq)


@pytest.fixture(scope="module")
def decode_asym(W):
    _, Wf = decode_inputs(1, 0)
    return _args(W, Wf, 128)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_full_size(W, decode_asym, M):
    xbits, _ = decode_inputs(M, seed=30 + M, with_weight=False)
    args, wdeq = decode_asym
    banner("decode asymmetric int4 full size M", M)
    y = W.wq_gemm(dev_bf16(xbits), *args, 14336)
    y2 = W.wq_gemm(dev_bf16(xbits), *args, 14336)
    assert torch.equal(y, y2)
    _check(y, xbits, wdeq)


def test_prefill_full_size_all_rows(W):
    xbits, Wf = prefill_inputs(0)
    args, wdeq = _args(W, Wf, 128)
    banner("prefill asymmetric int4 full size 8192x4096 . 14336x4096, all rows")
    y = W.wq_gemm(dev_bf16(xbits), *args, 14336)
    check_all_rows(y, xbits, wdeq)


def test_zero_point_shifts_the_result(W):
    # one-sided weights: the zero-point carries the offset; all-zero rows stay zero
    r = np.random.default_rng(8)
    Wf = (np.abs(r.standard_normal((200, 1024))) * 0.02 + 0.05).astype(np.float32)
    Wf[::9] = 0.0
    xbits = to_bf16_bits(r.standard_normal((4, 1024)).astype(np.float32))
    args, wdeq = _args(W, Wf, 64)
    banner("gemm asymmetric int4 one-sided")
    for M in (1, 4):
        y = W.wq_gemm(dev_bf16(xbits[:M]), *args, 200)
        _check(y, xbits[:M], wdeq)
        assert np.all(bf16_decode(host_bits16(y))[:, ::9] == 0.0)


def _random_cases(n, seed=2026):
    """Seeded random shapes: M 1-300, N 1-5000, K a multiple of 128 up to 5120,
    groups 32, 64 and 128 in turn."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(np.exp(g.uniform(0, np.log(300))))
        N = int(g.integers(1, 5001))
        K = 128 * int(g.integers(1, 41))
        if M * N * K > 1.5e9:
            continue
        out.append(((32, 64, 128)[len(out) % 3], M, N, K, int(g.integers(1 << 30))))
    return out


@pytest.mark.parametrize("group,M,N,K,seed", _random_cases(15))
def test_gemm_random_shapes(W, group, M, N, K, seed):
    r = np.random.default_rng(seed)
    Wf = (r.standard_normal((N, K)) * 0.02 + 0.01 * r.standard_normal((N, 1))).astype(np.float32)
    Wf[:, r.choice(K, 3, replace=False)] *= 40
    xbits = to_bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    args, wdeq = _args(W, Wf, group)
    banner("gemm random shape asymmetric int4", group, M, N, K, seed)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq)


def _random_quant_cases(n, seed=2031):
    """Seeded random shapes: 4-300 rows, 128-4096 columns in steps of 128,
    groups 32 to 128, shifted distributions."""
    g = np.random.default_rng(seed)
    return [((32, 64, 128)[i % 3], int(g.integers(4, 301)), 128 * int(g.integers(1, 33)), bool(i % 2),
             float(g.uniform(-0.8, 0.8)), int(g.integers(1 << 30))) for i in range(n)]


@pytest.mark.parametrize("group,rows,cols,bf16,shift,seed", _random_quant_cases(9))
def test_quantize_random_shapes(W, group, rows, cols, bf16, shift, seed):
    a = _wide(rows, cols, seed, shift)
    if bf16:
        bits = to_bf16_bits(a)
        x, ref_in = dev_bf16(bits), bf16_bits_to_f32(bits)
    else:
        x, ref_in = dev_f32(a), a
    banner("asymmetric int4 quantize random shape", group, rows, cols, "bf16" if bf16 else "fp32", shift)
    _quant_check(W, x, ref_in, group)
