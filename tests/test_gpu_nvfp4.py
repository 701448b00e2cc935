"""GPU parity of the NVFP4 path (E2M1 blocks of 16 with an E4M3 scale and a
per-tensor fp32 scale): the quantizer and the dequantized operand bit for bit,
the matmul within |y - y_ref| <= 8e-3 |y_ref| + 1e-3 sum_k |x_k w_k| of the
oracle's fp64 reference.  Weights for the matmul are quantized by the oracle."""
import numpy as np
import pytest
import torch

from oracle import gemm as OG
from oracle import nvfp4 as ON
from oracle.formats import bf16_decode
from synthetic import all_bf16_patterns, bf16_bits_to_f32, decode_inputs, prefill_inputs, to_bf16_bits
from tests.gpu_helpers import banner, check_all_rows, dev_bf16, dev_f32, dev_u8, host_bits16, host_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def W():
    import weight_only_quantized_quant_amd as W
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return W


def tensor_scale(Wf):
    """Per-tensor scale mapping the tensor's maximum to 6 * 448 (the largest
    E2M1 value times the largest E4M3 value)."""
    return float(np.float32(np.abs(Wf).max() / (6.0 * 448.0)))


def _wide(rows, cols, seed):
    g = np.random.default_rng(seed)
    a = (g.standard_normal((rows, cols)) * np.exp2(g.integers(-30, 30, (rows, 1)))).astype(np.float32)
    idx = g.choice(a.size, size=a.size // 300, replace=False)
    a.reshape(-1)[idx] *= np.float32(100.0)
    a[0, :16] = 0.0
    a[0, 16:32] = -0.0
    a[1, :16] = (g.standard_normal(16) * 1e-40).astype(np.float32)
    a[2, :16] = (g.standard_normal(16) * 3e37).astype(np.float32)
    return a


def _quant_check(W, x_dev, ref_in, g):
    codes, scales = W.quantize_nvfp4(x_dev, g)
    wc, ws = ON.quantize_nvfp4(ref_in, g)
    assert np.array_equal(host_u8(scales), ws), g
    assert np.array_equal(host_u8(codes), wc), g


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("g", [1.0, 0.37, 2.0 ** -20, 3.0e6])
def test_quantize_wide_values(W, bf16, g):
    a = _wide(41, 512, seed=int(bf16) + 3)
    if bf16:
        bits = to_bf16_bits(a)
        x, ref_in = dev_bf16(bits), bf16_bits_to_f32(bits)
    else:
        x, ref_in = dev_f32(a), a
    banner("quantize_nvfp4 wide", "bf16" if bf16 else "fp32", g, a.shape)
    _quant_check(W, x, ref_in, g)


def test_quantize_all_bf16_patterns_as_blocks(W):
    bits = all_bf16_patterns()
    bits = bits[np.isfinite(bf16_bits_to_f32(bits))]
    bits = bits[: bits.size // 512 * 512].reshape(-1, 512)
    for g in (1.0, 2.0 ** -12, 1.0e-30):
        banner("quantize_nvfp4 bf16 patterns", g, bits.shape)
        _quant_check(W, dev_bf16(bits), bf16_bits_to_f32(bits), g)


def test_quantize_scale_decision_points(W):
    # block maxima at 6 * (every E4M3 value and the midpoints between them) * g,
    # and one ulp either side, so that both roundings are exercised
    from oracle.formats import E4M3_POS_VALUES
    v = E4M3_POS_VALUES
    mids = np.concatenate([v, (v[:-1] + v[1:]) / 2, [464.0, 500.0, 2.0 ** -10, 2.0 ** -11]])
    for g in (1.0, 0.0123):
        amax = (6.0 * mids * g).astype(np.float32)
        amax = np.concatenate([amax, np.nextafter(amax, np.float32(np.inf)), np.nextafter(amax, np.float32(0))])
        n = amax.size + (-amax.size) % 32
        amax = np.concatenate([amax, np.ones(n - amax.size, np.float32)])
        r = np.random.default_rng(5)
        blocks = (r.uniform(-1, 1, (n, 16)) * amax[:, None]).astype(np.float32)
        blocks[np.arange(n), r.integers(0, 16, n)] = amax
        x = blocks.reshape(-1, 512)
        banner("quantize_nvfp4 scale decision points", g, x.shape)
        _quant_check(W, dev_f32(x), x, g)


def test_quantize_full_size_weights(W):
    _, Wf = prefill_inputs(0, with_x=False)
    g = tensor_scale(Wf)
    banner("quantize_nvfp4 14336x4096 fp32", g)
    _quant_check(W, dev_f32(Wf), Wf, g)


def test_dequant_every_code_and_scale(W):
    # rows: scale codes 0..0x7E (all finite E4M3 values); each row holds every
    # E2M1 code in every nibble position
    K = 512
    codes = np.tile(np.arange(256, dtype=np.uint8), (127, 1))
    sc = np.repeat(np.arange(127, dtype=np.uint8)[:, None], K // 16, axis=1)
    banner("dequant nvfp4 every code x scale")
    out = W.wq_dequant(dev_u8(codes), W.WQ_E2M1X2, dev_u8(sc), W.WQ_E4M3, 16, 127, K)
    assert np.array_equal(host_bits16(out), ON.dequant_nvfp4(codes, sc))


def _nv_args(W, Wf, g):
    codes, s8 = ON.quantize_nvfp4(Wf, g)
    return (dev_u8(codes), W.WQ_E2M1X2, dev_u8(s8), W.WQ_E4M3, 16), ON.dequant_nvfp4(codes, s8)


def _check(y_dev, xbits, wdeq, g, rows=None):
    y = bf16_decode(host_bits16(y_dev))
    xb = xbits if rows is None else xbits[rows]
    if rows is not None:
        y = y[rows]
    ref, asum = OG.reference(xb, wdeq, np.full(wdeq.shape[0], g))
    ratio = OG.worst_ratio(y, ref, asum)
    assert np.isfinite(y).all()
    assert ratio <= 1.0, f"worst error / bound = {ratio:.3f}"


@pytest.mark.parametrize("M,N,K", [(1, 1000, 384), (3, 520, 512), (4, 272, 8192), (1, 300, 8192), (8, 272, 1024),
                                   (16, 300, 4096), (5, 17, 128), (2, 4096, 2048), (17, 256, 256), (300, 520, 512),
                                   (257, 33, 128), (512, 512, 1024),
                                   (9, 300, 14336), (12, 4500, 1536)])
def test_gemm_ragged(W, M, N, K):
    r = np.random.default_rng(M * 7 + N + K)
    Wf = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, r.choice(K, 3, replace=False)] *= 40
    xbits = to_bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    g = tensor_scale(Wf)
    args, wdeq = _nv_args(W, Wf, g)
    banner("gemm nvfp4", M, N, K, g)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N, alpha=g), xbits, wdeq, g)


@pytest.mark.parametrize("M,N,K", [(3, 9001, 4096), (1, 8200, 2048), (1, 4795, 4096), (2, 3205, 8192)])
def test_gemv_more_shapes(W, M, N, K):
    # ragged last tiles and balancing rounds of 8-row tiles, K 2048 to 8192
    r = np.random.default_rng(M * 13 + N + K)
    Wf = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, r.choice(K, 3, replace=False)] *= 40
    xbits = to_bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    g = tensor_scale(Wf)
    args, wdeq = _nv_args(W, Wf, g)
    banner("gemv more shapes nvfp4", M, N, K, g)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N, alpha=g), xbits, wdeq, g)


def test_gemm_alpha_one_and_unit_scales(W):
    # g = 1 with every block scale 1.0: y = x . e2m1 values exactly representable
    K, N, M = 512, 64, 3
    r = np.random.default_rng(2)
    codes = r.integers(0, 256, (N, K // 2), dtype=np.uint8)
    s8 = np.full((N, K // 16), 0x38, np.uint8)                     # E4M3 1.0
    xbits = to_bf16_bits(r.integers(-4, 5, (M, K)).astype(np.float32))
    banner("gemm nvfp4 unit scales")
    for m in (1, M):
        y = W.wq_gemm(dev_bf16(xbits[:m]), dev_u8(codes), W.WQ_E2M1X2, dev_u8(s8), W.WQ_E4M3, 16, N)
        ref, _ = OG.reference(xbits[:m], ON.dequant_nvfp4(codes, s8))
        # small integers times E2M1 values sum exactly in fp32 (multiples of 0.5
        # below 2^14), so y is the single bf16 rounding of the exact result
        assert np.array_equal(bf16_decode(host_bits16(y)), bf16_decode(to_bf16_bits(ref.astype(np.float32))))


@pytest.fixture(scope="module")
def decode_nv(W):
    _, Wf = decode_inputs(1, 0)
    g = tensor_scale(Wf)
    return _nv_args(W, Wf, g) + (g,)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_full_size(W, decode_nv, M):
    xbits, _ = decode_inputs(M, seed=20 + M, with_weight=False)
    args, wdeq, g = decode_nv
    banner("decode nvfp4 full size M", M)
    y = W.wq_gemm(dev_bf16(xbits), *args, 14336, alpha=g)
    y2 = W.wq_gemm(dev_bf16(xbits), *args, 14336, alpha=g)
    assert torch.equal(y, y2)
    _check(y, xbits, wdeq, g)


def test_prefill_full_size_all_rows(W):
    xbits, Wf = prefill_inputs(0)
    g = tensor_scale(Wf)
    args, wdeq = _nv_args(W, Wf, g)
    banner("prefill nvfp4 full size 8192x4096 . 14336x4096, all rows")
    y = W.wq_gemm(dev_bf16(xbits), *args, 14336, alpha=g)
    check_all_rows(y, xbits, wdeq, np.full(wdeq.shape[0], g))


def test_alpha_scales_the_output(W):
    r = np.random.default_rng(9)
    Wf = (r.standard_normal((272, 512)) * 0.02).astype(np.float32)
    xbits = to_bf16_bits(r.standard_normal((2, 512)).astype(np.float32))
    args, wdeq = _nv_args(W, Wf, 1.0)
    banner("gemm nvfp4 alpha")
    for M in (2, 20):
        xb = np.tile(xbits, (M // 2, 1))
        y1 = W.wq_gemm(dev_bf16(xb), *args, 272)
        y4 = W.wq_gemm(dev_bf16(xb), *args, 272, alpha=4.0)
        assert torch.equal(y4.float(), 4 * y1.float())             # a power of two commutes with the rounding
        _check(W.wq_gemm(dev_bf16(xb), *args, 272, alpha=-0.3), xb, wdeq, -0.3)
    with pytest.raises(ValueError):
        W.wq_gemm(dev_bf16(xbits), *args, 272, alpha=float("nan"))


def _random_cases(n, seed=2025):
    """Seeded random shapes: M 1-300, N 1-5000, K a multiple of 128 up to 5120."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(np.exp(g.uniform(0, np.log(300))))
        N = int(g.integers(1, 5001))
        K = 128 * int(g.integers(1, 41))
        if M * N * K > 1.5e9:
            continue
        out.append((M, N, K, int(g.integers(1 << 30))))
    return out


@pytest.mark.parametrize("M,N,K,seed", _random_cases(16))
def test_gemm_random_shapes(W, M, N, K, seed):
    r = np.random.default_rng(seed)
    Wf = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, r.choice(K, 3, replace=False)] *= 40
    xbits = to_bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    g = tensor_scale(Wf)
    args, wdeq = _nv_args(W, Wf, g)
    banner("gemm random shape nvfp4", M, N, K, seed)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N, alpha=g), xbits, wdeq, g)


def _random_quant_cases(n, seed=2030):
    """Seeded random shapes: 3-300 rows, 32-2048 columns in steps of 16."""
    g = np.random.default_rng(seed)
    return [(int(g.integers(3, 301)), 16 * int(g.integers(2, 129)), bool(i % 2), int(g.integers(1 << 30)))
            for i in range(n)]


@pytest.mark.parametrize("rows,cols,bf16,seed", _random_quant_cases(8))
def test_quantize_random_shapes(W, rows, cols, bf16, seed):
    # seeded random shapes, wide values: codes and scales bit for bit
    a = _wide(rows, cols, seed)
    if bf16:
        bits = to_bf16_bits(a)
        x, ref_in = dev_bf16(bits), bf16_bits_to_f32(bits)
    else:
        x, ref_in = dev_f32(a), a
    banner("nvfp4 quantize random shape", rows, cols, "bf16" if bf16 else "fp32")
    _quant_check(W, x, ref_in, tensor_scale(ref_in))
