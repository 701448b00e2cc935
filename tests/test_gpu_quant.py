"""GPU parity of the quantizers and the dequantizer against the CPU oracle:
codes, scales and dequantized weights must match bit for bit."""
import numpy as np
import pytest
import torch

from oracle import dequant as OD
from oracle import e4m3 as OE
from oracle import int4 as OI
from oracle import mxfp4 as OM
from oracle.formats import E4M3_POS_VALUES, bf16_decode, f32_from_bits
from synthetic import (act_quant_inputs, all_bf16_patterns, bf16_bits_to_f32, decode_inputs, mxfp4_gemv_inputs,
                       prefill_inputs, to_bf16_bits)
from tests.gpu_helpers import (banner, dev_bf16, dev_f32, dev_u8, dev_words, host_bits16, host_f32, host_u8,
                               host_words)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def W():
    import weight_only_quantized_quant_amd as W
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return W


def _wide(shape, seed, zero_blocks=0, block=128):
    """fp32 data with per-row exponent spread, outliers, zero and tiny blocks."""
    g = np.random.default_rng(seed)
    rows, cols = shape
    a = (g.standard_normal(shape) * np.exp2(g.integers(-40, 40, (rows, 1)))).astype(np.float32)
    idx = g.choice(a.size, size=max(1, a.size // 500), replace=False)
    a.reshape(-1)[idx] *= np.float32(100.0)
    nb = cols // block
    for i in range(zero_blocks):
        r, b = g.integers(0, rows), g.integers(0, nb)
        a[r, b * block:(b + 1) * block] = 0.0
    if rows > 2:
        a[1, :block] = (g.standard_normal(block) * 1e-40).astype(np.float32)      # subnormal-range block
        a[2, :block] = (g.standard_normal(block) * 3e37).astype(np.float32)       # near the top of fp32
    return a


# ---------------------------------------------------------------------------
# E4M3
# ---------------------------------------------------------------------------

def test_e4m3_cast_all_bf16_patterns(W):
    bits = all_bf16_patterns().reshape(256, 256)
    banner("e4m3 plain cast, 65,536 bf16 patterns")
    codes, _ = W.quantize_e4m3(dev_bf16(bits), 0)
    want = OE.e4m3_from_f32(bf16_bits_to_f32(bits))
    assert np.array_equal(host_u8(codes), want)


def test_e4m3_cast_fp32_sweep(W):
    v = E4M3_POS_VALUES
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    pts = [v.astype(np.float32), mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0))]
    g = np.random.default_rng(3)
    pts += [g.uniform(-600, 600, 300000).astype(np.float32), g.uniform(-2.0 ** -6, 2.0 ** -6, 50000).astype(np.float32),
            np.array([np.float32(200.04), 448, 464, 465, np.inf, -np.inf, np.nan, 0.0, -0.0, 1e-45], np.float32)]
    x = np.concatenate(pts + [-p for p in pts])
    x = np.concatenate([x, np.zeros((-x.size) % 64, np.float32)]).reshape(-1, 64)
    banner("e4m3 plain cast, fp32 sweep", x.shape)
    codes, _ = W.quantize_e4m3(dev_f32(x), 0)
    assert np.array_equal(host_u8(codes), OE.e4m3_from_f32(x))
    assert OE.e4m3_from_f32(np.array([np.float32(200.04)]))[0] == 0x75


@pytest.mark.parametrize("block", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("bf16", [False, True])
def test_e4m3_block(W, block, bf16):
    a = _wide((37, 1024), seed=block + bf16, zero_blocks=5, block=block)
    if bf16:
        bits = to_bf16_bits(a)
        x, ref_in = dev_bf16(bits), bf16_bits_to_f32(bits)
    else:
        x, ref_in = dev_f32(a), a
    banner("e4m3 per-block", block, "bf16" if bf16 else "fp32", a.shape)
    codes, scales = W.quantize_e4m3(x, block)
    wc, ws = OE.quantize_e4m3(ref_in, block)
    assert np.array_equal(host_f32(scales).view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(host_u8(codes), wc)


# rows held in registers in 1, 2 or 4 rounds of 2048 elements (up to 8192
# columns, each bound crossed) and longer rows read twice
@pytest.mark.parametrize("shape", [(5, 4096), (3, 136), (64, 1536), (1, 8), (2, 2056), (9, 6144), (4, 8192),
                                   (7, 8200), (3, 20000)])
def test_e4m3_per_row(W, shape):
    a = _wide(shape, seed=shape[1], block=8)
    bits = to_bf16_bits(a)
    banner("e4m3 per-row", shape)
    codes, scales = W.quantize_e4m3(dev_bf16(bits), -1)
    wc, ws = OE.quantize_e4m3(bf16_bits_to_f32(bits), -1)
    assert np.array_equal(host_f32(scales).view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(host_u8(codes), wc)


def test_e4m3_block128_activation_full_size(W):
    bits = act_quant_inputs(0)
    banner("e4m3 per-1x128, 4096x7168 bf16")
    codes, scales = W.quantize_e4m3(dev_bf16(bits), 128)
    codes2, scales2 = W.quantize_e4m3(dev_bf16(bits), 128)
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)      # deterministic
    wc, ws = OE.quantize_e4m3(bf16_bits_to_f32(bits), 128)
    assert np.array_equal(host_f32(scales).view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(host_u8(codes), wc)


# ---------------------------------------------------------------------------
# MXFP4
# ---------------------------------------------------------------------------

def test_mxfp4_gemv_weights(W):
    _, Wf = mxfp4_gemv_inputs(0)
    banner("mxfp4 block 32, 1024x512 fp32")
    codes, scales = W.quantize_mxfp4(dev_f32(Wf), 32)
    wc, ws = OM.quantize_mxfp4(Wf, 32)
    assert np.array_equal(host_u8(scales), ws)
    assert np.array_equal(host_u8(codes), wc)


@pytest.mark.parametrize("block", [16, 32])
@pytest.mark.parametrize("bf16", [False, True])
def test_mxfp4_wide_values(W, block, bf16):
    a = _wide((29, 512), seed=7 + block, zero_blocks=4, block=block)
    if bf16:
        bits = to_bf16_bits(a)
        x, ref_in = dev_bf16(bits), bf16_bits_to_f32(bits)
    else:
        x, ref_in = dev_f32(a), a
    banner("mxfp4", block, "bf16" if bf16 else "fp32", a.shape)
    codes, scales = W.quantize_mxfp4(x, block)
    wc, ws = OM.quantize_mxfp4(ref_in, block)
    assert np.array_equal(host_u8(scales), ws)
    assert np.array_equal(host_u8(codes), wc)


def test_mxfp4_all_bf16_patterns_as_blocks(W):
    # every finite bf16 value appears, blocks of 32 consecutive patterns
    bits = all_bf16_patterns()
    x = bf16_bits_to_f32(bits)
    bits = bits[np.isfinite(x)]
    bits = bits[: bits.size // 512 * 512].reshape(-1, 512)
    banner("mxfp4 block 32/16 over finite bf16 patterns", bits.shape)
    for block in (32, 16):
        codes, scales = W.quantize_mxfp4(dev_bf16(bits), block)
        wc, ws = OM.quantize_mxfp4(bf16_bits_to_f32(bits), block)
        assert np.array_equal(host_u8(scales), ws)
        assert np.array_equal(host_u8(codes), wc)


def test_mxfp4_block16_activation_full_size(W):
    bits = act_quant_inputs(0)
    banner("mxfp4 block 16, 4096x7168 bf16")
    codes, scales = W.quantize_mxfp4(dev_bf16(bits), 16)
    wc, ws = OM.quantize_mxfp4(bf16_bits_to_f32(bits), 16)
    assert np.array_equal(host_u8(scales), ws)
    assert np.array_equal(host_u8(codes), wc)


def test_mxfp4_prefill_weights_full_size(W):
    _, Wf = prefill_inputs(0, with_x=False)
    banner("mxfp4 block 32, 14336x4096 fp32")
    codes, scales = W.quantize_mxfp4(dev_f32(Wf), 32)
    wc, ws = OM.quantize_mxfp4(Wf, 32)
    assert np.array_equal(host_u8(scales), ws)
    assert np.array_equal(host_u8(codes), wc)


# ---------------------------------------------------------------------------
# INT4
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("bf16", [False, True])
def test_int4_groups(W, group, bf16):
    a = _wide((23, 768), seed=group + 3 * bf16, zero_blocks=3, block=group)
    a[0, :group] = 0.0
    if bf16:
        bits = to_bf16_bits(a)
        x, ref_in = dev_bf16(bits), bf16_bits_to_f32(bits)
    else:
        x, ref_in = dev_f32(a), a
    banner("int4", group, "bf16" if bf16 else "fp32", a.shape)
    packed, scales = W.quantize_int4(x, group)
    wp, ws, _ = OI.quantize_int4(ref_in, group)
    assert np.array_equal(host_bits16(scales), ws)
    assert np.array_equal(host_words(packed), wp)


def test_int4_decode_weights_full_size(W):
    _, Wf = decode_inputs(1, 0)
    banner("int4 group 128, 14336x4096 fp32")
    packed, scales = W.quantize_int4(dev_f32(Wf), 128)
    wp, ws, _ = OI.quantize_int4(Wf, 128)
    assert np.array_equal(host_bits16(scales), ws)
    assert np.array_equal(host_words(packed), wp)


def test_e4m3_per_channel_weights_full_size(W):
    _, Wf = decode_inputs(1, 0)
    banner("e4m3 per-channel, 14336x4096 fp32")
    codes, scales = W.quantize_e4m3(dev_f32(Wf), -1)
    wc, ws = OE.quantize_e4m3(Wf, -1)
    assert np.array_equal(host_f32(scales).view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(host_u8(codes), wc)


# ---------------------------------------------------------------------------
# Dequantization (the matmul operand) -- every code
# ---------------------------------------------------------------------------

def test_dequant_e2m1_every_code_and_scale(W):
    # rows: scale code 0..254; each row holds all 256 byte patterns (512 codes)
    codes = np.tile(np.arange(256, dtype=np.uint8), (255, 1))
    scales = np.repeat(np.arange(255, dtype=np.uint8)[:, None], 512 // 32, axis=1)
    banner("dequant e2m1 x e8m0, all codes")
    out = W.wq_dequant(dev_u8(codes), W.WQ_E2M1X2, dev_u8(scales), W.WQ_E8M0, 32, 255, 512)
    assert np.array_equal(host_bits16(out), OD.dequant_mxfp4(codes, scales, 32))
    out16 = W.wq_dequant(dev_u8(codes), W.WQ_E2M1X2, dev_u8(np.repeat(scales, 2, axis=1)), W.WQ_E8M0, 16, 255, 512)
    assert np.array_equal(host_bits16(out16), OD.dequant_mxfp4(codes, np.repeat(scales, 2, axis=1), 16))


def test_dequant_e4m3_every_code(W):
    codes = np.tile(np.arange(256, dtype=np.uint8), (4, 1))
    banner("dequant e4m3, all codes")
    out = W.wq_dequant(dev_u8(codes), W.WQ_E4M3, None, W.WQ_F32, 256, 4, 256)
    got, want = host_bits16(out), OD.dequant_e4m3(codes)
    gv, wv = bf16_decode(got), bf16_decode(want)
    assert np.array_equal(np.isnan(gv), np.isnan(wv))
    assert np.array_equal(got[~np.isnan(wv)], want[~np.isnan(wv)])


def test_dequant_int4_every_code_and_scale(W):
    s = all_bf16_patterns()
    s = s[np.isfinite(bf16_decode(s))]
    s = s[: s.size // 2 * 2]
    N = s.size // 2
    q = np.tile(np.arange(-8, 8, dtype=np.int8), (N, 4))          # 64 per row: 2 groups of 32
    packed = OI.pack_int4(q)
    sc = s.reshape(N, 2)
    banner("dequant int4 x every finite bf16 scale", N)
    out = W.wq_dequant(dev_words(packed), W.WQ_INT4X8, dev_bf16(sc), W.WQ_BF16, 32, N, 64)
    assert np.array_equal(host_bits16(out), OD.dequant_int4(packed, sc, 32))
    for group in (64, 128):
        g = np.random.default_rng(group)
        qq = g.integers(-8, 8, (64, 512)).astype(np.int8)
        ss = to_bf16_bits((g.uniform(0.5, 2, (64, 512 // group)) * 0.01).astype(np.float32))
        pk = OI.pack_int4(qq)
        out = W.wq_dequant(dev_words(pk), W.WQ_INT4X8, dev_bf16(ss), W.WQ_BF16, group, 64, 512)
        assert np.array_equal(host_bits16(out), OD.dequant_int4(pk, ss, group))


# ---------------------------------------------------------------------------
# seeded random shapes: every quantizer, codes and scales bit for bit
# ---------------------------------------------------------------------------
def _random_quant_cases(n, seed=2029):
    g = np.random.default_rng(seed)
    kinds = [("e4m3", 16), ("e4m3", 64), ("e4m3", 128), ("e4m3", 256), ("e4m3", -1),
             ("mxfp4", 16), ("mxfp4", 32), ("int4", 32), ("int4", 64), ("int4", 128)]
    out = []
    for i in range(n):
        kind, block = kinds[i % len(kinds)]
        unit = 128 if block == -1 else 32 if kind == "mxfp4" else block      # MXFP4: cols % 32 (either block)
        out.append((kind, block, int(g.integers(1, 301)), unit * int(g.integers(1, 65)), bool(i % 2),
                    int(g.integers(1 << 30))))
    return out


@pytest.mark.parametrize("kind,block,rows,cols,bf16,seed", _random_quant_cases(30))
def test_quantizers_random_shapes(W, kind, block, rows, cols, bf16, seed):
    a = _wide((rows, cols), seed=seed, zero_blocks=2, block=128 if block == -1 else block)
    if bf16:
        bits = to_bf16_bits(a)
        x, ref_in = dev_bf16(bits), bf16_bits_to_f32(bits)
    else:
        x, ref_in = dev_f32(a), a
    banner("quantizer random shape", kind, block, rows, cols, "bf16" if bf16 else "fp32")
    if kind == "e4m3":
        codes, scales = W.quantize_e4m3(x, block)
        wc, ws = OE.quantize_e4m3(ref_in, block)
        assert np.array_equal(host_f32(scales).view(np.uint32), ws.view(np.uint32))
        assert np.array_equal(host_u8(codes), wc)
    elif kind == "mxfp4":
        codes, scales = W.quantize_mxfp4(x, block)
        wc, ws = OM.quantize_mxfp4(ref_in, block)
        assert np.array_equal(host_u8(scales), ws)
        assert np.array_equal(host_u8(codes), wc)
    else:
        packed, scales = W.quantize_int4(x, block)
        wp, ws, _ = OI.quantize_int4(ref_in, block)
        assert np.array_equal(host_bits16(scales), ws)
        assert np.array_equal(host_words(packed), wp)
