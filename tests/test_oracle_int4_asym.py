"""Pins of the asymmetric INT4 oracle (x = s * (q - z), unsigned codes) on the CPU."""
import numpy as np
import pytest
import torch

from oracle import int4_asym as A
from oracle.formats import bf16_decode


def _data(seed, rows=24, cols=512, shift=0.0):
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, cols)) * np.exp2(g.integers(-10, 10, (rows, 1)))
    return (x + shift * np.abs(x).max(axis=1, keepdims=True)).astype(np.float32)


@pytest.mark.parametrize("group", [32, 64, 128])
def test_integer_grids_are_exact(group):
    # a group holding k - c for k = 0..15 has s = 1 (times a power of two),
    # z = c and q = k: the reconstruction is exact
    rows = []
    for c in range(16):
        for j in (-3, 0, 5):
            k = np.resize(np.arange(16), group)
            rows.append(((k - c) * 2.0 ** j).astype(np.float32))
    x = np.stack(rows)
    packed, sb, z = A.quantize_int4_asym(x, group)
    q = A.unpack_uint4(packed)
    assert np.array_equal(q, np.stack([np.resize(np.arange(16), group)] * len(rows)))
    assert np.array_equal(z[:, 0], np.repeat(np.arange(16), 3))
    assert np.array_equal(bf16_decode(sb[:, 0]), np.tile(2.0 ** np.array([-3, 0, 5]), 16))
    assert np.array_equal(bf16_decode(A.dequant_int4_asym(packed, sb, z, group)), x.astype(np.float64))


@pytest.mark.parametrize("shift", [0.0, 0.7, -0.9, 3.0])
def test_reconstruction_bound(shift):
    x = _data(1, shift=shift)
    for group in (32, 128):
        packed, sb, z = A.quantize_int4_asym(x, group)
        q = A.unpack_uint4(packed).reshape(x.shape[0], -1, group)
        s = bf16_decode(sb)[..., None]
        rec = (q - z[..., None].astype(np.int64)) * s
        err = np.abs(rec - x.reshape(q.shape))
        inner = (q > 0) & (q < 15)
        assert np.all(err[inner] <= 0.5 * np.broadcast_to(s, q.shape)[inner] * (1 + 2.0 ** -20))
        # the range ends may clamp by the bf16 rounding of s: still within 0.55 s
        assert np.all(err <= 0.55 * s)
        assert np.all(z <= 15)


def test_codes_are_the_nearest_grid_points():
    # brute force over all 16 codes on the fp32 quotient, ties to an even q - z
    x = _data(2, rows=6, cols=128, shift=0.3)
    packed, sb, z = A.quantize_int4_asym(x, 32)
    q = A.unpack_uint4(packed).reshape(6, 4, 32)
    s = bf16_decode(sb).astype(np.float32)[..., None]
    v = (x.reshape(6, 4, 32) / s).astype(np.float32).astype(np.float64) + z[..., None]
    c = np.arange(16)
    d = np.abs(v[..., None] - c)
    best = d.min(axis=-1, keepdims=True)
    ties = d == best
    even = ties & (((c - z[..., None, None]) % 2) == 0)
    pick = np.where(even.any(-1), even.argmax(-1), ties.argmax(-1))
    assert np.array_equal(q, pick)


def test_zero_point_placement():
    g = np.random.default_rng(3)
    a = np.abs(g.standard_normal((40, 64))).astype(np.float32) + 0.1
    pos, neg = a, -a
    sym = np.concatenate([a[:, :32], -a[:, :32]], axis=1)
    sym[:, 32:] = -sym[:, :32]                                          # lo = -hi exactly
    _, _, zp = A.quantize_int4_asym(pos, 32)
    _, _, zn = A.quantize_int4_asym(neg, 32)
    _, _, zs = A.quantize_int4_asym(sym, 64)
    assert np.all(zp == 0) and np.all(zn == 15)
    assert set(np.unique(zs)) <= {7, 8}


def test_zero_is_exact_and_all_zero_groups():
    x = _data(4, shift=0.2)
    x[:, 5] = 0.0
    x[3, :128] = 0.0
    packed, sb, z = A.quantize_int4_asym(x, 128)
    deq = bf16_decode(A.dequant_int4_asym(packed, sb, z, 128))
    assert np.all(deq[:, 5] == 0.0)
    assert sb[3, 0] == 0x3F80 and z[3, 0] == 0 and np.all(deq[3, :128] == 0.0)


def test_dequant_matches_torch_cast():
    x = _data(5, shift=-0.4)
    packed, sb, z = A.quantize_int4_asym(x, 64)
    q = torch.from_numpy(A.unpack_uint4(packed).astype(np.float32))
    s = torch.from_numpy(bf16_decode(sb).astype(np.float32)).repeat_interleave(64, dim=1)
    zz = torch.from_numpy(z.astype(np.float32)).repeat_interleave(64, dim=1)
    want = ((q - zz) * s).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(A.dequant_int4_asym(packed, sb, z, 64), want)


def test_invalid_inputs():
    x = np.zeros((2, 64), np.float32)
    with pytest.raises(ValueError):
        A.quantize_int4_asym(x, 48)
    x[0, 0] = np.nan
    with pytest.raises(ValueError):
        A.quantize_int4_asym(x, 32)
    y = np.zeros((1, 32), np.float32)
    y[0, 0], y[0, 1] = 3e38, -3e38
    with pytest.raises(ValueError):
        A.quantize_int4_asym(y, 32)
