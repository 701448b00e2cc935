"""Pins of the oracle's number-format algebra (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import formats as F
from tests.conftest import golden_rows


def test_printed_maxima():
    for row in golden_rows("format_maxima.txt"):
        name, e, m, layout, mx, mn = row
        if layout == "int":
            bits = int(name[3:])
            assert F.int_range(bits) == (int(mn), int(mx))
        elif layout == "fn":
            assert F.max_finite_extended(int(e), int(m), nan_mantissas=1) == float(mx)
        else:
            assert F.max_finite_ieee(int(e), int(m)) == float(mx)


def test_e4m3_closed_form_448():
    # (1 + 6/8) * 2^(15 - 7)
    assert F.max_finite_extended(4, 3, 1) == (1 + 6 / 8) * 2.0 ** 8 == 448.0


def test_closed_forms_agree_with_library_finfo():
    assert F.max_finite_ieee(5, 10) == float(np.finfo(np.float16).max)
    assert F.min_normal(5) == float(np.finfo(np.float16).tiny)
    assert F.epsilon(10) == float(np.finfo(np.float16).eps)
    assert F.max_finite_ieee(8, 23) == float(np.finfo(np.float32).max)
    assert F.min_normal(8) == float(np.finfo(np.float32).tiny)
    assert F.min_subnormal(8, 23) == float(np.finfo(np.float32).smallest_subnormal)
    assert F.max_finite_ieee(8, 7) == float(torch.finfo(torch.bfloat16).max)
    assert F.epsilon(7) == float(torch.finfo(torch.bfloat16).eps)
    assert F.max_finite_extended(4, 3, 1) == float(torch.finfo(torch.float8_e4m3fn).max)
    assert F.min_normal(4) == float(torch.finfo(torch.float8_e4m3fn).tiny)
    assert F.max_finite_ieee(5, 2) == float(torch.finfo(torch.float8_e5m2).max)


def test_e4m3_min_subnormal_is_2_pow_minus_9():
    assert F.min_subnormal(4, 3) == 2.0 ** -9
    assert abs(F.min_subnormal(4, 3) - 0.00195) < 1e-5


def test_e2m1_grid_and_max():
    rows = {r[0]: r[1:] for r in golden_rows("e2m1_grid.txt")}
    grid = [float(v) for v in rows["values"]]
    assert list(F.E2M1_GRID) == grid
    assert F.max_finite_extended(2, 1, nan_mantissas=0) == float(rows["max"][0]) == F.E2M1_MAX
    # bounds are the midpoints of adjacent magnitudes
    mids = [(a + b) / 2 for a, b in zip(grid[:-1], grid[1:])]
    assert mids == [float(v) for v in rows["bounds"]]
    assert 4 + 8 / 32 == float(rows["bits_per_element"][0])
    # sign bit gives the negative half, all 16 codes finite
    full = F.e2m1_decode(np.arange(16))
    assert np.isfinite(full).all()
    assert list(-full[8:]) == grid


def test_e4m3_table_against_torch_decode():
    codes = np.arange(256, dtype=np.uint8)
    mine = F.e4m3_decode(codes)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    ok = ~np.isnan(mine)
    assert np.array_equal(mine[ok], lib[ok])
    # NaN only at 0x7F / 0xFF; max finite matches the closed form; min normal 2^-6
    assert list(np.where(np.isnan(mine))[0]) == [0x7F, 0xFF]
    assert np.nanmax(mine) == F.max_finite_extended(4, 3, 1)
    assert mine[0x08] == F.min_normal(4)


def test_e5m2_decode_via_library_matches_closed_form():
    # the IEEE closed form also fixes e5m2; decode its largest finite code via torch
    assert torch.tensor([0x7B], dtype=torch.uint8).view(torch.float8_e5m2).float().item() == F.max_finite_ieee(5, 2)


def test_e8m0_decode():
    c = np.arange(256)
    v = F.e8m0_decode(c)
    assert np.isnan(v[255])
    assert v[127] == 1.0 and v[0] == 2.0 ** -127 and v[254] == 2.0 ** 127
    assert np.all(np.diff(v[:255]) > 0)


def _bf16_sweep():
    g = np.random.default_rng(7)
    vals = [g.standard_normal(200000).astype(np.float32),
            (g.standard_normal(100000) * 1e-38).astype(np.float32),
            (g.standard_normal(50000) * 3e38).astype(np.float32),
            np.array([0.0, -0.0, np.inf, -np.inf, 3.3961e38, 3.3895313892515355e38, 1e-45, -1e-45], np.float32)]
    # exact midpoints between consecutive bf16 values and their fp32 neighbours
    b = np.arange(0, 0x7F80, 97, dtype=np.uint32)
    lo = (b << 16).view(np.float32).astype(np.float64)
    hi = ((b + 1) << 16).view(np.float32).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    vals += [mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0)), -mid]
    return np.concatenate(vals)


def test_bf16_round_matches_torch_cast():
    x = _bf16_sweep()
    mine = F.bf16_round(x.astype(np.float64))
    lib = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, lib)


def test_bf16_round_bruteforce_small():
    # every bf16 value in a narrow window, and points between them: nearest, ties even
    base = np.arange(0x3F70, 0x3F90, dtype=np.uint32)
    vals = (base << 16).view(np.float32).astype(np.float64)
    probe = np.linspace(vals[0], vals[-1], 4001)
    probe = np.concatenate([probe, (vals[:-1] + vals[1:]) / 2])
    d = np.abs(probe[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    ties = d == best
    even = ties & ((base[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), ties.argmax(axis=1))
    assert np.array_equal(F.bf16_round(probe), base[pick].astype(np.uint16))


def test_bf16_relative_error_bound():
    # a normal bf16 rounding is within 2^-8 relative error
    g = np.random.default_rng(3)
    x = g.standard_normal(100000) * np.exp2(g.integers(-100, 100, 100000))
    r = F.bf16_decode(F.bf16_round(x))
    assert np.max(np.abs(r - x) / np.abs(x)) <= 2.0 ** -8
