"""Number-format algebra and decode/encode tables.

Follows "Numerics: FP32 to INT4, and why bf16 won": the paragraph on the
exponent/mantissa split (bias B = 2^(e-1) - 1, smallest normal 2^(1-B),
epsilon 2^-m), the paragraph on the two formats that break the IEEE rules
(E4M3 "fn" reuses the all-ones exponent and burns only mantissa 111 for NaN;
E2M1 has neither infinity nor NaN), the printed maxima of the scalar-type
registry, and "MXFP4 and the block-scaled family" (the E2M1 value list and the
E8M0 scale as a bare power of two).

The max-finite formula itself is missing from the extracted page; the reading
used here is the IEEE closed form, (2 - 2^-m) * 2^(2^e - 2 - B), with the
extended-range variant for formats that use the all-ones exponent.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------


def exponent_bias(e: int) -> int:
    return 2 ** (e - 1) - 1


def max_finite_ieee(e: int, m: int) -> float:
    """IEEE layout: all-ones exponent reserved, so the top finite binade has
    unbiased exponent 2^e - 2 - B and significand 2 - 2^-m."""
    B = exponent_bias(e)
    return (2.0 - 2.0 ** -m) * 2.0 ** (2 ** e - 2 - B)


def max_finite_extended(e: int, m: int, nan_mantissas: int) -> float:
    """Extended range: the all-ones exponent holds finite values; the top
    `nan_mantissas` mantissa patterns of that binade are NaN (1 for E4M3 "fn",
    0 for E2M1)."""
    B = exponent_bias(e)
    top = 2 ** m - 1 - nan_mantissas
    return (1.0 + top / 2 ** m) * 2.0 ** (2 ** e - 1 - B)


def min_normal(e: int) -> float:
    return 2.0 ** (1 - exponent_bias(e))


def min_subnormal(e: int, m: int) -> float:
    return 2.0 ** (1 - exponent_bias(e) - m)


def epsilon(m: int) -> float:
    return 2.0 ** -m


def int_range(bits: int) -> tuple[int, int]:
    """Two's-complement range of a signed integer of `bits` bits."""
    return -(2 ** (bits - 1)), 2 ** (bits - 1) - 1


# ---------------------------------------------------------------------------
# Decoders (code -> exact value as fp64; NaN where the format says NaN)
# ---------------------------------------------------------------------------


def e4m3_decode(codes) -> np.ndarray:
    """OCP E4M3 "fn": sign | 4-bit exponent (bias 7) | 3-bit mantissa.
    Exponent field 0 is subnormal (M/8 * 2^-6); 0x7F/0xFF are NaN; no inf."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = (c & 0x7).astype(np.float64)
    mag = np.where(E == 0, M / 8.0 * 2.0 ** -6, (1.0 + M / 8.0) * np.exp2(E.astype(np.float64) - 7.0))
    v = s * mag
    return np.where((E == 15) & ((c & 7) == 7), np.nan, v)


def e2m1_decode(codes) -> np.ndarray:
    """FP4 E2M1: sign | 2-bit exponent (bias 1) | 1-bit mantissa; every code
    finite.  Exponent field 0 is subnormal (M/2)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    s = np.where(c & 0x8, -1.0, 1.0)
    E = (c >> 1) & 0x3
    M = (c & 0x1).astype(np.float64)
    mag = np.where(E == 0, M / 2.0, (1.0 + M / 2.0) * np.exp2(E.astype(np.float64) - 1.0))
    return s * mag


def e8m0_decode(codes) -> np.ndarray:
    """E8M0 (unsigned exponent only, bias 127): 2^(c-127); 0xFF is NaN."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2(c.astype(np.float64) - 127.0))


def bf16_decode(bits) -> np.ndarray:
    """bf16 is the upper half of an fp32 pattern; widening is exact."""
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# Value grids ---------------------------------------------------------------

E2M1_GRID = e2m1_decode(np.arange(8))          # non-negative E2M1 magnitudes
E4M3_POS_CODES = np.array([c for c in range(0x7F)], dtype=np.int64)  # 0x00..0x7E, all finite
E4M3_POS_VALUES = e4m3_decode(E4M3_POS_CODES)
E4M3_MAX = float(E4M3_POS_VALUES.max())
E2M1_MAX = float(E2M1_GRID.max())


# ---------------------------------------------------------------------------
# bf16 encoder: nearest bf16 value, ties to even significand.
# ---------------------------------------------------------------------------


def bf16_round(values) -> np.ndarray:
    """Round fp64 values to bf16 (8 significant bits, exponent range of fp32),
    round to nearest with ties to even, overflow to +-inf, and return bit
    patterns (uint16).  NaN becomes the quiet NaN 0x7FC0 with the input's sign.

    Arithmetic derivation: for |v| >= 2^-126 the spacing in the binade
    [2^E, 2^(E+1)) is 2^(E-7); below it (subnormals) the spacing is 2^-133.
    The rounded value is rint(|v| / spacing) * spacing (exact in fp64), which is
    a bf16 value; its bit pattern is the upper half of its fp32 pattern."""
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    neg = np.signbit(v)
    nan = np.isnan(v)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        _, ex = np.frexp(np.where(np.isfinite(a) & (a > 0), a, 1.0))
        E = ex.astype(np.int64) - 1                      # a in [2^E, 2^(E+1))
        E = np.maximum(E, -126)                          # subnormal spacing
        spacing = np.exp2((E - 7).astype(np.float64))
        r = np.rint(a / spacing) * spacing
        r = np.where(np.isfinite(a), r, a)
    over = r >= 2.0 ** 128
    out = np.where(over, np.inf, r)
    f32 = out.astype(np.float32)                         # exact: out is a bf16 value or inf
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(neg, bits | np.uint16(0x8000), bits)
    bits = np.where(nan, np.where(neg, np.uint16(0xFFC0), np.uint16(0x7FC0)), bits)
    return bits.astype(np.uint16)


def f32_bits(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)


def f32_from_bits(b) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(b, dtype=np.uint32)).view(np.float32)
