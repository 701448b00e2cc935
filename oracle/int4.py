"""Symmetric INT4 group quantizer with bf16 group scales (weight preparation).

Follows "Numerics: FP32 to INT4, and why bf16 won": the affine map
x = s * (q - z) with z = 0 for symmetric quantization, the scale policy
s = max|x| / qmax with an all-zero-group policy s = 1, the int4 range
[-8, 7] of the scalar-type registry, and (section "The tie back to the
roofline") group size 128 along K with a 16-bit scale per group.

Readings where the pages are silent:
* qmax = 7 (the largest positive code), so a symmetric group never needs -8;
* the scale is stored as a bf16 value whose significand has at most 5
  significant bits: s = RN_5(RN_f32(amax / 7)), the fp32 quotient rounded to
  the nearest multiple of 2^(e-4) (e its binary exponent; 2^-130 below the
  normal range), ties to even.  The pages fix the scale as amax / qmax and the
  dequantized weight as (q - z) * s cast to the element type, but not the
  precision of the stored scale; with a 5-bit significand every product q * s
  (|q| <= 8) has at most 8 significant bits, so the cast to bf16 is exact and
  the dequantized weight equals q * s.  The group is quantized with the stored
  scale, so that dequantization is self-consistent; a scale that is zero
  after the rounding (including the all-zero group) is replaced by 1.  The
  rounding moves the scale by at most 2^-5 of itself, so amax / s stays in
  [6.79, 7.23] and the largest element of a group always gets |q| = 7;
* q = clamp(rint(RN_f32(x / s)), -8, 7): an IEEE fp32 division, then round
  half to even;
* packing: eight two's-complement nibbles per uint32, element 8i + j in bits
  4j..4j+3 (parity unpinned: the pages only say eight values share an int32).
Parity beyond the range and the bits-per-weight overhead is unpinned; the
self-consistency bound |x - q*s| <= s/2 (unless clamped) is tested.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_decode, bf16_round


def round_significand5(v) -> np.ndarray:
    """Nearest value with a 5-bit significand (multiples of 2^(e-4) in the
    binade [2^e, 2^(e+1)), of 2^-130 below 2^-126), ties to even; fp64 in and
    out (every such value and every fp32 input is exact in fp64)."""
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(v)                                                   # v = m 2^ex, m in [0.5, 1)
    ulp = np.maximum(np.ldexp(1.0, ex - 5), 2.0 ** -130)
    return np.rint(v / ulp) * ulp                                         # v / ulp exact: power-of-two ulp


def int4_scale_bits(amax_f32) -> np.ndarray:
    s32 = np.asarray(amax_f32, dtype=np.float32) / np.float32(7.0)       # IEEE fp32
    bits = bf16_round(round_significand5(s32.astype(np.float64)))        # exact: 5 significant bits
    return np.where(bf16_decode(bits) == 0, np.uint16(0x3F80), bits).astype(np.uint16)


def quantize_int4(w, group: int):
    """w: N x K fp32.  Returns (packed uint32 N x K/8, scale bits uint16
    N x K/group, q int8 N x K)."""
    w32 = np.ascontiguousarray(np.asarray(w, dtype=np.float32))
    if w32.ndim != 2:
        raise ValueError("expected a 2-D array")
    N, K = w32.shape
    if group <= 0 or K % group or K % 8:
        raise ValueError("K must be a multiple of the group size and of 8")
    if not np.isfinite(w32).all():
        raise ValueError("non-finite weight")
    g = w32.reshape(N, K // group, group)
    amax = np.abs(g).max(axis=2)
    sbits = int4_scale_bits(amax)
    s32 = bf16_decode(sbits).astype(np.float32)
    r = g / s32[:, :, None]                                              # IEEE fp32
    q = np.clip(np.rint(r.astype(np.float64)), -8, 7).astype(np.int8).reshape(N, K)
    return pack_int4(q), sbits, q


def pack_int4(q: np.ndarray) -> np.ndarray:
    q = np.asarray(q, dtype=np.int8)
    N, K = q.shape
    nib = (q.astype(np.int64) & 0xF).reshape(N, K // 8, 8)
    shifts = (4 * np.arange(8)).astype(np.int64)
    return (nib << shifts).sum(axis=2).astype(np.uint32)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint32).astype(np.int64)
    N, W = p.shape
    nib = (p[:, :, None] >> (4 * np.arange(8))[None, None, :]) & 0xF
    q = np.where(nib >= 8, nib - 16, nib)
    return q.reshape(N, W * 8).astype(np.int8)
