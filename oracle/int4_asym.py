"""Asymmetric (affine) INT4: x = s * (q - z) with unsigned 4-bit codes q, a
bf16 group scale s and an integer zero-point z per group along K.

Follows "Numerics: FP32 to INT4, and why bf16 won": the affine map from an
integer code back to the reals with a float scale and an integer zero-point
(z = 0 is the symmetric case, z != 0 represents a range not centred on zero
at the cost of one subtraction in the dequantization), the dequantization
step (q - z) * s followed by a cast to the element type, the remark that
asymmetric quantization also computes a zero point, and the all-zero-group
policy s = 1; section "Granularity" for the groups of 128 or 64 along K.

Readings where the pages are silent:
* codes are the unsigned 4-bit range [0, 15] and z is an integer in [0, 15];
* the quantizer is min-max over a range that contains 0 (so that 0 stays
  exactly representable and z needs no clamping): lo = min(min x, 0),
  hi = max(max x, 0) over the group, s = bf16(RN_f32(RN_f32(hi - lo) / 15)),
  replaced by 1 when it is zero;
  z = clamp(rint(RN_f32(-lo / s)), 0, 15); q = clamp(rint(RN_f32(x / s)) + z, 0, 15)
  (rint rounds half to even);
* the matmul operand is bf16((q - z) * s), one rounding of the exact product;
* a group whose range hi - lo overflows fp32 is outside the contract.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_decode, bf16_round
from .int4 import pack_int4, unpack_int4


def _groups(x32: np.ndarray, group: int) -> np.ndarray:
    rows, cols = x32.shape
    if group <= 0 or cols % group:
        raise ValueError("cols must be a multiple of the group size")
    return x32.reshape(rows, cols // group, group)


def scale_zero(lo_f32, hi_f32):
    """bf16 scale bits and zero-points of groups with minimum lo and maximum hi."""
    lo = np.asarray(lo_f32, np.float32)
    hi = np.asarray(hi_f32, np.float32)
    if not (np.isfinite(lo).all() and np.isfinite(hi).all()):
        raise ValueError("non-finite group")
    with np.errstate(over="ignore"):
        rng = (hi - lo).astype(np.float32)
    if not np.isfinite(rng).all():
        raise ValueError("group range overflows fp32")
    s32 = (rng / np.float32(15.0)).astype(np.float32)
    sb = bf16_round(s32.astype(np.float64))
    sb = np.where(bf16_decode(sb) == 0, np.uint16(0x3F80), sb)        # s = 1
    s = bf16_decode(sb).astype(np.float32)
    with np.errstate(over="ignore"):
        zf = np.rint((-lo / s).astype(np.float32).astype(np.float64))
    z = np.clip(zf, 0, 15).astype(np.uint8)
    return sb.astype(np.uint16), z


def quantize_int4_asym(w, group: int):
    """w: rows x cols fp32.  Returns (packed uint32 rows x cols/8 holding the
    codes in the INT4X8 nibble order, bf16 scale bits rows x cols/group,
    zero-points uint8 rows x cols/group)."""
    x32 = np.ascontiguousarray(np.asarray(w, dtype=np.float32))
    if x32.ndim != 2:
        raise ValueError("expected a 2-D array")
    if not np.isfinite(x32).all():
        raise ValueError("non-finite input")
    g = _groups(x32, group)
    sb, z = scale_zero(np.minimum(g.min(axis=2), 0), np.maximum(g.max(axis=2), 0))
    s = bf16_decode(sb).astype(np.float32)[:, :, None]
    with np.errstate(over="ignore"):
        v = np.rint((g / s).astype(np.float32).astype(np.float64))
    q = np.clip(v + z[:, :, None], 0, 15).astype(np.int8).reshape(x32.shape)
    return pack_int4(q), sb, z          # the low 4 bits of each code, INT4X8 order


def unpack_uint4(packed) -> np.ndarray:
    """uint32 words -> unsigned codes 0..15, rows x cols."""
    return (unpack_int4(packed).astype(np.int64) & 0xF).astype(np.int64)


def dequant_int4_asym(packed, scale_bits, zeros, group: int) -> np.ndarray:
    """bf16 bit patterns of bf16((q - z) * s)."""
    q = unpack_uint4(packed)
    N, K = q.shape
    s = bf16_decode(scale_bits)[:, :, None]
    z = np.asarray(zeros, np.int64)[:, :, None]
    d = (q.reshape(N, K // group, group) - z).astype(np.float64) * s
    return bf16_round(d.reshape(N, K))
