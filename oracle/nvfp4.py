"""NVFP4: E2M1 element codes in blocks of 16 sharing an E4M3 scale.

Follows "Numerics: FP32 to INT4, and why bf16 won", section "MXFP4 and the
block-scaled family" (NVFP4 uses blocks of 16 and stores the block scale in
FP8 E4M3 instead of E8M0, so the scale carries mantissa bits and need not be a
power of two), "Your 3090 Isn't Missing Anything for FP8/NVFP4 Weight-Only
Inference", section 2.1 (the weight-only kernels decode each 16-value E2M1
block with its E4M3 scale to bf16 and multiply in bf16 with fp32
accumulation), and the review note on vLLM PR #43557 (the elements must be
divided by the dequantized scale, not by the unrounded one).

Quantizer, per 1 x 16 block of x with a per-tensor fp32 scale g > 0:
  s   = RN_f32(RN_f32(amax / 6) / g)         the block scale in units of g
  s8  = e4m3(s)                               RNE, saturating at 448
  d   = RN_f32(e4m3_value(s8) * g)            the dequantized scale
  v   = RN_f32(x / d), or a zero of x's sign when d == 0
  code = e2m1(v)                              nearest, ties to even, saturating at 6
Dequantized weight: g * e4m3_value(s8) * e2m1_value(code).  The matmul
operand is the exact product e2m1_value * e4m3_value (every such product is a
bf16 number); g multiplies the fp32 accumulator.

Readings where the pages are silent:
* the per-tensor scale g is not on the pages (the format as deployed has one);
  it is a caller-supplied fp32 value, and g = 1 gives exactly the pages'
  description (block scale amax / 6 in E4M3);
* ties and saturation of the element step are those of the MXFP4 quantizer;
* packing: element 2j in the low nibble of byte j, as MXFP4.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import e4m3_from_f32
from .e8m0 import block_absmax
from .formats import bf16_round, e2m1_decode, e4m3_decode, f32_bits
from .mxfp4 import e2m1_from_f64, pack_nibbles, unpack_nibbles

BLOCK = 16


def block_scale(amax_f32, g: float = 1.0):
    """E4M3 code of each block's scale and the dequantized scale d (fp32)."""
    g32 = np.float32(g)
    if not (np.isfinite(g32) and g32 > 0):
        raise ValueError("tensor scale must be finite and positive")
    a = np.asarray(amax_f32, dtype=np.float32)
    if not np.isfinite(a).all():
        raise ValueError("non-finite block maximum")
    with np.errstate(under="ignore", over="ignore"):      # fp32 overflow saturates the scale
        s = ((a / np.float32(6.0)).astype(np.float32) / g32).astype(np.float32)
        s8 = e4m3_from_f32(s)
        d = (e4m3_decode(s8).astype(np.float32) * g32).astype(np.float32)
    return s8, d


def quantize_nvfp4(x, g: float = 1.0):
    """x: rows x cols fp32, cols % 16 == 0.  Returns (packed E2M1 codes uint8
    rows x cols/2, E4M3 scale codes uint8 rows x cols/16)."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if x32.ndim != 2:
        raise ValueError("expected a 2-D array")
    rows, cols = x32.shape
    s8, d = block_scale(block_absmax(x32, BLOCK), g)
    xb = x32.reshape(rows, cols // BLOCK, BLOCK)
    dd = np.broadcast_to(d[:, :, None], xb.shape)
    with np.errstate(divide="ignore", invalid="ignore", under="ignore", over="ignore"):
        v = np.where(dd > 0, (xb / np.where(dd > 0, dd, np.float32(1))).astype(np.float32), np.float32(0))
    sign = (f32_bits(xb) >> 31).astype(np.uint8)
    codes = e2m1_from_f64(v.astype(np.float64), sign).reshape(rows, cols)
    return pack_nibbles(codes), s8


def operand_values(packed, s8) -> np.ndarray:
    """Exact fp64 values e2m1_value * e4m3_value of the matmul operand."""
    codes = unpack_nibbles(packed)
    rows, cols = codes.shape
    e = e2m1_decode(codes).reshape(rows, cols // BLOCK, BLOCK)
    s = e4m3_decode(np.asarray(s8, np.uint8)).astype(np.float64)
    return (e * s[:, :, None]).reshape(rows, cols)


def dequant_nvfp4(packed, s8) -> np.ndarray:
    """bf16 bit patterns of the operand (each value is a bf16 number, so the
    rounding is exact)."""
    return bf16_round(operand_values(packed, s8))
