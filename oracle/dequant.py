"""Packed weights + scales -> the bf16 operand that the matmul consumes.

Follows "Your 3090 Isn't Missing Anything for FP8/NVFP4 Weight-Only
Inference", section "4.1 The Marlin implementation" (weights are converted to
bf16 for a bf16 x bf16 multiply; every E4M3 and E2M1 value is exactly
representable in bf16, so those conversions never round) and the integer
dequantization step quoted in "Numerics: FP32 to INT4, and why bf16 won"
((q - z) * s, then a cast to the element type), with z = 0.

* E2M1 + E8M0: bf16(v * 2^(c - 127)); exact for every finite result, bf16
  subnormals included; overflow becomes inf; scale code 0xFF is NaN.
* E4M3: bf16(v), exact; the per-output-channel fp32 scale is not part of the
  operand (it factors out of the dot product and is applied to the fp32
  accumulator), so it is not applied here.  NaN codes give a NaN.
* INT4: bf16(q * s) with one round to nearest even of the exact product.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_decode, bf16_round, e2m1_decode, e4m3_decode, e8m0_decode
from .int4 import unpack_int4
from .mxfp4 import unpack_nibbles


def dequant_mxfp4(packed, scale_codes, block: int) -> np.ndarray:
    codes = unpack_nibbles(packed)
    rows, cols = codes.shape
    v = e2m1_decode(codes).reshape(rows, cols // block, block)
    s = e8m0_decode(scale_codes)[:, :, None]
    with np.errstate(invalid="ignore", over="ignore"):
        return bf16_round((v * s).reshape(rows, cols))


def dequant_e4m3(codes) -> np.ndarray:
    return bf16_round(e4m3_decode(codes))


def dequant_int4(packed, scale_bits, group: int) -> np.ndarray:
    q = unpack_int4(packed).astype(np.float64)
    N, K = q.shape
    s = bf16_decode(scale_bits)[:, :, None]
    with np.errstate(invalid="ignore", over="ignore"):
        return bf16_round((q.reshape(N, K // group, group) * s).reshape(N, K))
