"""E8M0 shared block scale: the exponent-first rule with 0.75-threshold rounding.

Follows "Fix the E8M0 scale computation in the MXFP4 (W4A4) MOE CUTLASS
kernel" (vLLM PR #43557), sections "Fix: Exponent-First with 0.75-Threshold
Rounding" and "Origin: Matching the Quantization Toolchain".  The block maximum
magnitude is taken as an fp32 bit pattern; adding 2^21 to it carries into the
exponent field exactly when the mantissa fraction is at least 0.75; the
rounded biased exponent minus 2 (clamped at 0) is the E8M0 code, i.e. the
scale 2^(code - 127).

Two derivations are given and must agree:
* `e8m0_code_bits`: the bit formulation (round the fp32 pattern, extract the
  biased exponent, subtract 2);
* `e8m0_code_arith`: the arithmetic formulation of the same rule for a normal
  maximum (1 + f) * 2^E: code = E + 127 - 2 + [f >= 0.75], clamped at 0.

Readings: a block containing a non-finite value is out of contract
(ValueError); an all-zero block gives code 0 (the literal formula).
"""
from __future__ import annotations

import numpy as np

from .formats import f32_bits


def block_absmax(x32: np.ndarray, block: int) -> np.ndarray:
    """Maximum magnitude of each 1 x block group along the last axis (exact)."""
    rows, cols = x32.shape
    if block <= 0 or cols % block:
        raise ValueError("cols must be a multiple of the block size")
    return np.abs(x32.reshape(rows, cols // block, block)).max(axis=2)


def e8m0_code_bits(vecmax) -> np.ndarray:
    v = np.asarray(vecmax, dtype=np.float32)
    if not np.isfinite(v).all():
        raise ValueError("non-finite block maximum")
    bits = f32_bits(np.abs(v)).astype(np.uint64)
    rounded = (bits + (1 << 21)) & 0xFF800000
    biased = (rounded >> 23) & 0xFF
    return np.where(biased > 2, biased - 2, 0).astype(np.uint8)


def e8m0_code_arith(vecmax) -> np.ndarray:
    v = np.abs(np.asarray(vecmax, dtype=np.float32).astype(np.float64))
    if not np.isfinite(v).all():
        raise ValueError("non-finite block maximum")
    out = np.zeros(v.shape, np.int64)
    normal = v >= 2.0 ** -126
    fr, ex = np.frexp(np.where(normal, v, 1.0))      # v = fr * 2^ex, fr in [0.5, 1)
    E = ex.astype(np.int64) - 1                       # v = (1 + f) * 2^E
    f = fr * 2.0 - 1.0
    code = E + 127 - 2 + (f >= 0.75).astype(np.int64)
    out = np.where(normal, np.maximum(code, 0), 0)
    # an fp32 subnormal maximum has biased exponent 0 (or 1 after the carry),
    # which the rule clamps to code 0
    return out.astype(np.uint8)


def e8m0_scale(code) -> np.ndarray:
    """Scale value 2^(code - 127) as fp64 (exact)."""
    return np.exp2(np.asarray(code, dtype=np.float64) - 127.0)
