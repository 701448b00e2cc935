"""fp32 -> OCP FP8-E4M3 ("fn"), round to nearest even, saturating; and the
scaled (per-block / per-row) E4M3 quantizer.

Rounding semantics follow FreeToken PR #805 (fp32 -> E4M3 double rounding on
sm_89): the conversion is a single round-to-nearest-even step from fp32 with
saturation to the largest finite value (the "rn.satfinite" conversion), and
200.04 must become 208, not the 192 that an fp32 -> fp16 -> E4M3 double
rounding gives.  The saturating clamp (an out-of-range value becomes +-448,
never inf) follows the fp8 linear walkthrough of "Numerics: FP32 to INT4, and
why bf16 won" (step 2, the scaled conversion helper).

Readings where the pages are silent:
* NaN input -> 0x7F with the input's sign bit (the pages only say to validate
  non-finite values; clamping it to 448 would hide it).
* +-inf -> +-448 (satfinite).
* The sign of zero and of values that round to zero is kept (0x80 for
  negative), as the ROCm validation in the same PR lists signed zero.

The scaled quantizer follows step 1 of the same walkthrough (dynamic per-token
FP8): amax over the group, scale = amax / 448 in fp32, the group divided by the
scale in fp32, then the saturating conversion.  Readings:
* division is the correctly rounded fp32 division (the text says the row is
  divided by the scale in fp32; the reciprocal-multiply of the quoted code is
  a performance variant, not the definition);
* the scale clamp constant is not printed; the all-zero-group policy s = 1 of
  the scale-policy paragraph is used, extended to any group whose fp32 scale
  rounds to zero;
* groups holding a non-finite value are out of contract (ValueError).
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3_POS_CODES, E4M3_POS_VALUES, f32_bits

E4M3_MAX = 448.0


def e4m3_from_f32(x) -> np.ndarray:
    """Arithmetic derivation.  |x| is taken exactly in fp64; below the smallest
    normal 2^-6 the grid spacing is 2^-9 (subnormals), in the binade
    [2^E, 2^(E+1)) it is 2^(E-3); the magnitude is rint(|x| / spacing) on that
    grid (ties to even), and anything at or above 448 saturates to 448."""
    xf = np.asarray(x, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        a = np.abs(xf.astype(np.float64))
    sign = ((f32_bits(xf) >> 31) & 1).astype(np.uint8) << 7
    nan = np.isnan(a)
    sat = ~nan & (a >= E4M3_MAX)
    with np.errstate(invalid="ignore"):
        fin = np.where(nan | sat, 1.0, a)
        _, ex = np.frexp(np.where(fin > 0, fin, 1.0))
        E = np.maximum(ex.astype(np.int64) - 1, -6)        # subnormal spacing at E = -6
        spacing = np.exp2((E - 3).astype(np.float64))
        q = np.rint(fin / spacing).astype(np.int64)         # significand on the grid
    # q in [0, 16]; q == 16 means a carry into the next binade.
    carry = q == 16
    E = np.where(carry, E + 1, E)
    q = np.where(carry, 8, q)
    # normal when q >= 8 (implicit bit present); subnormal when E == -6 and q < 8
    is_norm = q >= 8
    exp_field = np.where(is_norm, E + 7, 0)
    man = np.where(is_norm, q - 8, q)
    code = (exp_field << 3) | man
    code = np.where(sat, 0x7E, code)
    code = np.where(nan, 0x7F, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_from_f32_bruteforce(x) -> np.ndarray:
    """Second derivation: nearest value of the full E4M3 table (all 127
    non-negative finite codes), ties to the even code, saturating."""
    xf = np.asarray(x, dtype=np.float32).reshape(-1)
    # Beyond 1024 every finite value is nearest to the largest grid value; the
    # clamp keeps the fp64 distances exact for huge inputs.
    a = np.minimum(np.abs(xf.astype(np.float64)), 1024.0)
    sign = ((f32_bits(xf) >> 31) & 1).astype(np.uint8) << 7
    out = np.empty(a.shape, np.uint8)
    vals = E4M3_POS_VALUES
    for i0 in range(0, a.size, 1 << 16):
        blk = a[i0:i0 + (1 << 16)]
        with np.errstate(invalid="ignore"):
            d = np.abs(blk[:, None] - vals[None, :])
        dmin = d.min(axis=1, keepdims=True)
        ties = d == dmin
        # among the nearest codes prefer the even one (its mantissa LSB is 0)
        even = ties & ((E4M3_POS_CODES[None, :] & 1) == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), ties.argmax(axis=1))
        c = E4M3_POS_CODES[pick]
        c = np.where(np.isnan(blk), 0x7F, c)
        out[i0:i0 + blk.size] = c
    return (out | sign).reshape(np.shape(x)).astype(np.uint8)


def _group_view(x32: np.ndarray, block: int) -> np.ndarray:
    rows, cols = x32.shape
    if block == -1:
        return x32.reshape(rows, 1, cols)
    if block <= 0 or cols % block:
        raise ValueError("cols must be a multiple of the block size")
    return x32.reshape(rows, cols // block, block)


def e4m3_scale(amax_f32: np.ndarray) -> np.ndarray:
    """scale = RN_f32(amax / 448); a scale that is zero (all-zero group, or an
    fp32 quotient that underflows) is replaced by 1."""
    amax = np.asarray(amax_f32, dtype=np.float32)
    s = amax / np.float32(E4M3_MAX)                     # IEEE fp32 division
    return np.where(s == 0, np.float32(1.0), s).astype(np.float32)


def quantize_e4m3(x, block: int):
    """x: rows x cols fp32 (bf16 inputs are widened exactly by the caller).
    block == 0: plain cast, returns (codes, None).
    block > 0: one fp32 scale per 1 x block group; block == -1: one per row.
    Returns (codes uint8 rows x cols, scales fp32 rows x groups)."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if block == 0:
        return e4m3_from_f32(x32), None
    if x32.ndim != 2:
        raise ValueError("expected a 2-D array")
    if not np.isfinite(x32).all():
        raise ValueError("non-finite input to a scaled E4M3 quantizer")
    g = _group_view(x32, block)
    amax = np.abs(g).max(axis=2)                        # exact
    scale = e4m3_scale(amax)
    q = g / scale[:, :, None]                           # IEEE fp32 division
    codes = e4m3_from_f32(q.astype(np.float32)).reshape(x32.shape)
    return codes, scale
