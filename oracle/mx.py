"""MX block quantizers with a choice of E8M0 scale rule, for E2M1 (MXFP4) or
E4M3 (MXFP8) elements.

Follows "Fix the E8M0 scale computation in the MXFP4 (W4A4) MOE CUTLASS
kernel" (vLLM PR #43557): section "Root Cause" (the old rule, the biased
exponent of vecMax / 6), "Fix: Exponent-First with 0.75-Threshold Rounding"
and "Origin: Matching the Quantization Toolchain" (add a rounding increment to
the fp32 pattern of vecMax, take the biased exponent, subtract the element
format's exponent offset; compressed-tensors writes the increment as
1 << (23 - m - 1) for an element format with m mantissa bits), and "Why This
Helps Precision (Not Strict OCP MX)" (strict OCP: no increment; threshold 0.5:
increment 1 << 22).  And "Numerics: FP32 to INT4, and why bf16 won", section
"MXFP4 and the block-scaled family" (the OCP MX element formats include
mxfp8_e4m3; SGLang's quantizer: descale = amax / 6, scale exponent
ceil(log2(descale)) with a floor of -127, stored biased by 127).

Element formats: E2M1 (m = 1, largest value 6 = 1.5 * 2^2, offset 2) and E4M3
(m = 3, largest value 448 = 1.75 * 2^8, offset 8).

Rules (vmax = the block's maximum magnitude, an fp32 value):
  "round":     biased_exp((bits(vmax) + 2^(22 - m)) & 0xFF800000) - offset,
               clamped at 0 (E2M1: + 2^21, the 0.75 threshold of quantize_mxfp4)
  "half":      the same with + 2^22 (threshold 0.5)
  "ocp":       biased_exp(vmax) - offset, clamped at 0
  "floor_div": biased_exp(RN_f32(vmax * RN_f32(1 / max_elem)))
  "ceil_div":  max(ceil(log2(RN_f32(vmax / max_elem))), -127) + 127

Readings where the pages are silent:
* the E4M3 offset is its largest binade, 8, as 2 is for E2M1, and its "round"
  increment is the compressed-tensors value for m = 3, 2^19;
* "half" uses 2^22 for both element formats (the page gives it as a
  threshold, not as a function of m);
* "floor_div" multiplies by the fp32 reciprocal of the element maximum (the
  listing multiplies by an approximate reciprocal of 6, whose exact value is
  not given; the correctly rounded one is taken), "ceil_div" divides by it in
  fp32 with correct rounding;
* "ceil_div" rounds the fp32 quotient up to a power of two exactly, as the
  prose describes (an fp32 log2 followed by ceil would lose the rounding up for
  quotients a few ulps above a power of two); an all-zero block gives code 0
  under every rule;
* elements: v = x * 2^(127 - code) exactly, then the element rounding of
  quantize_mxfp4 (E2M1) or of the E4M3 cast (nearest even, saturating at 448).
Two derivations are given for every rule: `scale_code` works on fp32 bit
patterns, `scale_code_arith` on exact real arithmetic (frexp, fractions).
"""
from __future__ import annotations

import numpy as np

from .e4m3 import e4m3_from_f32
from .e8m0 import block_absmax
from .formats import f32_bits
from .mxfp4 import e2m1_from_f64, pack_nibbles

RULES = ("round", "half", "ocp", "floor_div", "ceil_div")
ELEMS = {"e2m1": (1, 2, 6.0), "e4m3": (3, 8, 448.0)}   # mantissa bits, offset, largest value


def _check(vmax):
    v = np.abs(np.asarray(vmax, dtype=np.float32))
    if not np.isfinite(v).all():
        raise ValueError("non-finite block maximum")
    return v


def _quotient(v, rule, emax):
    """The fp32 value whose exponent the division rules take."""
    with np.errstate(under="ignore"):
        if rule == "floor_div":
            return (v * (np.float32(1.0) / np.float32(emax))).astype(np.float32)
        return (v / np.float32(emax)).astype(np.float32)


def scale_code(vmax, rule: str, elem: str) -> np.ndarray:
    """E8M0 code of each block maximum under `rule` for element format `elem`."""
    m, off, emax = ELEMS[elem]
    v = _check(vmax)
    bits = f32_bits(v).astype(np.int64)
    if rule in ("round", "half", "ocp"):
        inc = {"round": 1 << (22 - m), "half": 1 << 22, "ocp": 0}[rule]
        biased = (((bits + inc) & 0xFF800000) >> 23) & 0xFF
        return np.where(biased > off, biased - off, 0).astype(np.uint8)
    q = _quotient(v, rule, emax)
    qb = f32_bits(q).astype(np.int64)
    biased = (qb >> 23) & 0xFF
    if rule == "floor_div":
        return biased.astype(np.uint8)
    if rule == "ceil_div":
        frac = qb & 0x7FFFFF
        # normal q: ceil(log2 q) = E + [fraction != 0]; subnormal or zero q is
        # below 2^-126, so its ceiling is at most -126 (zero: -inf), and the
        # floor of -127 applies unless q > 2^-127
        e = np.where(biased > 0, biased - 127 + (frac != 0), np.where(qb > (1 << 22), -126, -127))
        return (np.maximum(e, -127) + 127).astype(np.uint8)
    raise ValueError(f"unknown rule {rule}")


def scale_code_arith(vmax, rule: str, elem: str) -> np.ndarray:
    """Second derivation in exact arithmetic: vmax = (1 + f) * 2^E."""
    m, off, emax = ELEMS[elem]
    v = _check(vmax).astype(np.float64)
    if rule in ("round", "half", "ocp"):
        thr = {"round": 1.0 - 2.0 ** -(m + 1), "half": 0.5, "ocp": 2.0}[rule]
        normal = v >= 2.0 ** -126
        fr, ex = np.frexp(np.where(normal, v, 1.0))
        E = ex.astype(np.int64) - 1
        f = fr * 2.0 - 1.0
        code = E + 127 - off + (f >= thr).astype(np.int64)
        # subnormal maxima: biased exponent 0, or 1 after the carry of "half" for
        # fractions >= 0.5 of the subnormal range; both clamp to 0 for off >= 2
        return np.where(normal, np.maximum(code, 0), 0).astype(np.uint8)
    q = _quotient(_check(vmax), rule, emax).astype(np.float64)
    pos = q > 0
    fr, ex = np.frexp(np.where(pos, q, 1.0))                    # q = fr * 2^ex, fr in [0.5, 1)
    if rule == "floor_div":
        fl = ex.astype(np.int64) - 1                              # floor(log2 q)
        return np.where(pos, np.maximum(fl + 127, 0), 0).astype(np.uint8)
    if rule == "ceil_div":
        ce = np.where(fr == 0.5, ex - 1, ex).astype(np.int64)      # ceil(log2 q)
        return np.where(pos, np.maximum(ce, -127) + 127, 0).astype(np.uint8)
    raise ValueError(f"unknown rule {rule}")


def quantize_mx(x, block: int, elem: str, rule: str):
    """x: rows x cols fp32; block in {16, 32}.  Returns (codes, E8M0 scales):
    E2M1 codes packed two per byte (element 2j in the low nibble of byte j),
    rows x cols/2; E4M3 codes rows x cols; scales rows x cols/block."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if x32.ndim != 2:
        raise ValueError("expected a 2-D array")
    rows, cols = x32.shape
    vmax = block_absmax(x32, block)
    code = scale_code(vmax, rule, elem)
    inv = np.exp2(127.0 - code.astype(np.float64))
    v = x32.astype(np.float64).reshape(rows, cols // block, block) * inv[:, :, None]
    v = v.reshape(rows, cols)
    if elem == "e2m1":
        sign = (f32_bits(x32) >> 31).astype(np.uint8)
        return pack_nibbles(e2m1_from_f64(v, sign)), code
    # v is exact in fp64; E4M3 of it equals E4M3 of the fp32 value when v is an
    # fp32 number, which holds unless v underflows fp32 (then it rounds to zero)
    return e4m3_from_f32(v.astype(np.float32)), code
