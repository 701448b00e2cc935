"""MXFP4: E2M1 element codes under an E8M0 block scale.

Follows "Numerics: FP32 to INT4, and why bf16 won", section "MXFP4 and the
block-scaled family" (32-element blocks sharing one power-of-two scale, the
E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their midpoints, 4.25 bits per
weight) and vLLM PR #43557 (the E8M0 rule, "Why This Helps Precision": the
block maximum saturates at 6.0; the same rule is used on 16-element blocks).

Element step: v = x * 2^(127 - code) (exact in fp64), then v is rounded to the
nearest E2M1 magnitude with saturation at 6; the sign bit is the sign of x.

Readings:
* ties at the midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 go to the even
  code (the same round-to-nearest-even convention as E4M3), so
  0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4;
* a negative value that rounds to zero keeps its sign (code 0x8);
* packing: element 2j goes to the low nibble of byte j (the pages only say two
  codes share a byte) -- parity unpinned, self-consistency only.
"""
from __future__ import annotations

import numpy as np

from .e8m0 import block_absmax, e8m0_code_bits
from .formats import E2M1_GRID, f32_bits


def e2m1_from_f64(v, sign_bits) -> np.ndarray:
    """Arithmetic derivation.  Below 2 the grid spacing is 0.5 (codes 0..4 are
    rint(2|v|)), in [2, 4) it is 1 (codes 4..6 are rint(|v|) + 2), in [4, 6]
    it is 2 (codes 6..7 are rint(|v|/2) + 4), and anything above 6 saturates.
    `sign_bits` (0/1) is the sign of the unscaled input."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    c = np.where(a < 2.0, np.rint(a * 2.0),
         np.where(a < 4.0, np.rint(a) + 2.0,
          np.where(a <= 6.0, np.rint(a / 2.0) + 4.0, 7.0)))
    # rint(a*2) can reach 4 (=2.0), rint(a) can reach 4 (=4.0 -> code 6): both are
    # the correct codes of the next binade's first value.
    c = np.minimum(c, 7.0).astype(np.uint8)
    return (c | (np.asarray(sign_bits, dtype=np.uint8) << 3)).astype(np.uint8)


def e2m1_from_f64_bruteforce(v, sign_bits) -> np.ndarray:
    """Second derivation: nearest of the eight magnitudes, ties to the even
    code, values beyond 6 saturate to 6."""
    # beyond 16 every value is nearest to 6; the clamp keeps fp64 distances exact
    a = np.minimum(np.abs(np.asarray(v, dtype=np.float64)).reshape(-1), 16.0)
    d = np.abs(a[:, None] - E2M1_GRID[None, :])
    dmin = d.min(axis=1, keepdims=True)
    ties = d == dmin
    codes = np.arange(8)
    even = ties & ((codes[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), ties.argmax(axis=1))
    c = pick.astype(np.uint8).reshape(np.shape(v))
    return (c | (np.asarray(sign_bits, dtype=np.uint8) << 3)).astype(np.uint8)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """rows x cols 4-bit codes -> rows x cols/2 bytes; element 2j in the low
    nibble of byte j."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def quantize_mxfp4(x, block: int):
    """x: rows x cols fp32 (bf16 widened exactly by the caller); block in {32, 16}.
    Returns (packed codes uint8 rows x cols/2, E8M0 codes uint8 rows x cols/block)."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if x32.ndim != 2:
        raise ValueError("expected a 2-D array")
    rows, cols = x32.shape
    vmax = block_absmax(x32, block)                  # raises on bad block
    scale_codes = e8m0_code_bits(vmax)               # raises on non-finite input
    inv = np.exp2(127.0 - scale_codes.astype(np.float64))          # 2^(127 - code)
    v = x32.astype(np.float64).reshape(rows, cols // block, block) * inv[:, :, None]
    sign = ((f32_bits(x32) >> 31) & 1).astype(np.uint8).reshape(v.shape)
    codes = e2m1_from_f64(v, sign).reshape(rows, cols)
    return pack_nibbles(codes), scale_codes
