"""W8A8 FP8: E4M3 activations times E4M3 weights with fp32 accumulation and
the dequantization scales folded in per K block.

Follows "Numerics: FP32 to INT4, and why bf16 won": the Triton block-scaled
FP8 GEMM quoted in the section on storage versus accumulation dtypes (an fp32
accumulator; per K block the product of the two fp8 tiles is scaled by the
activation scale of each row and the weight scale of each column and added;
one narrowing cast at the store), the fp8 linear walkthrough (step 2: value
divided by the scale in fp32, saturating clamp to +-448, conversion; step 3:
quantized row times quantized weight with both scales folded in inside the K
loop, one cast to bf16) and section "Granularity" (per-tensor, per-token,
per-channel and per-group scales; per-tensor and per-channel scales factor
out of the inner product).  The per-tensor static activation quantizer is the
one FreeToken PR #805 lists among its E4M3 cast sites.

Readings where the pages are silent:
* K blocks of 128 (the group size the pages use along K); the weight scale of
  a K block is shared by 128 consecutive output channels (128 x 128 weight
  blocks) or is per channel;
* weight block quantization uses the activation recipe on 2-D blocks:
  s = RN_f32(amax / 448) (1 if zero), codes e4m3(RN_f32(w / s));
* static per-tensor quantization: codes e4m3(RN_f32(x / s)) with the given
  fp32 scale s > 0, correctly rounded division, saturating;
* the product's exact value is sum_k (a_k s_a) (b_k s_b) over the dequantized
  operands; a GEMM result is accepted within the matmul bound.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import e4m3_from_f32, e4m3_scale
from .formats import e4m3_decode

KBLOCK = 128


def quantize_e4m3_static(x, scale: float) -> np.ndarray:
    """Per-tensor static E4M3 quantization with a given fp32 scale."""
    s = np.float32(scale)
    if not (np.isfinite(s) and s > 0):
        raise ValueError("scale must be finite and positive")
    x32 = np.asarray(x, dtype=np.float32)
    if not np.isfinite(x32).all():
        raise ValueError("non-finite input")
    with np.errstate(over="ignore", under="ignore"):
        q = (x32 / s).astype(np.float32)                # IEEE fp32 division
    return e4m3_from_f32(q)


def quantize_e4m3_block2d(w, bn: int = 128, bk: int = KBLOCK):
    """w: N x K fp32.  One fp32 scale per bn x bk block.  Returns (codes uint8
    N x K, scales fp32 ceil(N/bn) x K/bk).  A partial last row block uses the
    rows it has."""
    w32 = np.ascontiguousarray(np.asarray(w, dtype=np.float32))
    N, K = w32.shape
    if K % bk:
        raise ValueError("K must be a multiple of the block size")
    if not np.isfinite(w32).all():
        raise ValueError("non-finite weight")
    nb = (N + bn - 1) // bn
    scales = np.empty((nb, K // bk), np.float32)
    codes = np.empty((N, K), np.uint8)
    for i in range(nb):
        blk = w32[i * bn:(i + 1) * bn].reshape(-1, K // bk, bk)
        amax = np.abs(blk).max(axis=(0, 2))
        s = e4m3_scale(amax)
        scales[i] = s
        q = (blk / s[None, :, None]).astype(np.float32)
        codes[i * bn:(i + 1) * bn] = e4m3_from_f32(q).reshape(-1, K)
    return codes, scales


def expand_scales(scale, rows: int, kblocks: int, group_rows: int = 1) -> np.ndarray:
    """Scale of every (row, K block) from a scalar (per tensor), a vector (per
    row group, the same for every K block) or a matrix (per row group and K
    block); a row group holds group_rows consecutive rows."""
    s = np.asarray(scale, np.float64)
    if s.ndim == 0:
        s, group_rows = np.full((1, kblocks), float(s)), rows
    elif s.ndim == 1:
        s = np.repeat(s[:, None], kblocks, axis=1)
    return np.repeat(s, group_rows, axis=0)[:rows]


def reference(a_codes, a_scale_rk, b_codes, b_scale_rk):
    """Exact fp64 y[m, n] = sum_kb a_s[m, kb] b_s[n, kb] sum_{k in kb} a[m, k] b[n, k]
    and the acceptance weight sum_k |a_k s_a b_k s_b|.  Scales are given per
    (row, K block)."""
    a = e4m3_decode(a_codes)
    b = e4m3_decode(b_codes)
    M, K = a.shape
    N = b.shape[0]
    kb = K // KBLOCK
    y = np.zeros((M, N))
    asum = np.zeros((M, N))
    for j in range(kb):
        sl = slice(j * KBLOCK, (j + 1) * KBLOCK)
        part = a[:, sl] @ b[:, sl].T
        apart = np.abs(a[:, sl]) @ np.abs(b[:, sl]).T
        f = np.asarray(a_scale_rk)[:, j][:, None] * np.asarray(b_scale_rk)[:, j][None, :]
        y += part * f
        asum += apart * np.abs(f)
    return y, asum
