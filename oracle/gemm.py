"""fp64 reference for y = x . dequant(Wq)^T and the acceptance bound.

Follows "Numerics: FP32 to INT4, and why bf16 won" (storage dtype is not the
accumulate dtype: narrow operands, fp32 accumulator, one narrowing cast at the
end; the serial-sum error bound gamma_(n-1) * sum|x_i| for an fp32 accumulator;
the 2^-8 relative bound of a bf16 rounding) and the per-channel scale that
factors out of the inner product (section "Granularity: one scale for how many
numbers?").

With the dequantized operands fixed, the exact result is an fp64 dense matmul:
y_ref[m, n] = chan[n] * sum_k x[m, k] * w[n, k].  The acceptance bound for a
bf16 output computed with fp32 accumulation is
    |y - y_ref| <= 8e-3 * |y_ref| + 1e-3 * sum_k |x[m, k] * w_eff[n, k]|
where w_eff includes the channel scale.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_decode

REL_TOL = 8e-3
ABS_SUM_TOL = 1e-3


def reference(x_bf16_bits, w_bf16_bits, chan_scale=None):
    """Returns (y_ref fp64 M x N, abs_sum fp64 M x N)."""
    x = bf16_decode(x_bf16_bits)
    w = bf16_decode(w_bf16_bits)
    y = x @ w.T
    a = np.abs(x) @ np.abs(w).T
    if chan_scale is not None:
        c = np.asarray(chan_scale, dtype=np.float64).reshape(1, -1)
        y = y * c
        a = a * np.abs(c)
    return y, a


def reference_rows(x_bf16_bits, w_bf16_bits, rows, chan_scale=None):
    """Reference restricted to the given rows of x (for large-M spot checks)."""
    return reference(np.asarray(x_bf16_bits)[rows], w_bf16_bits, chan_scale)


def within_tolerance(y, y_ref, abs_sum):
    """Element-wise acceptance mask."""
    y = np.asarray(y, dtype=np.float64)
    return np.abs(y - y_ref) <= REL_TOL * np.abs(y_ref) + ABS_SUM_TOL * abs_sum


def worst_ratio(y, y_ref, abs_sum) -> float:
    """max |y - y_ref| / bound (<= 1 means every element passes)."""
    y = np.asarray(y, dtype=np.float64)
    bound = REL_TOL * np.abs(y_ref) + ABS_SUM_TOL * abs_sum
    err = np.abs(y - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    return float(r.max()) if r.size else 0.0
