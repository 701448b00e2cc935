"""Oracle-side work for the W4A8 parity tests that runs in worker processes
(NumPy and the oracle only; no GPU): quantize one expert's fp32 weights and
compute the fp64 reference for sampled grouped rows of that expert."""
import numpy as np

from oracle import e4m3 as OE
from oracle import int4 as OI
from oracle import w4a8 as OW
from oracle.formats import e4m3_decode


def expert_case(Wf, x8_rows, a_rows):
    """Wf: N x K fp32 weights of one expert; x8_rows / a_rows: E4M3 codes and
    fp32 scales of the tokens of the sampled rows.  Returns (packed, scale bits,
    s8, ch, y_ref, abs_sum) with y_ref and abs_sum of shape rows x N."""
    packed, sb, _ = OI.quantize_int4(Wf, 128)
    s8, ch = OW.scale_recipe(sb)
    w = OW.expert_operand(packed, s8, 128)
    xv = e4m3_decode(x8_rows)
    sc = a_rows.astype(np.float64)[:, None] * ch.astype(np.float64)[None, :]
    y = (xv @ w.T) * sc
    a = (np.abs(xv) @ np.abs(w).T) * np.abs(sc)
    return packed, sb, s8, ch, y, a


def token_rows(x_bits_rows):
    """Per-token E4M3 quantization of bf16 rows (codes, fp32 scales)."""
    return OW.quantize_tokens(x_bits_rows)
