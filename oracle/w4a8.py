"""W4A8 mixture-of-experts grouped GEMM: routing, the scale recipe, the
INT4 -> E4M3 lookup table and the fp64 reference.

Follows "Production-Ready W4A8: vLLM Integration and Quality Recovery
Techniques Explained" (Cohere), sections "High-Performance W4A8 GEMM Kernel"
(for one fp8 scale s there are only 16 values s * w over the INT4 codes w, so
the dequantization is a table lookup feeding an fp8 x fp8 multiply with fp32
accumulation) and "Accurate W4A8 Kernel" (each output channel's bf16 group
scales are themselves quantized to fp8 with an fp32 channel scale, the same
operation as per-token activation quantization; the fp8 scales are multiplied
by 1/8 and the channel scales by 8 so that every s * w stays inside the E4M3
range; the per-token and per-channel fp32 scales are applied in the epilogue).

Readings where the page is silent:
* the 1/8 is folded into the channel scale before the fp8 rounding of the
  group scales: ch_n = 8 * RN_f32(amax_n / 448) (= RN_f32(amax_n / 56)),
  s8[n, g] = e4m3(RN_f32(s[n, g] / ch_n)), so the largest group scale of a
  channel maps to 56 = 448 / 8 and |w * s8| <= 448 never clips;
* LUT[n, g][w] = e4m3(w * s8[n, g]) for all 16 codes, each product rounded
  once to nearest even ("precompute eight of them" is read as a storage detail:
  the negative half is the positive half with the sign bit set);
* activations: per-token E4M3 with one fp32 scale per row (amax / 448);
* routing: softmax over the expert logits, top-k by probability, equal
  probabilities resolved towards the lower expert id (softmax is increasing,
  so this is the top-k of the logits); rows are grouped by expert, in
  increasing token order within an expert; re-normalisation of the top-k
  weights and the activation between the two GEMMs are outside this op.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import e4m3_from_f32, e4m3_scale, quantize_e4m3
from .formats import bf16_decode, bf16_round, e4m3_decode
from .int4 import unpack_int4


def route_topk(logits, k: int):
    """logits: T x E fp32.  Returns (ids int32 T x k, weights fp32 T x k), the
    experts in order of decreasing probability (ties: lower id first)."""
    z = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = z.shape
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    # stable sort on (-logit) keeps lower ids first among equal logits
    order = np.argsort(-np.asarray(logits, dtype=np.float32), axis=1, kind="stable")[:, :k]
    w = np.take_along_axis(p, order, axis=1)
    return order.astype(np.int32), w.astype(np.float32)


def group_by_expert(ids, n_experts: int):
    """Returns (offsets int32 E+1, row_token int32 T*k, row_slot int32 T*k):
    grouped row r belongs to expert e for offsets[e] <= r < offsets[e+1], reads
    token row_token[r], and came from top-k position row_slot[r]."""
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    counts = np.bincount(ids.reshape(-1), minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")            # stable: increasing token id
    return offsets, (order // k).astype(np.int32), (order % k).astype(np.int32)


def scale_recipe(scale_bits):
    """scale_bits: N x G bf16 INT4 group scales of one expert.
    Returns (s8 E4M3 codes N x G, ch fp32 N)."""
    s = bf16_decode(scale_bits).astype(np.float32)
    amax = np.abs(s).max(axis=1)
    ch = (np.float32(8.0) * e4m3_scale(amax)).astype(np.float32)
    s8 = e4m3_from_f32((s / ch[:, None]).astype(np.float32))            # IEEE fp32 division
    return s8, ch


def lut(s8_codes) -> np.ndarray:
    """s8: N x G E4M3 codes -> N x G x 16 E4M3 codes; entry u is the two's-
    complement nibble u (u >= 8 means u - 16)."""
    v = e4m3_decode(s8_codes)
    w = np.arange(16)
    w = np.where(w >= 8, w - 16, w).astype(np.float64)
    prod = v[..., None] * w                                             # exact
    return e4m3_from_f32(prod.astype(np.float32))


def expert_operand(packed, s8_codes, group: int) -> np.ndarray:
    """Exact E4M3 values of the looked-up weights, N x K (fp64)."""
    q = unpack_int4(packed).astype(np.int64)
    N, K = q.shape
    table = lut(s8_codes)                                               # N x G x 16
    g = np.arange(K) // group
    codes = table[np.arange(N)[:, None], g[None, :], q & 0xF]
    return e4m3_decode(codes)


def quantize_tokens(x_bf16_bits):
    """Per-token E4M3: returns (codes T x H, scale fp32 T)."""
    x = bf16_decode(x_bf16_bits).astype(np.float32)
    codes, scale = quantize_e4m3(x, -1)
    return codes, scale[:, 0]


def grouped_gemm_reference(x8_codes, a_scale, offsets, row_token, experts, group: int, rows=None):
    """x8_codes: T x K token codes, a_scale: T; experts: list of
    (packed N x K/8, s8 N x G, ch N).  Grouped row r uses expert e(r) and token
    row_token[r].  Returns (y_ref fp64, abs_sum fp64) for the requested rows
    (all rows if None), each of width N."""
    offsets = np.asarray(offsets)
    R = int(offsets[-1])
    rows = np.arange(R) if rows is None else np.asarray(rows)
    e_of = np.searchsorted(offsets, rows, side="right") - 1
    N = experts[0][0].shape[0]
    y = np.zeros((len(rows), N))
    a = np.zeros((len(rows), N))
    for e in np.unique(e_of):
        sel = np.where(e_of == e)[0]
        packed, s8, ch = experts[e]
        w = expert_operand(packed, s8, group)                           # N x K exact
        xv = e4m3_decode(x8_codes[row_token[rows[sel]]])                # exact
        acc = xv @ w.T
        absacc = np.abs(xv) @ np.abs(w).T
        sc = a_scale[row_token[rows[sel]]].astype(np.float64)[:, None] * ch.astype(np.float64)[None, :]
        y[sel] = acc * sc
        a[sel] = absacc * np.abs(sc)
    return y, a


def bf16_out(y_ref) -> np.ndarray:
    return bf16_round(y_ref)
