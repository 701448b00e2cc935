"""GPU parity of wq_gemm (decode GEMV and prefill GEMM) against the oracle's
fp64 reference, with the acceptance bound
    |y - y_ref| <= 8e-3 |y_ref| + 1e-3 sum_k |x_k w_k|
per element.  Weights are quantized by the oracle (inputs never come from the
GPU path)."""
import numpy as np
import pytest
import torch

from oracle import dequant as OD
from oracle import e4m3 as OE
from oracle import gemm as OG
from oracle import int4 as OI
from oracle import mxfp4 as OM
from oracle.formats import bf16_decode
from synthetic import decode_inputs, mxfp4_gemv_inputs, prefill_inputs, to_bf16_bits
from tests.gpu_helpers import banner, check_all_rows, dev_bf16, dev_f32, dev_u8, dev_words, host_bits16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def W():
    import weight_only_quantized_quant_amd as W
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return W


def _prep(W, kind, Wf, group=128):
    """Quantize fp32 weights with the oracle; return (device args, oracle bf16 operand, chan scale)."""
    if kind == "int4":
        packed, sb, _ = OI.quantize_int4(Wf, group)
        args = (dev_words(packed), W.WQ_INT4X8, dev_bf16(sb), W.WQ_BF16, group)
        return args, OD.dequant_int4(packed, sb, group), None
    if kind == "mxfp4":
        codes, sc = OM.quantize_mxfp4(Wf, 32)
        args = (dev_u8(codes), W.WQ_E2M1X2, dev_u8(sc), W.WQ_E8M0, 32)
        return args, OD.dequant_mxfp4(codes, sc, 32), None
    codes, s = OE.quantize_e4m3(Wf, -1)
    args = (dev_u8(codes), W.WQ_E4M3, dev_f32(s[:, 0]), W.WQ_F32, Wf.shape[1])
    return args, OD.dequant_e4m3(codes), s[:, 0]


def _check(y_dev, xbits, wdeq, chan, rows=None):
    y = bf16_decode(host_bits16(y_dev))
    xb = xbits if rows is None else xbits[rows]
    if rows is not None:
        y = y[rows]
    ref, asum = OG.reference(xb, wdeq, chan)
    ratio = OG.worst_ratio(y, ref, asum)
    assert np.isfinite(y).all()
    assert ratio <= 1.0, f"worst error / bound = {ratio:.3f}"
    return ratio


@pytest.mark.parametrize("kind", ["int4", "mxfp4", "e4m3"])
@pytest.mark.parametrize("M,N,K", [(1, 1000, 384), (3, 520, 512), (16, 272, 1024), (5, 17, 128), (2, 4096, 2048)])
def test_gemv_ragged(W, kind, M, N, K):
    g = np.random.default_rng(M * 1000 + N + K)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, g.choice(K, 3, replace=False)] *= 40
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, kind, Wf)
    banner("gemv", kind, M, N, K)
    y = W.wq_gemm(dev_bf16(xbits), *args, N)
    _check(y, xbits, wdeq, chan)


@pytest.mark.parametrize("kind", ["int4", "mxfp4", "e4m3"])
@pytest.mark.parametrize("M", [1, 4])
@pytest.mark.parametrize("N,K", [(3205, 1024), (4795, 4096), (4105, 1024), (4097, 2048)])
def test_gemv_tile_rounds(W, kind, M, N, K):
    # With 256 CUs: 201 tiles of 16 columns (no half tiles, ragged last tile);
    # 300 tiles, whose last 44 become 88 tiles of 8 columns (the last one holds
    # 3 columns); 257 tiles, the last split in two (1 column in the second
    # half); 257 tiles with 1 column in the last (the second half tile is empty).
    g = np.random.default_rng(M * 7 + N + K)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[-3:] *= 30
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, kind, Wf)
    banner("gemv tile rounds", kind, M, N, K)
    y = W.wq_gemm(dev_bf16(xbits), *args, N)
    _check(y, xbits, wdeq, chan)


@pytest.mark.parametrize("kind,group,M,N,K", [
    ("int4", 128, 1, 8190, 2048),     # 512 tiles (2 per CU on 256 CUs), the last with 14 rows
    ("int4", 128, 3, 9001, 4096),     # 563 tiles: the last 51 become 102 tiles of 8 rows
    ("int4", 32, 4, 8200, 4096),      # 513 tiles: the last in two 8-row halves, the second empty
    ("int4", 64, 2, 16400, 8192),     # 16 steps per wave slice
    ("mxfp4", 32, 4, 14335, 4096),    # the decode workload's shape less one row
    ("int4", 128, 4, 8200, 14336),    # 28 steps per wave slice with x through the ring slots
    ("int4", 128, 2, 4097, 4096),     # 257 tiles, the last one with 1 row
    ("int4", 32, 1, 3205, 8192),
    ("int4", 64, 2, 17, 4096),        # one full tile of 16 rows and one of 1
    ("mxfp4", 32, 2, 4105, 8192),
    ("mxfp4", 32, 1, 14336, 4096),
    ("int4", 128, 1, 33000, 2048),    # 2063 tiles, 8 rounds over 256 CUs: the last 15 tiles become 30 halves
    ("int4", 128, 3, 40000, 1024),    # 2500 tiles, a last round of 196 kept as full tiles
])
def test_gemv_more_shapes(W, kind, group, M, N, K):
    # N from 17 to 40000 with ragged last tiles and balancing rounds of 8-row
    # tiles, K from 2048 to 14336, scale groups 32 to 128, M = 1-4
    g = np.random.default_rng(M * 11 + N + K + group)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, g.choice(K, 3, replace=False)] *= 40
    Wf[-2:] *= 30                                                # the ragged last tile
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, kind, Wf, group)
    del Wf
    banner("gemv more shapes", kind, group, M, N, K)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq, chan)


@pytest.mark.parametrize("group", [32, 64])
def test_gemv_int4_small_groups(W, group):
    g = np.random.default_rng(group)
    Wf = (g.standard_normal((300, 512)) * 0.02).astype(np.float32)
    xbits = to_bf16_bits(g.standard_normal((4, 512)).astype(np.float32))
    args, wdeq, chan = _prep(W, "int4", Wf, group)
    banner("gemv int4 group", group)
    _check(W.wq_gemm(dev_bf16(xbits), *args, 300), xbits, wdeq, chan)


@pytest.mark.parametrize("group", [32, 64])
@pytest.mark.parametrize("M", [1, 4])
def test_gemv_int4_small_groups_long_k(W, group, M):
    # K = 8192 with group 32: each row of a wave's slice holds 128 bytes of
    # scales, which take two staging loads per wave
    K, N = 8192, 272
    g = np.random.default_rng(group + 10 * M)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[g.choice(N, 20, replace=False)] *= 8                      # rows with their own scales
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, "int4", Wf, group)
    banner("gemv int4 group", group, "M", M, "K", K)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq, chan)


@pytest.mark.parametrize("form", ["short", "long", "mixed"])
@pytest.mark.parametrize("M,N,K", [(1, 14336, 4096), (3, 4795, 4096), (4, 4105, 1024), (1, 300, 512)])
def test_gemv_int4_scale_forms(W, form, M, N, K):
    # The quantizer stores scales with a 5-bit significand, for which the decode
    # multiplies the codes exactly and scales the group sums; any other bf16
    # scale in a step sends that step through the per-weight conversion.
    # "long": every scale gets nonzero low mantissa bits; "mixed": one group
    # in ten does, so waves switch between the two forms step by step.
    g = np.random.default_rng(M * 31 + N + K)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[g.choice(N, 7, replace=False)] *= 25
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    packed, sb, _ = OI.quantize_int4(Wf, 128)
    assert np.all(sb & 7 == 0)
    if form != "short":
        low = g.integers(1, 8, sb.shape).astype(np.uint16)
        if form == "mixed":
            low = np.where(g.random(sb.shape) < 0.1, low, 0).astype(np.uint16)
        sb = (sb | low).astype(np.uint16)
    banner("gemv int4 scales", form, M, N, K)
    y = W.wq_gemm(dev_bf16(xbits), dev_words(packed), W.WQ_INT4X8, dev_bf16(sb), W.WQ_BF16, 128, N)
    _check(y, xbits, OD.dequant_int4(packed, sb, 128), None)


def test_gemv_mxfp4_small_config(W):
    xbits, Wf = mxfp4_gemv_inputs(0)
    args, wdeq, chan = _prep(W, "mxfp4", Wf)
    banner("gemv mxfp4 1x512 . 1024x512")
    _check(W.wq_gemm(dev_bf16(xbits), *args, 1024), xbits, wdeq, chan)


@pytest.fixture(scope="module")
def decode_weights(W):
    _, Wf = decode_inputs(1, 0)
    return {k: _prep(W, k, Wf) for k in ("int4", "e4m3")}


@pytest.mark.parametrize("kind", ["int4", "e4m3"])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_full_size(W, decode_weights, kind, M):
    xbits, _ = decode_inputs(M, seed=10 + M, with_weight=False)
    args, wdeq, chan = decode_weights[kind]
    banner("decode full size", kind, "M", M)
    y = W.wq_gemm(dev_bf16(xbits), *args, 14336)
    y2 = W.wq_gemm(dev_bf16(xbits), *args, 14336)
    assert torch.equal(y, y2)                                       # fixed reduction order
    _check(y, xbits, wdeq, chan)


@pytest.mark.parametrize("M", [1, 4])
def test_decode_repeatable_with_cached_weights(W, decode_weights, M):
    # back-to-back launches over weights that stay in the last-level cache:
    # every launch must give the same bits (each ring slot is refilled only
    # after its reads have returned)
    xbits, _ = decode_inputs(M, seed=40 + M, with_weight=False)
    args, wdeq, chan = decode_weights["int4"]
    x = dev_bf16(xbits)
    banner("decode repeatable M", M)
    ys = [W.wq_gemm(x, *args, 14336) for _ in range(40)]
    for y in ys[1:]:
        assert torch.equal(y, ys[0])
    _check(ys[0], xbits, wdeq, chan)


@pytest.mark.parametrize("kind", ["int4", "mxfp4", "e4m3"])
@pytest.mark.parametrize("M", [20, 33, 64, 65, 100, 256])
def test_gemm_row_groups(W, kind, M):
    # 16 < M <= 64 runs the decode forms in launches of up to 32 rows (a last
    # launch of 1 and 32 rows); at this small N the decode launches also win
    # up to M = 256 (3, 4 and 8 launches, the last of 1, 4 and 32 rows)
    N, K = 1000, 2048
    g = np.random.default_rng(1500 + M)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, g.choice(K, 5, replace=False)] *= 30
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, kind, Wf)
    banner("gemm row groups", kind, M, N, K)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq, chan)


@pytest.mark.parametrize("kind", ["int4", "mxfp4", "e4m3"])
@pytest.mark.parametrize("M,N,K", [(256, 9000, 256), (129, 20000, 128), (65, 30000, 128)])
def test_gemm_mid_rows_prefill(W, kind, M, N, K):
    # 64 < M <= 256 at large N and short K, where the prefill grid fills the
    # CUs and the 256x256 kernel is the estimated faster path (ragged M tile
    # of 256, 129 and 65 rows)
    g = np.random.default_rng(1600 + M + N + K)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, g.choice(K, 3, replace=False)] *= 30
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, kind, Wf)
    banner("gemm mid rows prefill", kind, M, N, K)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq, chan)


@pytest.mark.parametrize("kind", ["int4", "mxfp4", "e4m3"])
@pytest.mark.parametrize("M,N,K", [(300, 520, 512), (17, 256, 256), (512, 512, 1024), (257, 33, 128)])
def test_gemm_ragged(W, kind, M, N, K):
    g = np.random.default_rng(M + N + K)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, kind, Wf)
    banner("gemm", kind, M, N, K)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq, chan)


@pytest.mark.parametrize("kind", ["mxfp4", "int4"])
def test_prefill_full_size_all_rows(W, kind):
    # the prefill workload (8192 x 4096 . 14336 x 4096, MXFP4 per 32 or INT4
    # per 128): every one of the 117 M outputs against the fp64 reference
    xbits, Wf = prefill_inputs(0)
    args, wdeq, chan = _prep(W, kind, Wf)
    banner("prefill full size", kind, "8192x4096 . 14336x4096, all rows")
    y = W.wq_gemm(dev_bf16(xbits), *args, 14336)
    check_all_rows(y, xbits, wdeq, chan)


@pytest.mark.parametrize("M", [1, 64])
def test_fp32_accumulation_all_ones(W, M):
    # K = 4096 ones: an fp32 accumulator gives exactly 4096; bf16 would stall at 256
    K, N = 4096, 64
    xbits = to_bf16_bits(np.ones((M, K), np.float32))
    codes = np.full((N, K), 0x38, np.uint8)                      # E4M3 1.0
    banner("accumulation all ones", M)
    y = W.wq_gemm(dev_bf16(xbits), dev_u8(codes), W.WQ_E4M3, dev_f32(np.ones(N, np.float32)), W.WQ_F32, K, N)
    assert np.all(bf16_decode(host_bits16(y)) == 4096.0)
    fp4 = np.full((N, K // 2), 0x22, np.uint8)                   # E2M1 1.0, 1.0
    y = W.wq_gemm(dev_bf16(xbits), dev_u8(fp4), W.WQ_E2M1X2, dev_u8(np.full((N, K // 32), 127, np.uint8)),
                  W.WQ_E8M0, 32, N)
    assert np.all(bf16_decode(host_bits16(y)) == 4096.0)


@pytest.mark.parametrize("M", [1, 3, 4])
def test_gemv_int4_zero_rows_and_groups(W, M):
    # all-zero weight rows must give exactly zero (the bound is zero there);
    # zeroed groups inside other rows must not disturb the rest
    K, N = 4096, 200
    g = np.random.default_rng(500 + M)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[::7] = 0.0
    Wf[3, 128:1024] = 0.0
    Wf[5, :128] = 0.0
    xbits = to_bf16_bits((g.standard_normal((M, K)) * 3).astype(np.float32))
    args, wdeq, chan = _prep(W, "int4", Wf)
    banner("gemv int4 zero rows", M)
    y = W.wq_gemm(dev_bf16(xbits), *args, N)
    _check(y, xbits, wdeq, chan)
    assert np.all(bf16_decode(host_bits16(y))[:, ::7] == 0.0)


@pytest.mark.parametrize("M", [1, 4])
def test_gemv_int4_offset_activations(W, M):
    # activations with a large common offset: sum_k x_k dominates every group
    K, N = 4096, 512
    g = np.random.default_rng(600 + M)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    xbits = to_bf16_bits((40.0 + g.standard_normal((M, K))).astype(np.float32))
    args, wdeq, chan = _prep(W, "int4", Wf)
    banner("gemv int4 offset x", M)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq, chan)


@pytest.mark.parametrize("kind", ["int4", "mxfp4", "e4m3"])
@pytest.mark.parametrize("M", [1, 3, 4])
def test_gemv_ring_28_steps(W, kind, M):
    # 28 ring steps per wave: K = 14336 for 4-bit weights (the MLP down
    # projection's K), 7168 for E4M3; 300 columns (ragged last tile)
    K = 7168 if kind == "e4m3" else 14336
    N = 300
    g = np.random.default_rng(1300 + M + K)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, g.choice(K, 6, replace=False)] *= 30
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, kind, Wf)
    banner("gemv ring 28 steps", kind, M, N, K)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq, chan)


@pytest.mark.parametrize("kind", ["int4", "mxfp4", "e4m3"])
@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("N,K", [(100, 11008), (70, 14336), (90, 640)])
def test_gemv_uneven_k_split(W, kind, M, N, K):
    # K whose step count the ring forms do not take (86, 112 or 5 steps of
    # 128 for 4-bit weights): the general GEMV splits the steps over up to 8
    # waves with shares differing by one chunk
    g = np.random.default_rng(1100 + M * 5 + N + K)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, g.choice(K, 4, replace=False)] *= 25
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, kind, Wf)
    banner("gemv uneven K split", kind, M, N, K)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq, chan)


@pytest.mark.parametrize("kind", ["int4", "mxfp4", "e4m3"])
@pytest.mark.parametrize("M", [5, 8, 13, 16])
@pytest.mark.parametrize("N,K", [(300, 2048), (1000, 4096), (64, 4096)])
def test_gemv_few_tiles_5_to_16(W, kind, M, N, K):
    # 5 <= M <= 16 with at most one 16-column tile per CU: one tile and up to
    # 16 waves per workgroup (ragged last tile, a single workgroup, every M
    # that leaves MFMA rows without a token)
    g = np.random.default_rng(900 + M * 3 + N + K)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, g.choice(K, 5, replace=False)] *= 30
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, kind, Wf)
    banner("gemv few tiles", kind, M, N, K)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq, chan)


@pytest.mark.parametrize("kind", ["int4", "mxfp4", "e4m3"])
@pytest.mark.parametrize("M", [17, 25, 32, 40, 64])
@pytest.mark.parametrize("N,K", [(1000, 2048), (4500, 1152)])
def test_gemv_32_rows(W, kind, M, N, K):
    # 16 < M <= 64 in launches of up to 32 rows: two 16-row groups share every
    # converted weight fragment, one 16-column tile per workgroup (N = 1000) or
    # two with at most 8 waves (N = 4500, ragged last workgroup); M = 40 and 64
    # take a second launch of 8 and 32 rows
    g = np.random.default_rng(990 + M * 3 + N + K)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, g.choice(K, 5, replace=False)] *= 30
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, kind, Wf)
    banner("gemv 32 rows", kind, M, N, K)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq, chan)


@pytest.mark.parametrize("kind", ["int4", "mxfp4", "e4m3"])
@pytest.mark.parametrize("M", [5, 11, 16])
@pytest.mark.parametrize("N,K", [(300, 14336), (70, 1152), (4500, 1536), (40, 640), (4100, 8192)])
def test_gemv_x_through_lds(W, kind, M, N, K):
    # 5 <= M <= 16 with x rows fetched whole and staged in LDS chunk by chunk,
    # the next chunk in flight: 7 chunks per wave at K = 14336 (odd count), one
    # chunk per wave at K = 1152 and 640 (9 and 5 waves); two 16-column tiles
    # per workgroup when the tiles outnumber the CUs, with a last workgroup of
    # 16 + 4 columns (N = 4500) or of 4 columns and an empty second tile
    # (N = 4100)
    g = np.random.default_rng(970 + M * 3 + N + K)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, g.choice(K, 5, replace=False)] *= 30
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, kind, Wf)
    banner("gemv x through lds", kind, M, N, K)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq, chan)


@pytest.mark.parametrize("kind", ["int4", "mxfp4", "e4m3"])
@pytest.mark.parametrize("M", [5, 16])
@pytest.mark.parametrize("N,K", [(4200, 2048), (4136, 4096), (9000, 4096), (16400, 2048)])
def test_gemv_x_once_per_workgroup(W, kind, M, N, K):
    # 5 <= M <= 16, more 16-column tiles than CUs, K = 2048 or 4096: x staged
    # once in LDS per 16-wave workgroup of up to 64 columns, as few as cover N
    # with one workgroup per CU (256 CUs: 24 columns at N = 4200 and 4136,
    # last workgroups of 24 and 8 columns; 40 at N = 9000, the last one whole;
    # 64 at N = 16400, a last workgroup of 16 columns)
    g = np.random.default_rng(950 + M * 3 + N + K)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, g.choice(K, 5, replace=False)] *= 30
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, kind, Wf)
    banner("gemv x once per workgroup", kind, M, N, K)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq, chan)


@pytest.mark.parametrize("kind", ["int4", "mxfp4"])
@pytest.mark.parametrize("M,N", [(1, 300), (4, 272)])
def test_gemv_long_k(W, kind, M, N):
    # K = 8192: 16 steps per wave; at M = 4 the workgroup needs more than 64 KB of LDS
    K = 8192
    g = np.random.default_rng(700 + M + N)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, kind, Wf)
    banner("gemv long K", kind, M, N, K)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq, chan)


def _random_cases(n, seed=2024):
    """Seeded random shapes over every dispatch range: M from 1 to 300 (the
    decode forms, launches of 32 rows and the prefill tiles), N from 1 to
    5000, K a multiple of 128 up to 5120, each format and INT4 group."""
    g = np.random.default_rng(seed)
    kinds = [("int4", 128), ("int4", 64), ("int4", 32), ("mxfp4", 32), ("e4m3", 0)]
    out = []
    while len(out) < n:
        M = int(np.exp(g.uniform(0, np.log(300))))
        N = int(g.integers(1, 5001))
        K = 128 * int(g.integers(1, 41))
        kind, group = kinds[len(out) % len(kinds)]
        if M * N * K > 1.5e9:
            continue
        out.append((kind, group, M, N, K, int(g.integers(1 << 30))))
    return out


@pytest.mark.parametrize("kind,group,M,N,K,seed", _random_cases(60))
def test_gemm_random_shapes(W, kind, group, M, N, K, seed):
    g = np.random.default_rng(seed)
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, g.choice(K, min(3, K), replace=False)] *= 40
    xbits = to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    args, wdeq, chan = _prep(W, kind, Wf, group or 128)
    banner("gemm random shape", kind, group, M, N, K, seed)
    _check(W.wq_gemm(dev_bf16(xbits), *args, N), xbits, wdeq, chan)
