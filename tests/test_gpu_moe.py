"""GPU parity of the W4A8 mixture-of-experts path (routing, grouping, scale
recipe, INT4 -> E4M3 tables, grouped fp8 GEMM) against the oracle.  Codes,
scales, ids and row maps are compared bit for bit; GEMM outputs with the bound
    |y - y_ref| <= 8e-3 |y_ref| + 1e-3 sum_k |x_k w_k|
against the fp64 product of the E4M3 operands.  Every checked output is
computed from oracle-produced inputs."""
import multiprocessing as mp
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import torch

from oracle import gemm as OG
from oracle import int4 as OI
from oracle import w4a8 as OW
from oracle.formats import bf16_decode, e4m3_decode
from synthetic import (moe_down_input_gpu, moe_expert_weight_gpu, moe_router_logits, moe_tokens, to_bf16_bits)
from tests import moe_workers
from tests.gpu_helpers import banner, dev_bf16, dev_f32, dev_u8, dev_words, host_bits16, host_f32, host_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def W():
    import weight_only_quantized_quant_amd as W
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return W


def _i32(t):
    return t.detach().cpu().numpy().astype(np.int64)


# ---------------------------------------------------------------------------
# routing and grouping
# ---------------------------------------------------------------------------
def _route_check(W, logits, k):
    E = logits.shape[1]
    ids_o, w_o = OW.route_topk(logits, k)
    off_o, rt_o, rs_o = OW.group_by_expert(ids_o, E)
    ids, wts, off, rt, rs = W.wq_moe_route(dev_f32(logits), k)
    assert np.array_equal(_i32(ids), ids_o)
    assert np.array_equal(_i32(off), off_o)
    assert np.array_equal(_i32(rt), rt_o)
    assert np.array_equal(_i32(rs), rs_o)
    np.testing.assert_allclose(host_f32(wts), w_o, rtol=1e-5, atol=0)


def test_route_full_size(W):
    banner("moe route 4096 tokens x 64 experts, top 8")
    _route_check(W, moe_router_logits(0), 8)


@pytest.mark.parametrize("T,E,k", [(37, 5, 2), (1000, 64, 8), (64, 64, 1), (5, 1, 1), (1025, 33, 3), (2050, 64, 64)])
def test_route_ties_and_shapes(W, T, E, k):
    g = np.random.default_rng(T * 100 + E + k)
    logits = (np.round(g.standard_normal((T, E)) * 2) / 2).astype(np.float32)   # many equal logits
    logits[0, :] = 0.0
    if T > 1:
        logits[1, ::2] = -0.0
    banner("moe route ties", T, E, k)
    _route_check(W, logits, k)


def test_route_no_tokens(W):
    banner("moe route T = 0")
    ids, wts, off, rt, rs = W.wq_moe_route(torch.empty((0, 4), dtype=torch.float32, device="cuda"), 2)
    assert np.array_equal(_i32(off), np.zeros(5, np.int64))


# ---------------------------------------------------------------------------
# scale recipe, re-layout, tables
# ---------------------------------------------------------------------------
def _relayout(words):
    w = np.asarray(words, dtype=np.uint64)
    o = np.zeros_like(w)
    for j in range(4):
        o |= ((w >> np.uint64(4 * j)) & np.uint64(0xF)) << np.uint64(8 * j)
        o |= ((w >> np.uint64(4 * j + 16)) & np.uint64(0xF)) << np.uint64(8 * j + 4)
    return o.astype(np.uint32)


def test_prepack_from_quantized_weights(W):
    g = np.random.default_rng(11)
    E, N, K = 3, 200, 1024
    packed, sbits = [], []
    for e in range(E):
        Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
        Wf[e, :] = 0.0                                       # an all-zero channel
        p, sb, _ = OI.quantize_int4(Wf, 128)
        packed.append(p)
        sbits.append(sb)
    packed, sbits = np.stack(packed), np.stack(sbits)
    banner("w4a8 prepack", E, N, K)
    wq2, s8, ch = W.wq_w4a8_prepack(dev_words(packed), dev_bf16(sbits))
    for e in range(E):
        s8_o, ch_o = OW.scale_recipe(sbits[e])
        assert np.array_equal(host_u8(s8[e]), s8_o)
        assert np.array_equal(host_f32(ch[e]).view(np.uint32), ch_o.astype(np.float32).view(np.uint32))
    assert np.array_equal(wq2.cpu().numpy().view(np.uint32), _relayout(packed))


def test_prepack_scale_edge_cases(W):
    g = np.random.default_rng(12)
    N, G = 64, 8
    s = (np.abs(g.standard_normal((N, G))) * 0.01).astype(np.float32)
    s[0] = 0.0                                               # all-zero channel -> ch = 8
    s[1, 3] = 0.0
    s[2] *= -1.0                                             # negative scales
    s[3] = np.float32(1e-30)
    s[4] = np.float32(3e30)
    s[5] = np.float32(2.0 ** -133)                           # bf16 subnormal
    s[6, :4] = np.float32(1e-6)                              # group scales far below the channel max
    sbits = to_bf16_bits(s)
    words = g.integers(0, 2 ** 32, size=(1, N, G * 16), dtype=np.uint64).astype(np.uint32)
    banner("w4a8 prepack edge scales")
    _, s8, ch = W.wq_w4a8_prepack(dev_words(words), dev_bf16(sbits[None]))
    s8_o, ch_o = OW.scale_recipe(sbits)
    assert np.array_equal(host_u8(s8[0]), s8_o)
    assert np.array_equal(host_f32(ch[0]).view(np.uint32), ch_o.astype(np.float32).view(np.uint32))


def _oracle_codes(packed, s8):
    q = OI.unpack_int4(packed).astype(np.int64)
    N, K = q.shape
    table = OW.lut(s8)
    return table[np.arange(N)[:, None], (np.arange(K) // 128)[None, :], q & 0xF]


def test_w4a8_table_codes_quantized_weights(W):
    g = np.random.default_rng(13)
    N, K = 300, 1024
    Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wf[:, g.choice(K, 4, replace=False)] *= 30
    packed, sb, _ = OI.quantize_int4(Wf, 128)
    s8, _ = OW.scale_recipe(sb)
    banner("w4a8 table codes, quantized weights")
    wq2 = dev_words(_relayout(packed))
    codes = W.wq_w4a8_dequant(wq2, dev_u8(s8))
    assert np.array_equal(host_u8(codes), _oracle_codes(packed, s8))


def test_w4a8_table_codes_every_scale_code(W):
    # every finite E4M3 scale code against every INT4 code (including -8)
    scodes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    N, K = len(scodes), 128
    q = np.tile(np.arange(-8, 8), (N, K // 16))
    packed = OI.pack_int4(q)
    s8 = scodes[:, None]
    banner("w4a8 table codes, all scale codes")
    codes = W.wq_w4a8_dequant(dev_words(_relayout(packed)), dev_u8(s8))
    assert np.array_equal(host_u8(codes), _oracle_codes(packed, s8))


# ---------------------------------------------------------------------------
# grouped GEMM, small configurations, every output checked
# ---------------------------------------------------------------------------
def _small_case(W, T, E, k, K, N, seed, identity=False):
    g = np.random.default_rng(seed)
    if identity:
        # the down-projection form: rows already grouped, one activation row each
        R = T
        cuts = np.sort(g.integers(0, R + 1, size=E - 1))
        offsets = np.concatenate([[0], cuts, [R]]).astype(np.int32)
        row_token = None
    else:
        ids, _ = OW.route_topk(g.standard_normal((T, E)).astype(np.float32), k)
        offsets, row_token, _ = OW.group_by_expert(ids, E)
        R = T * k
    xbits = to_bf16_bits(g.standard_normal((T, K)).astype(np.float32))
    x8, a_s = OW.quantize_tokens(xbits)
    experts, packed, sbits = [], [], []
    for e in range(E):
        Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
        p, sb, _ = OI.quantize_int4(Wf, 128)
        s8, ch = OW.scale_recipe(sb)
        experts.append((p, s8, ch))
        packed.append(p)
        sbits.append(sb)
    banner("moe gemm small", T, E, k, K, N, "identity" if identity else "gathered")
    wq2, s8d, chd = W.wq_w4a8_prepack(dev_words(np.stack(packed)), dev_bf16(np.stack(sbits)))
    rt = None if identity else torch.from_numpy(row_token.astype(np.int32)).cuda()
    y = W.wq_moe_gemm_w4a8(dev_u8(x8), dev_f32(a_s), rt, torch.from_numpy(offsets.astype(np.int32)).cuda(),
                           wq2, s8d, chd)
    yv = bf16_decode(host_bits16(y))
    rtok = np.arange(R) if identity else row_token
    ref, asum = OW.grouped_gemm_reference(x8, a_s, offsets, rtok, experts, 128)
    assert np.isfinite(yv).all()
    ratio = OG.worst_ratio(yv, ref, asum)
    assert ratio <= 1.0, f"worst error / bound = {ratio:.3f}"


# K > 4096 (more than 32 groups: the kernel reloads its LDS copy of the group
# scales every 32 steps), group counts that are and are not multiples of 4
# (dword or byte loads of the scales), and experts of 1..256+ rows (partial
# row tiles of every size class)
@pytest.mark.parametrize("T,E,k,K,N", [(300, 8, 2, 512, 384), (20, 16, 1, 256, 100), (600, 4, 4, 1024, 520),
                                       (1, 3, 2, 128, 33), (150, 3, 2, 8448, 72), (90, 2, 2, 4224, 40),
                                       (40, 2, 1, 5120, 64), (50, 3, 2, 640, 48)])
def test_moe_gemm_small(W, T, E, k, K, N):
    _small_case(W, T, E, k, K, N, seed=T + E + k + K + N)


def _random_moe_cases(n, seed=2027):
    """Seeded random configurations: 1-800 tokens, 1-16 experts, top-k 1-4,
    K a multiple of 128 up to 2560, N 1-600, gathered or already grouped rows."""
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(g.integers(1, 17))
        out.append((int(g.integers(1, 801)), E, int(g.integers(1, min(E, 4) + 1)), 128 * int(g.integers(1, 21)),
                    int(g.integers(1, 601)), bool(g.integers(0, 2)), int(g.integers(1 << 30))))
    return out


@pytest.mark.parametrize("T,E,k,K,N,identity,seed", _random_moe_cases(12))
def test_moe_gemm_random(W, T, E, k, K, N, identity, seed):
    _small_case(W, T, E, k, K, N, seed=seed, identity=identity)


def test_moe_gemm_subnormal_group_scales(W):
    # Groups whose INT4 scale sits ~10^4 below the channel's largest: their
    # fp8 scale (56 * s / max s) lands in the E4M3 subnormal range and so do
    # many table entries q * s8, which the fp8 matrix cores read as zero.  The
    # result must stay within the bound of the exact-operand reference; the
    # size of the flushed terms is printed for the record.
    g = np.random.default_rng(21)
    E, T, K, N = 2, 96, 512, 64
    R = T
    offsets = np.array([0, 40, R], np.int32)
    xbits = to_bf16_bits(g.standard_normal((T, K)).astype(np.float32))
    x8, a_s = OW.quantize_tokens(xbits)
    experts, packed, sbits = [], [], []
    for e in range(E):
        Wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
        Wf[:, 128:] *= 1e-4                                    # groups 1-3 of every row
        p, sb, _ = OI.quantize_int4(Wf, 128)
        s8, ch = OW.scale_recipe(sb)
        assert np.all((s8[:, 1:] & 0x78) == 0)                 # subnormal fp8 group scales
        experts.append((p, s8, ch))
        packed.append(p)
        sbits.append(sb)
    banner("moe gemm subnormal group scales")
    wq2, s8d, chd = W.wq_w4a8_prepack(dev_words(np.stack(packed)), dev_bf16(np.stack(sbits)))
    y = W.wq_moe_gemm_w4a8(dev_u8(x8), dev_f32(a_s), None, torch.from_numpy(offsets).cuda(), wq2, s8d, chd)
    yv = bf16_decode(host_bits16(y))
    ref, asum = OW.grouped_gemm_reference(x8, a_s, offsets, np.arange(R), experts, 128)
    ratio = OG.worst_ratio(yv, ref, asum)
    dev = float(np.max(np.abs(yv - ref) / np.maximum(asum, 1e-30)))
    print(f"[w4a8 subnormal group scales] worst error / bound {ratio:.4f}, max |y - ref| / sum|x w| {dev:.2e}",
          flush=True)
    assert np.isfinite(yv).all()
    assert ratio <= 1.0, f"worst error / bound = {ratio:.3f}"


def test_moe_gemm_clamps_device_offsets_and_tokens(W):
    # offsets and row_token are device data the host cannot validate: the
    # kernel clamps every expert's rows to [0, R] and reads a token index
    # outside [0, T) as a zero row.  A run with offsets[E] far past R and a
    # few bad token indices must match the well-formed run on every other row
    # and give zeros on the rows with bad tokens.
    g = np.random.default_rng(77)
    T, E, k, K, N = 200, 4, 2, 256, 96
    ids, _ = OW.route_topk(g.standard_normal((T, E)).astype(np.float32), k)
    offsets, row_token, _ = OW.group_by_expert(ids, E)
    R = T * k
    xbits = to_bf16_bits(g.standard_normal((T, K)).astype(np.float32))
    x8, a_s = OW.quantize_tokens(xbits)
    packed, sbits = [], []
    for e in range(E):
        p, sb, _ = OI.quantize_int4((g.standard_normal((N, K)) * 0.02).astype(np.float32), 128)
        packed.append(p)
        sbits.append(sb)
    wq2, s8d, chd = W.wq_w4a8_prepack(dev_words(np.stack(packed)), dev_bf16(np.stack(sbits)))
    bad_rows = np.array([0, 17, R - 1])
    rt_bad = row_token.astype(np.int32).copy()
    rt_bad[bad_rows] = [-5, T + 7, 2 ** 30]
    off_bad = offsets.astype(np.int32).copy()
    off_bad[E] = R + 100000
    banner("moe gemm clamps offsets and token indices")
    args = (dev_u8(x8), dev_f32(a_s))
    y_ok = W.wq_moe_gemm_w4a8(*args, torch.from_numpy(row_token.astype(np.int32)).cuda(),
                              torch.from_numpy(offsets.astype(np.int32)).cuda(), wq2, s8d, chd)
    y_bad = W.wq_moe_gemm_w4a8(*args, torch.from_numpy(rt_bad).cuda(), torch.from_numpy(off_bad).cuda(),
                               wq2, s8d, chd)
    torch.cuda.synchronize()
    a, b = host_bits16(y_ok), host_bits16(y_bad)
    keep = np.setdiff1d(np.arange(R), bad_rows)
    assert np.array_equal(a[keep], b[keep])
    assert np.all(bf16_decode(b[bad_rows]) == 0.0)


@pytest.mark.parametrize("T,E,K,N", [(700, 5, 384, 300), (64, 64, 256, 64)])
def test_moe_gemm_identity_rows(W, T, E, K, N):
    _small_case(W, T, E, 1, K, N, seed=T * 3 + E, identity=True)


# ---------------------------------------------------------------------------
# full size (64 experts, 4096 tokens, top 8), sampled rows
# ---------------------------------------------------------------------------
def _checked_rows(lo, hi):
    """First and last grouped row of an expert and the rows on both sides of
    each of its 256-row tile boundaries."""
    rows = {lo, hi - 1}
    for b in range(lo + 256, hi, 256):
        rows |= {b - 1, b}
    return np.array(sorted(r for r in rows if lo <= r < hi))


def _full_size(W, which, pool):
    E, T, k, hidden, inter = 64, 4096, 8, 4096, 1536
    N, K = (2 * inter, hidden) if which == "gate_up" else (hidden, inter)
    ids, _ = OW.route_topk(moe_router_logits(0), k)
    offsets, row_token, _ = OW.group_by_expert(ids, E)
    R = T * k
    # activations: every row quantized on the GPU, the rows the checked outputs
    # read replaced by the oracle's
    if which == "gate_up":
        xb = moe_tokens()
        x_dev = dev_bf16(xb)
    else:
        x_dev = moe_down_input_gpu(rows=R, inter=inter)
    x8, a_s = W.quantize_e4m3(x_dev, -1)
    a_s = a_s.reshape(-1).contiguous()
    sampled = {e: _checked_rows(int(offsets[e]), int(offsets[e + 1])) for e in range(E)
               if offsets[e + 1] > offsets[e]}
    xrows = {}
    for e, rows in sampled.items():
        toks = row_token[rows] if which == "gate_up" else rows
        bits = xb[toks] if which == "gate_up" else host_bits16(x_dev[torch.from_numpy(toks).cuda()])
        c, s = moe_workers.token_rows(bits)
        x8[torch.from_numpy(toks).cuda()] = dev_u8(c)
        a_s[torch.from_numpy(toks).cuda()] = dev_f32(s)
        xrows[e] = (c, s)
    # weights: GPU-generated, every expert quantized by the oracle (in worker
    # processes), so that every checked output comes from oracle-made inputs
    banner("moe full size", which, "weights of", E, "experts")
    packed = torch.empty((E, N, K // 8), dtype=torch.int32, device="cuda")
    sbits = torch.empty((E, N, K // 128), dtype=torch.bfloat16, device="cuda")
    futures = {}
    for e in range(E):
        Wf = moe_expert_weight_gpu(e, which)
        if e in sampled:
            futures[e] = pool.submit(moe_workers.expert_case, Wf.cpu().numpy(), *xrows[e])
        else:
            W.quantize_int4(Wf, 128, packed=packed[e], scales=sbits[e])
    results = {e: f.result() for e, f in futures.items()}
    for e, (p, sb, _, _, _, _) in results.items():
        packed[e] = dev_words(p)
        sbits[e] = dev_bf16(sb)
    banner("moe full size", which, "prepack + grouped GEMM", R, N, K)
    wq2, s8, ch = W.wq_w4a8_prepack(packed, sbits)
    rt = torch.from_numpy(row_token.astype(np.int32)).cuda() if which == "gate_up" else None
    if which == "down":
        assert R == T * k
    y = W.wq_moe_gemm_w4a8(x8, a_s, rt, torch.from_numpy(offsets.astype(np.int32)).cuda(), wq2, s8, ch)
    torch.cuda.synchronize()
    worst, nrows = 0.0, 0
    for e, rows in sampled.items():
        _, _, s8_o, ch_o, ref, asum = results[e]
        assert np.array_equal(host_u8(s8[e]), s8_o)
        assert np.array_equal(host_f32(ch[e]).view(np.uint32), ch_o.astype(np.float32).view(np.uint32))
        yv = bf16_decode(host_bits16(y[torch.from_numpy(rows).cuda()]))
        assert np.isfinite(yv).all()
        worst = max(worst, OG.worst_ratio(yv, ref, asum))
        nrows += len(rows)
    assert len(sampled) == E and nrows >= 4 * E
    assert worst <= 1.0, f"worst error / bound = {worst:.3f}"


@pytest.fixture(scope="module")
def pool():
    with ProcessPoolExecutor(max_workers=8, mp_context=mp.get_context("spawn")) as ex:
        yield ex


@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_moe_full_size_every_expert(W, pool, which):
    _full_size(W, which, pool)
