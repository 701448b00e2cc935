"""Captured HIP-graph replays of the library's launches (the form the decode
benchmark times) reproduce the eager results bit for bit, on every replay,
with eager launches and host synchronisation between the replays.  The eager
results themselves are checked against the oracle by the other GPU tests;
here only replay == eager is asserted (both run the same kernels on the same
inputs, and every kernel is deterministic)."""
import numpy as np
import pytest
import torch

from oracle import e4m3 as OE
from oracle import int4 as OI
from oracle import mxfp4 as OM
from oracle import w4a8 as OW
from oracle import w8a8 as O8
from synthetic import decode_inputs, prefill_inputs, to_bf16_bits
from tests.gpu_helpers import banner, dev_bf16, dev_f32, dev_u8, dev_words

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def W():
    import weight_only_quantized_quant_amd as W
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return W


def _weights(W, kind, Wf):
    """Device weight arguments of wq_gemm, quantized by the oracle."""
    if kind == "int4":
        packed, sb, _ = OI.quantize_int4(Wf, 128)
        return dev_words(packed), W.WQ_INT4X8, dev_bf16(sb), W.WQ_BF16, 128
    if kind == "mxfp4":
        codes, sc = OM.quantize_mxfp4(Wf, 32)
        return dev_u8(codes), W.WQ_E2M1X2, dev_u8(sc), W.WQ_E8M0, 32
    codes, s = OE.quantize_e4m3(Wf, -1)
    return dev_u8(codes), W.WQ_E4M3, dev_f32(s[:, 0]), W.WQ_F32, Wf.shape[1]


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.uint8)


def _replay_matches(fill, eager_fn, capture_fn, outs, refs, interleave):
    """Capture capture_fn (writing outs), replay it REPLAYS times with outs
    overwritten, interleave() run eagerly and the host synchronised before
    each replay, and compare every replay with refs bit for bit."""
    eager_fn()                                   # warm: attributes set outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture_fn()
    for r in range(REPLAYS):
        for o in outs:
            o.view(torch.uint8).fill_(fill + r)
        interleave()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert torch.equal(_bits(o), _bits(ref)), f"replay {r} differs from the eager result"


@pytest.mark.parametrize("kind,M,N,K", [
    ("int4", 1, 14336, 4096),      # split-K ring
    ("int4", 4, 4105, 4096),       # ring with x in the slots, ragged N
    ("int4", 16, 14336, 4096),     # x-once workgroups
    ("e4m3", 1, 4096, 4096),       # weights straight into registers
    ("mxfp4", 3, 1000, 2048),      # ring, 3 tokens
    ("int4", 300, 520, 512),       # prefill GEMM, ragged tiles
    ("mxfp4", 40, 700, 1024),      # 17-64 rows: grouped decode launches
])
def test_gemm_graph_replays(W, kind, M, N, K):
    banner("graph replay wq_gemm", kind, M, N, K)
    if M <= 16:
        xbits, Wf = decode_inputs(M, K=K, N=N, seed=11)
    else:
        xbits, Wf = prefill_inputs(seed=11, M=M, K=K, N=N)
    x = dev_bf16(xbits)
    wq, wdt, sc, sdt, group = _weights(W, kind, Wf)
    ref = W.wq_gemm(x, wq, wdt, sc, sdt, group, N)
    torch.cuda.synchronize()
    y = torch.empty_like(ref)
    other = torch.empty_like(ref)
    _replay_matches(
        0x11,
        lambda: W.wq_gemm(x, wq, wdt, sc, sdt, group, N, y=y),
        lambda: W.wq_gemm(x, wq, wdt, sc, sdt, group, N, y=y),
        [y], [ref],
        lambda: W.wq_gemm(x, wq, wdt, sc, sdt, group, N, y=other))


def test_quantizer_graph_replays(W):
    banner("graph replay quantizers 300 x 512")
    rng = np.random.default_rng(5)
    a = torch.from_numpy(rng.standard_normal((300, 512)).astype(np.float32)).cuda().to(torch.bfloat16)
    c4, s4 = W.quantize_mxfp4(a, 32)
    c8, s8 = W.quantize_e4m3(a, 128)
    torch.cuda.synchronize()
    oc4, os4, oc8, os8 = (torch.empty_like(t) for t in (c4, s4, c8, s8))

    def run():
        W.quantize_mxfp4(a, 32, codes=oc4, scales=os4)
        W.quantize_e4m3(a, 128, codes=oc8, scales=os8)

    _replay_matches(0x5A, run, run, [oc4, os4, oc8, os8], [c4, s4, c8, s8],
                    lambda: W.quantize_e4m3(a, -1))


def test_w8a8_graph_replays(W):
    banner("graph replay wq_gemm_w8a8 300 x 520 x 512, 1x128 x 128x128 scales")
    g = np.random.default_rng(3)
    M, N, K = 300, 520, 512
    kb = K // 128
    ac, sa = OE.quantize_e4m3(g.standard_normal((M, K)).astype(np.float32), 128)
    bc, sb = O8.quantize_e4m3_block2d((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    a, a_s, b, b_s = dev_u8(ac), dev_f32(sa), dev_u8(bc), dev_f32(sb)
    ref = W.wq_gemm_w8a8(a, a_s, kb, 1, b, b_s, kb, 1, 128)
    torch.cuda.synchronize()
    y, other = torch.empty_like(ref), torch.empty_like(ref)
    run = lambda: W.wq_gemm_w8a8(a, a_s, kb, 1, b, b_s, kb, 1, 128, y=y)
    _replay_matches(0x33, run, run, [y], [ref], lambda: W.wq_gemm_w8a8(a, a_s, kb, 1, b, b_s, kb, 1, 128, y=other))


def test_moe_graph_replays(W):
    """Routing, grouping and the grouped W4A8 GEMM in one graph: the offsets
    and row map stay on the device between the launches."""
    banner("graph replay moe route + w4a8 gemm: T 64, E 8, k 2, K 512, N 256")
    g = np.random.default_rng(4)
    T, E, k, K, N = 64, 8, 2, 512, 256
    logits = torch.from_numpy(g.standard_normal((T, E)).astype(np.float32)).cuda()
    x8, a_s = OW.quantize_tokens(to_bf16_bits(g.standard_normal((T, K)).astype(np.float32)))
    x8d, a_sd = dev_u8(x8), dev_f32(a_s)
    packed, sbits = [], []
    for _ in range(E):
        p, sb, _ = OI.quantize_int4((g.standard_normal((N, K)) * 0.02).astype(np.float32), 128)
        packed.append(p)
        sbits.append(sb)
    wq2, s8d, chd = W.wq_w4a8_prepack(dev_words(np.stack(packed)), dev_bf16(np.stack(sbits)))
    ids_r, _, off_r, rt_r, _ = W.wq_moe_route(logits, k)
    ref = W.wq_moe_gemm_w4a8(x8d, a_sd, rt_r, off_r, wq2, s8d, chd)
    torch.cuda.synchronize()
    y = torch.empty_like(ref)
    held = {}

    def run():
        ids, _, off, rt, _ = W.wq_moe_route(logits, k)
        held.update(ids=ids, off=off)
        W.wq_moe_gemm_w4a8(x8d, a_sd, rt, off, wq2, s8d, chd, y=y)

    _replay_matches(0x44, run, run, [y], [ref], lambda: W.wq_moe_route(logits, k))
    assert torch.equal(held["ids"], ids_r) and torch.equal(held["off"], off_r)


def test_launches_follow_the_callers_stream(W):
    """Every entry point enqueues on the stream current at the call: a decode
    GEMV and a quantizer issued on a side stream (default priority), behind a
    busy kernel on that stream, are complete and equal to the default-stream
    results once that stream alone has been synchronised."""
    banner("side-stream launches: wq_gemm int4 M=2 and quantize_mxfp4")
    xbits, Wf = decode_inputs(2, K=2048, N=3000, seed=13)
    x = dev_bf16(xbits)
    wq, wdt, sc, sdt, group = _weights(W, "int4", Wf)
    a = x.float().repeat(8, 1).to(torch.bfloat16).contiguous()
    ref_y = W.wq_gemm(x, wq, wdt, sc, sdt, group, 3000)
    ref_c, ref_s = W.quantize_mxfp4(a, 32)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    y = torch.full_like(ref_y, 7.0)
    c, s = torch.zeros_like(ref_c), torch.zeros_like(ref_s)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        W.wq_util_spin(200000)
        W.wq_gemm(x, wq, wdt, sc, sdt, group, 3000, y=y)
        W.quantize_mxfp4(a, 32, codes=c, scales=s)
    side.synchronize()
    assert torch.equal(_bits(y), _bits(ref_y))
    assert torch.equal(c, ref_c) and torch.equal(s, ref_s)
