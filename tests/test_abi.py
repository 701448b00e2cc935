"""The C-ABI library loads and exports every entry point the headers under
include/ declare; invalid arguments are rejected on the host before any launch
(CPU only)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
LIB = os.path.join(ROOT, "weight_only_quantized_quant_amd", "libwq.so")


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libwq.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("quantize_e4m3", "quantize_mxfp4", "quantize_mx", "quantize_nvfp4", "quantize_int4", "quantize_int4_asym", "wq_dequant", "wq_gemm",
              "wq_gemm_workspace_size", "wq_status_string", "wq_moe_route", "wq_w4a8_prepack",
              "wq_w4a8_dequant", "wq_moe_gemm_w4a8", "quantize_e4m3_static", "quantize_e4m3_block2d",
              "wq_gemm_w8a8", "wq_util_stream_read", "wq_util_spin", "wq_util_clock",
              "wq_util_wall_clock_khz"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    lib.wq_status_string.restype = ctypes.c_char_p
    for code in range(5):
        assert lib.wq_status_string(code).startswith(b"WQ_")
    assert b"unknown" in lib.wq_status_string(99)


def test_binding_exposes_the_same_names():
    import weight_only_quantized_quant_amd as W
    for name in declared_functions():
        assert callable(getattr(W, name)), name


def _i64(v):
    return ctypes.c_int64(v)


def test_invalid_arguments_rejected_before_launch(lib):
    f = lib.quantize_e4m3
    f.restype = ctypes.c_int
    p = ctypes.c_void_p(0x1000)          # never dereferenced: validation fails first
    q = ctypes.c_void_p(0x1008)          # misaligned
    # NULL input, bad shapes, odd columns
    assert f(None, 1, _i64(4), _i64(64), 0, p, None, None) == 1
    assert f(p, 1, _i64(0), _i64(64), 0, p, None, None) == 1
    assert f(p, 1, _i64(4), _i64(12), 0, p, None, None) == 1
    assert f(p, 7, _i64(4), _i64(64), 0, p, None, None) == 3          # unsupported dtype
    assert f(q, 1, _i64(4), _i64(64), 0, p, None, None) == 2          # misaligned
    assert f(p, 1, _i64(4), _i64(64), 48, p, p, None) == 3            # unsupported block
    assert f(p, 1, _i64(4), _i64(64), 128, p, p, None) == 1           # cols % block
    assert f(p, 1, _i64(4), _i64(64), 32, p, None, None) == 1         # scales needed
    g = lib.quantize_mxfp4
    g.restype = ctypes.c_int
    assert g(p, 0, _i64(4), _i64(64), 8, p, p, None) == 3
    assert g(p, 0, _i64(4), _i64(48), 32, p, p, None) == 1
    m = lib.quantize_mx
    m.restype = ctypes.c_int
    assert m(p, 0, _i64(4), _i64(64), 32, 4, 0, p, p, None) == 3          # E8M0 is no element format
    assert m(p, 0, _i64(4), _i64(64), 32, 2, 5, p, p, None) == 1          # unknown rule
    assert m(p, 0, _i64(4), _i64(64), 32, 3, -1, p, p, None) == 1
    assert m(p, 0, _i64(4), _i64(64), 64, 2, 0, p, p, None) == 3          # block
    assert m(p, 0, _i64(4), _i64(48), 16, 2, 0, p, p, None) == 1          # cols % 32
    assert m(p, 0, _i64(4), _i64(64), 32, 2, 0, p, None, None) == 1       # scales NULL
    assert m(q, 0, _i64(4), _i64(64), 32, 3, 4, p, p, None) == 2          # misaligned
    h = lib.quantize_int4
    h.restype = ctypes.c_int
    assert h(p, 0, _i64(4), _i64(128), 96, p, p, None) == 3
    assert h(p, 0, _i64(4), _i64(96), 64, p, p, None) == 1
    d = lib.wq_dequant
    d.restype = ctypes.c_int
    assert d(p, 5, p, 0, 128, _i64(4), _i64(128), p, None) == 3       # int4 needs bf16 scales
    assert d(p, 9, p, 1, 128, _i64(4), _i64(128), p, None) == 3
    assert d(p, 5, p, 1, 128, _i64(4), _i64(100), p, None) == 1
    gm = lib.wq_gemm
    gm.restype = ctypes.c_int
    args = lambda M, N, K, wdt, sdt, grp, x=p, a=1.0: (x, _i64(M), _i64(N), _i64(K), p, wdt, p, sdt, grp,
                                                      ctypes.c_float(a), p, None, ctypes.c_size_t(0), None)
    assert gm(*args(1, 16, 100, 5, 1, 128)) == 1                        # K % 128
    # K a multiple of the group but not of 128: rejected for every format
    assert gm(*args(1, 16, 96, 5, 1, 32)) == 1                          # INT4 group 32
    assert gm(*args(4, 16, 192, 5, 1, 64)) == 1                         # INT4 group 64
    assert gm(*args(1, 16, 160, 3, 4, 32)) == 1                         # MXFP4 block 32
    assert gm(*args(300, 16, 224, 6, 7, 32)) == 1                       # asymmetric INT4, prefill rows
    assert gm(*args(0, 16, 128, 5, 1, 128)) == 1
    assert gm(*args(1, 16, 128, 5, 1, 96)) == 3                         # bad group
    assert gm(*args(1, 16, 128, 3, 1, 32)) == 3                         # fp4 needs E8M0
    assert gm(*args(1, 16, 256, 2, 0, 128)) == 3                        # e4m3 needs group == K
    assert gm(*args(1, 16, 128, 5, 1, 128, x=q)) == 2
    assert gm(*args(1, 16, 128, 3, 2, 32)) == 3                         # NVFP4 needs group 16
    assert gm(*args(1, 16, 128, 3, 2, 16, a=float("nan"))) == 1         # alpha must be finite
    assert gm(*args(1, 16, 128, 3, 2, 16, a=float("inf"))) == 1
    nv = lib.quantize_nvfp4
    nv.restype = ctypes.c_int
    assert nv(p, 0, _i64(4), _i64(24), ctypes.c_float(1.0), p, p, None) == 1   # cols % 16
    assert nv(p, 0, _i64(4), _i64(32), ctypes.c_float(0.0), p, p, None) == 1   # tensor scale > 0
    assert nv(p, 0, _i64(4), _i64(32), ctypes.c_float(-1.0), p, p, None) == 1
    assert nv(p, 0, _i64(4), _i64(32), ctypes.c_float(float("inf")), p, p, None) == 1
    assert nv(p, 5, _i64(4), _i64(32), ctypes.c_float(1.0), p, p, None) == 3
    assert nv(q, 0, _i64(4), _i64(32), ctypes.c_float(1.0), p, p, None) == 2
    assert d(p, 3, p, 2, 32, _i64(4), _i64(128), p, None) == 3       # NVFP4 dequant needs group 16
    assert d(p, 6, p, 1, 128, _i64(4), _i64(128), p, None) == 3      # asymmetric INT4 needs scale-zero words
    assert d(p, 6, p, 7, 96, _i64(4), _i64(192), p, None) == 3
    assert gm(*args(1, 16, 128, 6, 1, 128)) == 3
    assert gm(*args(1, 16, 128, 6, 7, 48)) == 3
    ia = lib.quantize_int4_asym
    ia.restype = ctypes.c_int
    assert ia(p, 0, _i64(4), _i64(128), 96, p, p, None) == 3
    assert ia(p, 0, _i64(4), _i64(96), 64, p, p, None) == 1
    assert ia(p, 0, _i64(4), _i64(128), 64, p, None, None) == 1
    assert ia(q, 0, _i64(4), _i64(128), 64, p, p, None) == 2
    lib.wq_gemm_workspace_size.restype = ctypes.c_size_t
    assert lib.wq_gemm_workspace_size(_i64(1), _i64(16), _i64(128), 5, 128) == 0



def test_w8a8_invalid_arguments_rejected_before_launch(lib):
    p = ctypes.c_void_p(0x1000)
    q = ctypes.c_void_p(0x1004)          # misaligned for 16-byte data, aligned for fp32 scales
    st = lib.quantize_e4m3_static
    st.restype = ctypes.c_int
    assert st(p, 1, _i64(4), _i64(24), p, p, None) == 1                  # cols % 16
    assert st(p, 1, _i64(4), _i64(32), None, p, None) == 1               # scale pointer
    assert st(p, 4, _i64(4), _i64(32), p, p, None) == 3
    assert st(q, 1, _i64(4), _i64(32), p, p, None) == 2
    bl = lib.quantize_e4m3_block2d
    bl.restype = ctypes.c_int
    assert bl(p, 0, _i64(300), _i64(200), p, p, None) == 1               # cols % 128
    assert bl(p, 0, _i64(0), _i64(256), p, p, None) == 1
    assert bl(p, 0, _i64(300), _i64(256), q, p, None) == 2
    g = lib.wq_gemm_w8a8
    g.restype = ctypes.c_int
    args = lambda M, N, K, gn=128, bsk=1, ask=1, a=p: (a, p, _i64(K // 128), _i64(ask), p, p, _i64(K // 128),
                                                       _i64(bsk), gn, _i64(M), _i64(N), _i64(K), p, None)
    assert g(*args(16, 256, 200)) == 1                                  # K % 128
    assert g(*args(0, 256, 256)) == 1
    assert g(*args(16, 256, 256, gn=64)) == 3                           # block of 128 channels or per channel
    assert g(*args(16, 256, 256, gn=1, bsk=1)) == 3                     # per-channel scales cannot depend on K
    assert g(*args(16, 256, 256, ask=-1)) == 1
    assert g(*args(16, 256, 256, a=q)) == 2


def test_moe_invalid_arguments_rejected_before_launch(lib):
    p = ctypes.c_void_p(0x1000)
    q = ctypes.c_void_p(0x1004)          # misaligned
    r = lib.wq_moe_route
    r.restype = ctypes.c_int
    assert r(p, _i64(16), 65, 8, p, p, p, p, p, None) == 1               # more than 64 experts
    assert r(p, _i64(16), 8, 9, p, p, p, p, p, None) == 1                # k > E
    assert r(p, _i64(16), 8, 0, p, p, p, p, p, None) == 1
    assert r(p, _i64(-1), 8, 2, p, p, p, p, p, None) == 1
    assert r(p, _i64(16), 8, 2, p, p, None, p, p, None) == 1             # offsets NULL
    pk = lib.wq_w4a8_prepack
    pk.restype = ctypes.c_int
    assert pk(p, p, _i64(2), _i64(16), _i64(100), p, p, p, None) == 1   # K % 128
    assert pk(p, p, _i64(0), _i64(16), _i64(128), p, p, p, None) == 1
    assert pk(q, p, _i64(2), _i64(16), _i64(128), p, p, p, None) == 2
    assert pk(p, None, _i64(2), _i64(16), _i64(128), p, p, p, None) == 1
    dq = lib.wq_w4a8_dequant
    dq.restype = ctypes.c_int
    assert dq(p, p, _i64(4), _i64(64), p, None) == 1
    gm = lib.wq_moe_gemm_w4a8
    gm.restype = ctypes.c_int
    args = lambda T, R, K, rt=p, x=p: (x, _i64(T), p, rt, _i64(R), p, 4, _i64(64), _i64(K), p, p, p, p, None)
    assert gm(*args(16, 32, 100)) == 1                                   # K % 128
    assert gm(*args(16, 32, 128, rt=None)) == 1                          # identity rows need R == T
    assert gm(*args(16, 32, 128, x=q)) == 2
    assert gm(*args(0, 0, 128)) == 1


def test_utilities_reject_bad_arguments(lib):
    sr = lib.wq_util_stream_read
    sr.restype = ctypes.c_int
    sr.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    fake = 1 << 20                                       # never dereferenced: rejected on the host
    assert sr(None, 1024, 0, fake, None) == 1
    assert sr(fake, 0, 0, fake, None) == 1
    assert sr(fake, 1000, 0, fake, None) == 1            # not a multiple of 16
    assert sr(fake, 1024, 0, None, None) == 1
    assert sr(fake + 8, 1024, 0, fake, None) == 2        # misaligned
    sp = lib.wq_util_spin
    sp.restype = ctypes.c_int
    sp.argtypes = [ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    assert sp(0, 0, fake, None) == 1
    assert sp((1 << 24) + 1, 0, fake, None) == 1
    assert sp(100, 0, None, None) == 1
    ck = lib.wq_util_clock
    ck.restype = ctypes.c_int
    ck.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    assert ck(0, fake, None) == 1
    assert ck((1 << 20) + 1, fake, None) == 1
    assert ck(200, None, None) == 1
    assert ck(200, fake + 8, None) == 2
    wk = lib.wq_util_wall_clock_khz
    wk.restype = ctypes.c_int
    wk.argtypes = [ctypes.c_void_p]
    assert wk(None) == 1
