"""MI355X (gfx950) block-scaled quantizers and weight-only quantized matmul.

Thin Python binding over the C ABI of ``libwq.so`` (declared in include/wq.h).
The functions here carry the same names as the C entry points and only
marshal arguments: they check devices, dtypes, shapes and contiguity of
PyTorch tensors, allocate outputs with PyTorch when none are given, and pass
raw device pointers plus the current HIP stream.  Every step of the
computation runs in the HIP kernels; there is no other code path.  If the
library has not been built the import fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwq.so")

# dtype enum of the C ABI
WQ_F32, WQ_BF16, WQ_E4M3, WQ_E2M1X2, WQ_E8M0, WQ_INT4X8, WQ_UINT4X8, WQ_BF16Z = range(8)
WQ_OK, WQ_EINVAL, WQ_EALIGN, WQ_EUNSUPPORTED, WQ_EHIP = range(5)
# E8M0 scale rules of quantize_mx (wq_mx_rule)
MX_RULES = {"round": 0, "half": 1, "ocp": 2, "floor_div": 3, "ceil_div": 4}
MX_ELEMS = {"e2m1": WQ_E2M1X2, "e4m3": WQ_E4M3}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python weight_only_quantized_quant_amd/build.py` "
        "(hipcc, gfx950). There is no fallback path.")

lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_SIGS = {
    "wq_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "quantize_e4m3": ([_vp, ctypes.c_int, _i64, _i64, _i32, _vp, _vp, _vp], ctypes.c_int),
    "quantize_mxfp4": ([_vp, ctypes.c_int, _i64, _i64, _i32, _vp, _vp, _vp], ctypes.c_int),
    "quantize_nvfp4": ([_vp, ctypes.c_int, _i64, _i64, ctypes.c_float, _vp, _vp, _vp], ctypes.c_int),
    "quantize_mx": ([_vp, ctypes.c_int, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp], ctypes.c_int),
    "quantize_int4": ([_vp, ctypes.c_int, _i64, _i64, _i32, _vp, _vp, _vp], ctypes.c_int),
    "quantize_int4_asym": ([_vp, ctypes.c_int, _i64, _i64, _i32, _vp, _vp, _vp], ctypes.c_int),
    "wq_dequant": ([_vp, ctypes.c_int, _vp, ctypes.c_int, _i32, _i64, _i64, _vp, _vp], ctypes.c_int),
    "wq_gemm": ([_vp, _i64, _i64, _i64, _vp, ctypes.c_int, _vp, ctypes.c_int, _i32, ctypes.c_float, _vp, _vp, _sz,
                 _vp], ctypes.c_int),
    "wq_gemm_workspace_size": ([_i64, _i64, _i64, ctypes.c_int, _i32], _sz),
    "quantize_e4m3_static": ([_vp, ctypes.c_int, _i64, _i64, _vp, _vp, _vp], ctypes.c_int),
    "quantize_e4m3_block2d": ([_vp, ctypes.c_int, _i64, _i64, _vp, _vp, _vp], ctypes.c_int),
    "wq_gemm_w8a8": ([_vp, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _i32, _i64, _i64, _i64, _vp, _vp], ctypes.c_int),
    "wq_moe_route": ([_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "wq_w4a8_prepack": ([_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp], ctypes.c_int),
    "wq_w4a8_dequant": ([_vp, _vp, _i64, _i64, _vp, _vp], ctypes.c_int),
    "wq_moe_gemm_w4a8": ([_vp, _i64, _vp, _vp, _i64, _vp, _i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "wq_util_stream_read": ([_vp, _i64, ctypes.c_uint32, _vp, _vp], ctypes.c_int),
    "wq_util_spin": ([_i64, ctypes.c_uint32, _vp, _vp], ctypes.c_int),
    "wq_util_clock": ([_i64, _vp, _vp], ctypes.c_int),
    "wq_util_wall_clock_khz": ([ctypes.POINTER(ctypes.c_int)], ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


class WQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib.wq_status_string(status).decode()}")


def _check(status: int, where: str) -> None:
    if status == WQ_OK:
        return
    if status in (WQ_EINVAL, WQ_EALIGN, WQ_EUNSUPPORTED):
        err = WQError(status, where)
        raise ValueError(str(err)) from err
    raise WQError(status, where)


def wq_status_string(status: int) -> str:
    return lib.wq_status_string(status).decode()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _x_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return WQ_F32
    if x.dtype == torch.bfloat16:
        return WQ_BF16
    raise ValueError("input must be float32 or bfloat16")


def _out(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _dev(t, name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}")
    return t


def quantize_e4m3(x: torch.Tensor, block: int, codes=None, scales=None):
    """x: 2-D fp32/bf16.  block 0 (plain cast), >0 (per 1 x block) or -1 (per row).
    Returns (codes uint8 [rows, cols], scales fp32 [rows, groups] or None)."""
    _dev(x, "x")
    rows, cols = x.shape
    codes = _out(codes, (rows, cols), torch.uint8, x.device, "codes")
    if block == 0:
        scales_ptr = None
    else:
        groups = 1 if block == -1 else (cols // block if block > 0 else 0)
        scales = _out(scales, (rows, groups), torch.float32, x.device, "scales")
        scales_ptr = scales.data_ptr()
    _check(lib.quantize_e4m3(x.data_ptr(), _x_dtype(x), rows, cols, block, codes.data_ptr(), scales_ptr, _stream()),
           "quantize_e4m3")
    return codes, (scales if block != 0 else None)


def quantize_mxfp4(x: torch.Tensor, block: int = 32, codes=None, scales=None):
    """x: 2-D fp32/bf16 -> (codes uint8 [rows, cols/2], E8M0 scales uint8 [rows, cols/block])."""
    _dev(x, "x")
    rows, cols = x.shape
    if block not in (16, 32) or cols % 32:
        raise ValueError("block must be 16 or 32 and cols a multiple of 32")
    codes = _out(codes, (rows, cols // 2), torch.uint8, x.device, "codes")
    scales = _out(scales, (rows, cols // block), torch.uint8, x.device, "scales")
    _check(lib.quantize_mxfp4(x.data_ptr(), _x_dtype(x), rows, cols, block, codes.data_ptr(), scales.data_ptr(),
                              _stream()), "quantize_mxfp4")
    return codes, scales


def quantize_nvfp4(x: torch.Tensor, tensor_scale: float = 1.0, codes=None, scales=None):
    """x: 2-D fp32/bf16 -> (codes uint8 [rows, cols/2], E4M3 scales uint8 [rows, cols/16]).
    Dequantized value: tensor_scale * e4m3(scale) * e2m1(code)."""
    _dev(x, "x")
    rows, cols = x.shape
    if cols % 16:
        raise ValueError("cols must be a multiple of 16")
    codes = _out(codes, (rows, cols // 2), torch.uint8, x.device, "codes")
    scales = _out(scales, (rows, cols // 16), torch.uint8, x.device, "scales")
    _check(lib.quantize_nvfp4(x.data_ptr(), _x_dtype(x), rows, cols, float(tensor_scale), codes.data_ptr(),
                              scales.data_ptr(), _stream()), "quantize_nvfp4")
    return codes, scales


def quantize_mx(x: torch.Tensor, block: int = 32, elem: str = "e4m3", rule: str = "round", codes=None,
                scales=None):
    """x: 2-D fp32/bf16 -> (codes uint8, E8M0 scales uint8 [rows, cols/block]).
    elem "e2m1": codes [rows, cols/2], two per byte; "e4m3": codes [rows, cols].
    rule: one of MX_RULES."""
    _dev(x, "x")
    rows, cols = x.shape
    if elem not in MX_ELEMS or rule not in MX_RULES:
        raise ValueError(f"elem must be one of {sorted(MX_ELEMS)} and rule one of {sorted(MX_RULES)}")
    if block not in (16, 32) or cols % 32:
        raise ValueError("block must be 16 or 32 and cols a multiple of 32")
    width = cols // 2 if elem == "e2m1" else cols
    codes = _out(codes, (rows, width), torch.uint8, x.device, "codes")
    scales = _out(scales, (rows, cols // block), torch.uint8, x.device, "scales")
    _check(lib.quantize_mx(x.data_ptr(), _x_dtype(x), rows, cols, block, MX_ELEMS[elem], MX_RULES[rule],
                           codes.data_ptr(), scales.data_ptr(), _stream()), "quantize_mx")
    return codes, scales


def quantize_int4(w: torch.Tensor, group: int = 128, packed=None, scales=None):
    """w: 2-D fp32/bf16 [N, K] -> (packed int32 [N, K/8] holding INT4X8 words,
    bf16 scales [N, K/group])."""
    _dev(w, "w")
    rows, cols = w.shape
    if group not in (32, 64, 128) or cols % group:
        raise ValueError("group must be 32, 64 or 128 and divide cols")
    packed = _out(packed, (rows, cols // 8), torch.int32, w.device, "packed")
    scales = _out(scales, (rows, cols // group), torch.bfloat16, w.device, "scales")
    _check(lib.quantize_int4(w.data_ptr(), _x_dtype(w), rows, cols, group, packed.data_ptr(), scales.data_ptr(),
                             _stream()), "quantize_int4")
    return packed, scales


def quantize_int4_asym(w: torch.Tensor, group: int = 128, packed=None, scalezero=None):
    """w: 2-D fp32/bf16 [N, K] -> (packed int32 [N, K/8] holding UINT4X8 words,
    scale-zero words int32 [N, K/group]: bf16 scale bits | zero-point << 16)."""
    _dev(w, "w")
    rows, cols = w.shape
    if group not in (32, 64, 128) or cols % group:
        raise ValueError("group must be 32, 64 or 128 and divide cols")
    packed = _out(packed, (rows, cols // 8), torch.int32, w.device, "packed")
    scalezero = _out(scalezero, (rows, cols // group), torch.int32, w.device, "scalezero")
    _check(lib.quantize_int4_asym(w.data_ptr(), _x_dtype(w), rows, cols, group, packed.data_ptr(),
                                  scalezero.data_ptr(), _stream()), "quantize_int4_asym")
    return packed, scalezero


_W_ELEM_BYTES2 = {WQ_INT4X8: 1, WQ_UINT4X8: 1, WQ_E2M1X2: 1, WQ_E4M3: 2}   # bytes per 2 elements


def _check_weight(wq, w_dtype, N, K):
    _dev(wq, "wq")
    if w_dtype not in _W_ELEM_BYTES2:
        raise ValueError("unsupported weight dtype")
    need = N * K * _W_ELEM_BYTES2[w_dtype] // 2
    if wq.numel() * wq.element_size() != need:
        raise ValueError(f"wq holds {wq.numel() * wq.element_size()} bytes, expected {need} for N={N}, K={K}")


def _check_scales(sc, s_dtype, N, K, group):
    if sc is None:
        return None
    _dev(sc, "w_scales")
    per = {WQ_BF16: 2, WQ_E8M0: 1, WQ_E4M3: 1, WQ_F32: 4, WQ_BF16Z: 4}[s_dtype]
    count = N if s_dtype == WQ_F32 else N * (K // group)
    if sc.numel() * sc.element_size() != count * per:
        raise ValueError("w_scales has the wrong size")
    return sc.data_ptr()


def wq_dequant(wq: torch.Tensor, w_dtype: int, w_scales, s_dtype: int, group: int, N: int, K: int, out=None):
    """Packed weights + scales -> bf16 [N, K] (the matmul's operand)."""
    _check_weight(wq, w_dtype, N, K)
    sp = _check_scales(w_scales, s_dtype, N, K, group) if w_scales is not None else None
    out = _out(out, (N, K), torch.bfloat16, wq.device, "out")
    _check(lib.wq_dequant(wq.data_ptr(), w_dtype, sp, s_dtype, group, N, K, out.data_ptr(), _stream()), "wq_dequant")
    return out


def wq_gemm_workspace_size(M: int, N: int, K: int, w_dtype: int, group: int) -> int:
    return int(lib.wq_gemm_workspace_size(M, N, K, w_dtype, group))


def wq_gemm(x: torch.Tensor, wq: torch.Tensor, w_dtype: int, w_scales: torch.Tensor, s_dtype: int, group: int,
            N: int, y=None, workspace=None, alpha: float = 1.0):
    """y[M, N] = alpha * x[M, K] . dequant(wq)^T in bf16 with fp32 accumulation."""
    _dev(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    M, K = x.shape
    _check_weight(wq, w_dtype, N, K)
    sp = _check_scales(w_scales, s_dtype, N, K, group)
    y = _out(y, (M, N), torch.bfloat16, x.device, "y")
    ws_ptr, ws_bytes = (None, 0)
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib.wq_gemm(x.data_ptr(), M, N, K, wq.data_ptr(), w_dtype, sp, s_dtype, group, float(alpha), y.data_ptr(),
                       ws_ptr, ws_bytes, _stream()), "wq_gemm")
    return y


# ---------------------------------------------------------------------------
# W8A8 FP8
# ---------------------------------------------------------------------------
def quantize_e4m3_static(x: torch.Tensor, scale: torch.Tensor, codes=None):
    """x: 2-D fp32/bf16; scale: a one-element fp32 device tensor.  Returns E4M3
    codes uint8 [rows, cols] = e4m3(x / scale)."""
    _dev(x, "x")
    _typed(scale, torch.float32, (1,), "scale")
    rows, cols = x.shape
    codes = _out(codes, (rows, cols), torch.uint8, x.device, "codes")
    _check(lib.quantize_e4m3_static(x.data_ptr(), _x_dtype(x), rows, cols, scale.data_ptr(), codes.data_ptr(),
                                    _stream()), "quantize_e4m3_static")
    return codes


def quantize_e4m3_block2d(w: torch.Tensor, codes=None, scales=None):
    """w: 2-D fp32/bf16 [N, K] -> (E4M3 codes uint8 [N, K], fp32 scales
    [ceil(N/128), K/128], one per 128 x 128 block)."""
    _dev(w, "w")
    rows, cols = w.shape
    codes = _out(codes, (rows, cols), torch.uint8, w.device, "codes")
    scales = _out(scales, ((rows + 127) // 128, cols // 128), torch.float32, w.device, "scales")
    _check(lib.quantize_e4m3_block2d(w.data_ptr(), _x_dtype(w), rows, cols, codes.data_ptr(), scales.data_ptr(),
                                     _stream()), "quantize_e4m3_block2d")
    return codes, scales


def wq_gemm_w8a8(a: torch.Tensor, a_scale: torch.Tensor, as_m: int, as_k: int, b: torch.Tensor, b_scale: torch.Tensor,
                 bs_n: int, bs_k: int, group_n: int, y=None):
    """y[M, N] (bf16) = sum over 128-wide K blocks kb of a_scale[m*as_m + kb*as_k] *
    b_scale[(n//group_n)*bs_n + kb*bs_k] * (a[m, kb] . b[n, kb]); a [M, K] and b [N, K]
    uint8 E4M3 codes, scales fp32 device tensors holding every index the strides reach."""
    for t, name in ((a, "a"), (b, "b"), (a_scale, "a_scale"), (b_scale, "b_scale")):
        _dev(t, name)
    if a.dtype != torch.uint8 or b.dtype != torch.uint8 or a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("a and b must be 2-D uint8 E4M3 codes with the same K")
    if a_scale.dtype != torch.float32 or b_scale.dtype != torch.float32:
        raise ValueError("scales must be float32")
    M, K = a.shape
    N = b.shape[0]
    kb = K // 128 if K % 128 == 0 else 0
    need_a = (M - 1) * as_m + (kb - 1) * as_k + 1 if kb else 0
    need_b = ((N - 1) // max(group_n, 1)) * bs_n + (kb - 1) * bs_k + 1 if kb else 0
    if kb and (a_scale.numel() < need_a or b_scale.numel() < need_b):
        raise ValueError("a scale array is smaller than its strides reach")
    y = _out(y, (M, N), torch.bfloat16, a.device, "y")
    _check(lib.wq_gemm_w8a8(a.data_ptr(), a_scale.data_ptr(), as_m, as_k, b.data_ptr(), b_scale.data_ptr(), bs_n, bs_k,
                            group_n, M, N, K, y.data_ptr(), _stream()), "wq_gemm_w8a8")
    return y


# ---------------------------------------------------------------------------
# W4A8 mixture of experts
# ---------------------------------------------------------------------------
def _typed(t, dtype, shape, name):
    _dev(t, name)
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}")


def wq_moe_route(logits: torch.Tensor, k: int):
    """logits fp32 [T, E] -> (ids int32 [T, k], weights fp32 [T, k], offsets int32 [E + 1],
    row_token int32 [T*k], row_slot int32 [T*k])."""
    _dev(logits, "logits")
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be a 2-D float32 tensor")
    T, E = logits.shape
    d = logits.device
    ids = torch.empty((T, k), dtype=torch.int32, device=d)
    weights = torch.empty((T, k), dtype=torch.float32, device=d)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=d)
    row_token = torch.empty(T * k, dtype=torch.int32, device=d)
    row_slot = torch.empty(T * k, dtype=torch.int32, device=d)
    _check(lib.wq_moe_route(logits.data_ptr(), T, E, k, ids.data_ptr(), weights.data_ptr(), offsets.data_ptr(),
                            row_token.data_ptr(), row_slot.data_ptr(), _stream()), "wq_moe_route")
    return ids, weights, offsets, row_token, row_slot


def wq_w4a8_prepack(wq: torch.Tensor, scales: torch.Tensor, wq_out=None):
    """wq int32 [E, N, K/8] INT4X8 words, scales bf16 [E, N, K/128] ->
    (re-laid words int32 [E, N, K/8], s8 uint8 [E, N, K/128], ch fp32 [E, N])."""
    _dev(wq, "wq")
    if wq.dtype != torch.int32 or wq.dim() != 3:
        raise ValueError("wq must be int32 [experts, N, K/8]")
    E, N, K8 = wq.shape
    K = 8 * K8
    _typed(scales, torch.bfloat16, (E, N, K // 128), "scales")
    wq_out = _out(wq_out, (E, N, K8), torch.int32, wq.device, "wq_out")
    s8 = torch.empty((E, N, K // 128), dtype=torch.uint8, device=wq.device)
    ch = torch.empty((E, N), dtype=torch.float32, device=wq.device)
    _check(lib.wq_w4a8_prepack(wq.data_ptr(), scales.data_ptr(), E, N, K, wq_out.data_ptr(), s8.data_ptr(),
                               ch.data_ptr(), _stream()), "wq_w4a8_prepack")
    return wq_out, s8, ch


def wq_w4a8_dequant(wq: torch.Tensor, s8: torch.Tensor):
    """Re-laid words int32 [N, K/8] + s8 [N, K/128] -> E4M3 codes uint8 [N, K]."""
    _dev(wq, "wq")
    N, K8 = wq.shape
    K = 8 * K8
    _typed(s8, torch.uint8, (N, K // 128), "s8")
    codes = torch.empty((N, K), dtype=torch.uint8, device=wq.device)
    _check(lib.wq_w4a8_dequant(wq.data_ptr(), s8.data_ptr(), N, K, codes.data_ptr(), _stream()), "wq_w4a8_dequant")
    return codes


def wq_moe_gemm_w4a8(x8: torch.Tensor, a_scale: torch.Tensor, row_token, offsets: torch.Tensor,
                     wq: torch.Tensor, s8: torch.Tensor, ch: torch.Tensor, y=None):
    """Grouped W4A8 GEMM.  x8 uint8 [T, K], a_scale fp32 [T], row_token int32 [R] or None
    (R = T), offsets int32 [E + 1], wq int32 [E, N, K/8] (re-laid), s8 uint8 [E, N, K/128],
    ch fp32 [E, N] -> y bf16 [R, N] in grouped row order."""
    _dev(x8, "x8")
    if x8.dtype != torch.uint8 or x8.dim() != 2:
        raise ValueError("x8 must be uint8 [T, K]")
    T, K = x8.shape
    _typed(a_scale, torch.float32, (T,), "a_scale")
    E, N, K8 = wq.shape
    if 8 * K8 != K:
        raise ValueError("wq and x8 disagree on K")
    _typed(wq, torch.int32, (E, N, K8), "wq")
    _typed(s8, torch.uint8, (E, N, K // 128), "s8")
    _typed(ch, torch.float32, (E, N), "ch")
    _typed(offsets, torch.int32, (E + 1,), "offsets")
    if row_token is None:
        R, rt = T, None
    else:
        _dev(row_token, "row_token")
        if row_token.dtype != torch.int32 or row_token.dim() != 1:
            raise ValueError("row_token must be int32 [R]")
        R, rt = row_token.shape[0], row_token.data_ptr()
    y = _out(y, (R, N), torch.bfloat16, x8.device, "y")
    _check(lib.wq_moe_gemm_w4a8(x8.data_ptr(), T, a_scale.data_ptr(), rt, R, offsets.data_ptr(), E, N, K,
                                wq.data_ptr(), s8.data_ptr(), ch.data_ptr(), y.data_ptr(), _stream()),
           "wq_moe_gemm_w4a8")
    return y


# ---------------------------------------------------------------------------
# measurement utilities (include/wq_util.h)
# ---------------------------------------------------------------------------
_SINK = {}
_MAGIC = 0x9E3779B9


def _sink(device) -> torch.Tensor:
    key = str(device)
    if key not in _SINK:
        _SINK[key] = torch.zeros(4, dtype=torch.int32, device=device)
    return _SINK[key]


def wq_util_stream_read(buf: torch.Tensor, nbytes: int = None) -> None:
    """Read the first `nbytes` bytes of `buf` (all of it by default) once from
    device memory and discard them."""
    _dev(buf, "buf")
    total = buf.numel() * buf.element_size()
    nbytes = total if nbytes is None else int(nbytes)
    if nbytes > total:
        raise ValueError("nbytes exceeds the buffer")
    _check(lib.wq_util_stream_read(buf.data_ptr(), nbytes, _MAGIC, _sink(buf.device).data_ptr(), _stream()),
           "wq_util_stream_read")


def wq_util_spin(iters: int, device=None) -> None:
    """Enqueue a bounded busy kernel of `iters` iterations (one workgroup per CU)."""
    dev = torch.device("cuda") if device is None else torch.device(device)
    _check(lib.wq_util_spin(int(iters), _MAGIC, _sink(dev).data_ptr(), _stream()), "wq_util_spin")


def wq_util_clock(out: torch.Tensor, ticks: int = 200) -> None:
    """Enqueue the one-wave clock probe; writes cycles and wall-clock ticks
    elapsed over about `ticks` wall-clock ticks into the two int64 of `out`."""
    _dev(out, "out")
    if out.dtype != torch.int64 or out.numel() < 2 or not out.is_contiguous():
        raise ValueError("out must be a contiguous int64 device tensor of at least 2 elements")
    _check(lib.wq_util_clock(int(ticks), out.data_ptr(), _stream()), "wq_util_clock")


def wq_util_wall_clock_khz() -> int:
    """Rate of the current device's wall clock in kHz."""
    khz = ctypes.c_int(0)
    _check(lib.wq_util_wall_clock_khz(ctypes.byref(khz)), "wq_util_wall_clock_khz")
    return khz.value
