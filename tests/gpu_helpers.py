"""Shared helpers for the GPU parity tests: host <-> device transfers of the
synthetic inputs, and a per-case banner printed before each GPU step."""
import sys

import numpy as np
import torch

from oracle import gemm as OG
from oracle.formats import bf16_decode


def banner(*parts):
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_words(a: np.ndarray) -> torch.Tensor:
    """uint32 words -> int32 device tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).cuda()


def host_bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint8)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().astype(np.float32)


def host_words(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def check_all_rows(y_dev, xbits, wdeq, chan=None, block=1024):
    """Every output of y = x . w^T against the oracle's fp64 reference, the
    reference computed in blocks of `block` rows (bounded host memory).
    Returns the worst error / bound over all outputs."""
    y_all = bf16_decode(host_bits16(y_dev))
    worst = 0.0
    for r0 in range(0, xbits.shape[0], block):
        rows = slice(r0, min(r0 + block, xbits.shape[0]))
        ref, asum = OG.reference(xbits[rows], wdeq, chan)
        y = y_all[rows]
        assert np.isfinite(y).all()
        worst = max(worst, OG.worst_ratio(y, ref, asum))
        assert worst <= 1.0, f"rows {r0}+: worst error / bound = {worst:.3f}"
    return worst
