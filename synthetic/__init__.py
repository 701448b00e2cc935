"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and rounds them to the storage dtype of
the input (fp32 or bf16).  It holds none of the quantization or matmul
arithmetic: the oracle and the HIP path both receive exactly the bytes made
here.  Every generator takes an explicit seed and uses NumPy's PCG64
(``numpy.random.default_rng``).

bf16 inputs are produced by rounding fp32 draws to bf16 with PyTorch's CPU
cast (round to nearest, ties to even); they are returned as uint16 bit
patterns so that nothing downstream can silently re-round them.

Workload recipes (shapes and distributions of the pages' workloads):

* MXFP4 GEMV: x 1x512 ~N(0,1) bf16; W 1024x512 ~N(0, 0.02) fp32, with 1 % of
  the input columns (5 of 512, chosen without replacement) multiplied by 50.
* Decode: x Mx4096 ~N(0,1) bf16 with 0.5 % of the channels (20 of 4096, the
  same in every row) multiplied by 30; W 14336x4096 ~N(0, 0.02) fp32.
* Prefill: x 8192x4096 ~N(0,1) bf16; W 14336x4096 ~N(0, 0.02) fp32 with 1 % of
  the rows (143 of 14336) replaced by 0.02 * Student-t(4).
* Activation block quantization: 4096x7168 ~N(0,1) bf16 with 0.1 % of the
  entries (29,360, without replacement) multiplied by 100.
* W4A8 MoE: router logits 4096x64 ~N(0,1) fp32; tokens 4096x4096 ~N(0,1)
  bf16; per expert W_gate_up 3072x4096 and W_down 4096x1536 ~N(0, 0.02)
  fp32; the down-projection input is an independent 32768x1536 ~N(0,1) bf16.
"""
from __future__ import annotations

import numpy as np
import torch


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), rounded by torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def all_bf16_patterns() -> np.ndarray:
    """Every one of the 65,536 bf16 bit patterns, in order."""
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def normal_f32(shape, std: float, seed: int) -> np.ndarray:
    return (rng(seed).standard_normal(shape, dtype=np.float64) * std).astype(np.float32)


def mxfp4_gemv_inputs(seed: int = 0, K: int = 512, N: int = 1024):
    """x (1xK bf16 bits), W (NxK fp32) with 1 % of the K columns scaled x50."""
    g = rng(seed)
    x = to_bf16_bits(g.standard_normal((1, K)).astype(np.float32))
    W = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    cols = g.choice(K, size=max(1, round(0.01 * K)), replace=False)
    W[:, cols] *= np.float32(50.0)
    return x, W


def decode_inputs(M: int, seed: int = 0, K: int = 4096, N: int = 14336, with_weight: bool = True):
    """x (MxK bf16 bits) with 0.5 % of channels x30, and W (NxK fp32)."""
    g = rng(seed)
    W = (g.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)) if with_weight else None
    xf = g.standard_normal((M, K), dtype=np.float32)
    ch = g.choice(K, size=max(1, round(0.005 * K)), replace=False)
    xf[:, ch] *= np.float32(30.0)
    return to_bf16_bits(xf), W


def prefill_inputs(seed: int = 0, M: int = 8192, K: int = 4096, N: int = 14336, with_x: bool = True):
    """x (MxK bf16 bits), W (NxK fp32) with 1 % of rows heavy-tailed Student-t(4)."""
    g = rng(seed)
    W = g.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    rows = g.choice(N, size=max(1, round(0.01 * N)), replace=False)
    W[rows] = (g.standard_t(4.0, size=(len(rows), K)) * 0.02).astype(np.float32)
    x = to_bf16_bits(g.standard_normal((M, K), dtype=np.float32)) if with_x else None
    return x, W


def act_quant_inputs(seed: int = 0, rows: int = 4096, cols: int = 7168):
    """bf16 bits rows x cols ~N(0,1) with 0.1 % of entries x100."""
    g = rng(seed)
    a = g.standard_normal((rows, cols), dtype=np.float32)
    n_out = round(0.001 * rows * cols)
    idx = g.choice(rows * cols, size=n_out, replace=False)
    a.reshape(-1)[idx] *= np.float32(100.0)
    return to_bf16_bits(a)


def moe_router_logits(seed: int = 0, tokens: int = 4096, experts: int = 64) -> np.ndarray:
    return rng(seed).standard_normal((tokens, experts), dtype=np.float32)


def moe_tokens(seed: int = 1, tokens: int = 4096, hidden: int = 4096) -> np.ndarray:
    return to_bf16_bits(rng(seed).standard_normal((tokens, hidden), dtype=np.float32))


def moe_expert_weight(expert: int, which: str, seed: int = 2, hidden: int = 4096, inter: int = 1536) -> np.ndarray:
    """Per-expert fp32 weight, N x K row-major: 'gate_up' is (2*inter) x hidden,
    'down' is hidden x inter.  Each (expert, which) pair has its own stream."""
    sub = 0 if which == "gate_up" else 1
    g = np.random.default_rng([seed, expert, sub])
    shape = (2 * inter, hidden) if which == "gate_up" else (hidden, inter)
    return g.standard_normal(shape, dtype=np.float32) * np.float32(0.02)


def moe_down_input(seed: int = 3, rows: int = 32768, inter: int = 1536) -> np.ndarray:
    return to_bf16_bits(rng(seed).standard_normal((rows, inter), dtype=np.float32))


def moe_expert_weight_gpu(expert: int, which: str, seed: int = 2, hidden: int = 4096, inter: int = 1536,
                          device: str = "cuda"):
    """Device-side stand-in for moe_expert_weight (torch's Philox generator, one
    stream per (seed, expert, which)); same shapes and N(0, 0.02) distribution.
    Used where host generation of all experts would take minutes."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(expert) * 2 + (0 if which == "gate_up" else 1))
    shape = (2 * inter, hidden) if which == "gate_up" else (hidden, inter)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * 0.02


def moe_down_input_gpu(seed: int = 3, rows: int = 32768, inter: int = 1536, device: str = "cuda"):
    """Device-side stand-in for moe_down_input: bf16 N(0, 1) rows in grouped order."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + 7)
    return torch.randn((rows, inter), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
