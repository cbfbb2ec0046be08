"""Seeded synthetic inputs for the block-quantized linear layer.

This module only draws random numbers and rounds them to bf16 bit patterns;
it holds none of the quantization or matmul arithmetic.  Both the tests and
the benchmark take their inputs from here, and the same bytes go to the CPU
oracle and to the HIP library.

Distributions (the workloads of the decode/prefill projections this library
targets): weights N(0, 0.02), activations N(0, 1), optionally 1 % outlier
weights replaced by +-10 sigma before the bf16 rounding.

Two generators:
  * host: numpy ``Generator(PCG64(seed))``, float32 normals scaled by a
    float32 sigma, rounded to bf16 with round-to-nearest-even;
  * device: ``torch.Generator`` on the GPU (Philox), the same recipe, for
    tensors too large to draw on the host in a test's time budget (the
    32-layer decoder).  Rows of such a tensor are copied back to the host for
    the oracle, so both sides still see identical bytes.
"""
from __future__ import annotations

import numpy as np

W_SIGMA = 0.02
X_SIGMA = 1.0
OUTLIER_RATE = 0.01
OUTLIER_SIGMAS = 10.0


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (no NaN inputs)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed: int, shape, sigma: float) -> np.ndarray:
    """bf16 bit patterns of N(0, sigma^2) draws, host PCG64 generator."""
    g = np.random.Generator(np.random.PCG64(seed))
    n = int(np.prod(shape))
    v = g.standard_normal(n, dtype=np.float32) * np.float32(sigma)
    return bf16_bits_from_f32(v).reshape(shape)


def weights_bf16(seed: int, rows: int, cols: int, outliers: bool = False) -> np.ndarray:
    """Weights [rows][cols] ~ N(0, 0.02); with ``outliers`` a Bernoulli(0.01)
    mask (seed+2) replaces entries by +-0.2 with a fair sign (seed+3)."""
    g = np.random.Generator(np.random.PCG64(seed))
    v = g.standard_normal(rows * cols, dtype=np.float32) * np.float32(W_SIGMA)
    if outliers:
        mask = np.random.Generator(np.random.PCG64(seed + 2)).random(rows * cols) < OUTLIER_RATE
        pos = np.random.Generator(np.random.PCG64(seed + 3)).random(rows * cols) < 0.5
        big = np.float32(OUTLIER_SIGMAS * W_SIGMA)
        v = np.where(mask, np.where(pos, big, -big), v).astype(np.float32)
    return bf16_bits_from_f32(v).reshape(rows, cols)


def activations_bf16(seed: int, rows: int, cols: int) -> np.ndarray:
    """Activations [rows][cols] ~ N(0, 1)."""
    return normal_bf16(seed, (rows, cols), X_SIGMA)


def seed_for(config: int, tensor: int) -> int:
    """Seed of tensor ``tensor`` (0 = weights, 1 = activations) of workload
    number ``config`` (1..5)."""
    return 1000 * config + 10 * tensor


def decoder_seed(layer: int, kind: int) -> int:
    """Seed of projection ``kind`` (q,k,v,o,gate,up,down = 0..6) of decoder
    layer ``layer`` in the 32-layer workload."""
    return 5000 + 16 * layer + kind


LM_HEAD_W_SEED = 5999
LM_HEAD_X_SEED = 5998


def device_normal_bf16(seed: int, shape, sigma: float, device="cuda"):
    """bf16 tensor of N(0, sigma^2) draws made on the GPU (torch Philox),
    for tensors too large for the host generator.  Returns a torch tensor."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    chunk = 1 << 27
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        t = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        t.mul_(sigma)
        flat[s:e].copy_(t)
    return out
