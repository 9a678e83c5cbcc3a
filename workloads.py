"""Seeded synthetic inputs for the W2A8 BitLinear matmul.

This module holds no step of the method: it only draws random latent weights and
bf16 activations of the shapes and distributions the workloads use, so that the HIP
path and the CPU oracle receive the very same tensors.  It imports neither of them.

Recipe (one torch CPU generator per tensor, so weights can be reused across M):
  W = 0.02 * randn(N, K)                 generator seeded with `seed`
  X = randn(M, K)                        generator seeded with `seed + 1`
  with outliers: idx = randperm(K)[:round(0.01 K)] from the X generator, X[:, idx] *= 20
  X = X.to(bfloat16)

Shapes follow the BitNet b1.58 layer structure (q, k, v, o, gate, up, down projections,
no bias; "BitNet 深度实战" §3.2) at 2B-, 8B- and 70B-class widths.
"""
from __future__ import annotations

import numpy as np
import torch

# name -> (N, K) for one transformer layer's seven BitLinear projections.
LAYER_2B = [("q", 2560, 2560), ("k", 640, 2560), ("v", 640, 2560), ("o", 2560, 2560),
            ("gate", 6912, 2560), ("up", 6912, 2560), ("down", 2560, 6912)]
LAYER_8B = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
            ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]
LAYER_70B = [("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192), ("o", 8192, 8192),
             ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672)]


# Projections of one layer that read the same activations (the attention block's input
# feeds q, k and v; the MLP's input feeds gate and up), in the order a decode step runs
# them: each tuple is one launch.
DECODE_GROUPS = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]


def distinct_shapes(layer):
    seen, out = set(), []
    for name, n, k in layer:
        if (n, k) not in seen:
            seen.add((n, k))
            out.append((name, n, k))
    return out


# The five workloads: tiny, 2B decode (M=1), 2B prefill (M=512), 8B sweep, 70B chain.
WORKLOADS = {
    "tiny": dict(layer=[("w", 128, 256)], Ms=[4], outliers=False),
    "2b_decode": dict(layer=LAYER_2B, Ms=[1], outliers=True),
    "2b_prefill": dict(layer=LAYER_2B, Ms=[512], outliers=True),
    "8b_sweep": dict(layer=LAYER_8B, Ms=[1, 4, 16, 64, 256, 2048], outliers=True),
    "70b_chain": dict(layer=LAYER_70B, Ms=[1, 32, 1024], outliers=True),
}


def latent_weights(N: int, K: int, seed: int = 0) -> torch.Tensor:
    """fp32 latent weights ~ N(0, 0.02^2), shape (N, K), on the CPU."""
    g = torch.Generator().manual_seed(seed)
    return 0.02 * torch.randn(N, K, generator=g, dtype=torch.float32)


def latent_weights_on(device, N: int, K: int, seed: int = 0):
    """The same distribution as latent_weights, drawn on `device` by its own seeded
    generator (a different stream of numbers: for timing runs, where only the shape and
    the distribution matter and host-side draws of 10^8 values would dominate)."""
    g = torch.Generator(device=device).manual_seed(seed)
    return 0.02 * torch.randn(N, K, generator=g, dtype=torch.float32, device=device)


def activations(M: int, K: int, seed: int = 0, outliers: bool = True) -> torch.Tensor:
    """bf16 activations ~ N(0, 1), with 1% of channels scaled by 20, shape (M, K), CPU."""
    g = torch.Generator().manual_seed(seed + 1)
    X = torch.randn(M, K, generator=g, dtype=torch.float32)
    if outliers:
        n_out = int(round(0.01 * K))
        if n_out > 0:
            idx = torch.randperm(K, generator=g)[:n_out]
            X[:, idx] *= 20.0
    return X.to(torch.bfloat16)


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 array of its bit patterns (a view, no arithmetic)."""
    assert x.dtype == torch.bfloat16
    return x.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
