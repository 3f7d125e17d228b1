"""Seeded synthetic inputs shaped like the 5120-hidden layers of the NVFP4
pretraining news page (zubnet.ai, "nvidia-nvfp4-paper-4-bit-pretrain-hits-fp8-parity",
paragraph 1: a 5120-hidden hybrid model).

This module holds no quantisation arithmetic: it draws random numbers with
numpy's PCG64 and rounds them to bf16 (nearest, ties to even).  Both the HIP
path and the CPU oracle consume the same bytes from here.
"""
from __future__ import annotations

import numpy as np

HIDDEN = 5120
FFN = 20480


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(rows: int, cols: int, seed: int, std: float = 1.0) -> np.ndarray:
    g = _rng(seed)
    return f32_to_bf16_bits(g.standard_normal((rows, cols), dtype=np.float32) * np.float32(std))


def laplace(rows: int, cols: int, seed: int, scale: float = 1e-3) -> np.ndarray:
    g = _rng(seed)
    return f32_to_bf16_bits(g.laplace(0.0, scale, size=(rows, cols)).astype(np.float32))


def outlier_tensor(rows: int = 256, cols: int = 256, seed: int = 101, n_outliers: int = 4,
                   magnitude: float = 50.0) -> np.ndarray:
    """N(0,1) with n distinct positions set to +m, -m, +m, -m, ... (small-tensor case)."""
    g = _rng(seed)
    x = g.standard_normal((rows, cols), dtype=np.float32)
    pos = g.choice(rows * cols, size=n_outliers, replace=False)
    for i, p in enumerate(pos):
        x.flat[p] = magnitude if i % 2 == 0 else -magnitude
    return f32_to_bf16_bits(x)


def activation(rows: int = 8192, cols: int = HIDDEN, seed: int = 202, outlier_frac: float = 1e-3,
               outlier_gain: float = 100.0) -> np.ndarray:
    """N(0,1) times a per-channel lognormal(0,1) scale, with exactly
    round(outlier_frac*rows*cols) entries (without replacement) multiplied by outlier_gain."""
    g = _rng(seed)
    x = g.standard_normal((rows, cols), dtype=np.float32)
    s = np.exp(g.standard_normal(cols)).astype(np.float32)
    x *= s[None, :]
    n_out = int(round(outlier_frac * rows * cols))
    pos = g.choice(rows * cols, size=n_out, replace=False)
    x.flat[pos] *= np.float32(outlier_gain)
    return f32_to_bf16_bits(x)


def token_outlier_gradient(rows: int, cols: int, seed: int, scale: float = 1e-3, gain: float = 30.0,
                           per_group: int = 1) -> np.ndarray:
    """Laplace(0, scale) gradient [tokens][channels] in which, in every aligned
    group of 16 tokens, `per_group` token rows (drawn without replacement
    within the group) are multiplied by `gain`: outliers that sit in a few
    tokens of each 16-token group, across all channels."""
    g = _rng(seed)
    x = g.laplace(0.0, scale, size=(rows, cols)).astype(np.float32)
    for g0 in range(0, rows - rows % 16, 16):
        x[g.choice(16, size=per_group, replace=False) + g0] *= np.float32(gain)
    return f32_to_bf16_bits(x)


def sparse_outlier_gradient(rows: int, cols: int, seed: int, scale: float = 1e-3, gain: float = 3e4,
                            count: int = 64) -> np.ndarray:
    """Laplace(0, scale) gradient with `count` entries, in distinct channels at
    random tokens, multiplied by `gain`: rare outliers far above the bulk."""
    g = _rng(seed)
    x = g.laplace(0.0, scale, size=(rows, cols)).astype(np.float32)
    ch = g.choice(cols, size=count, replace=False)
    tk = g.integers(0, rows, size=count)
    x[tk, ch] *= np.float32(gain)
    return f32_to_bf16_bits(x)


# The five workloads (shapes and distributions), keyed by name.
WORKLOADS = {
    "tiny_256": dict(desc="bf16 256x256, N(0,1) + 4 outliers at +/-50; row 1D, RTN, then dequantize"),
    "act_8192x5120": dict(desc="activation 8192x5120 bf16, N(0,1)*lognormal per channel, 0.1% x100; "
                               "row 1D + column 1D from one read, RTN"),
    "weight_5120x20480": dict(desc="FFN weight 5120x20480 bf16 N(0,0.02); 2D 16x16 RTN (+ transposed copy)"),
    "wgrad_8192x5120": dict(desc="dY Laplace(0,1e-3) and X N(0,1), 8192x5120 bf16; column 1D + RHT "
                                 "(dY SR seed 1234, X RTN); GEMM dW = dY^T X, 5120x5120, K=8192, fp32"),
    "linear_step_16384": dict(desc="linear layer step: hidden 5120, FFN 20480, 16384 tokens; "
                                   "Fprop/Dgrad/Wgrad for up and down projections"),
}


def tiny_256():
    return outlier_tensor(256, 256, 101)


def act_8192x5120(rows: int = 8192, cols: int = HIDDEN):
    return activation(rows, cols, 202)


def weight_5120x20480(rows: int = HIDDEN, cols: int = FFN):
    return normal(rows, cols, 303, std=0.02)


def wgrad_8192x5120(tokens: int = 8192, hidden: int = HIDDEN):
    return laplace(tokens, hidden, 404, 1e-3), normal(tokens, hidden, 405)


def linear_step_16384(tokens: int = 16384, hidden: int = HIDDEN, ffn: int = FFN):
    return dict(X=normal(tokens, hidden, 501), W1=normal(ffn, hidden, 502, std=0.02),
                W2=normal(hidden, ffn, 503, std=0.02), dY=laplace(tokens, hidden, 504, 1e-3))


def normal_device(rows: int, cols: int, seed: int, peak_at=None, peak: float = 64.0):
    """N(0,1) bf16 tensor drawn on the GPU by torch's seeded generator, for
    tensors too large to draw on the host (the maximum-size test); the value
    `peak` is planted at `peak_at` = (row, col) so that the tensor maximum is
    known.  Both sides read these bytes: the kernels on the device, the oracle
    from slices copied to the host."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((rows, cols), dtype=torch.bfloat16, device="cuda", generator=g)
    if peak_at is not None:
        x[peak_at[0], peak_at[1]] = peak
    return x
